"""MI355X-native batched gapped seed extension (FastZ-style inspector /
executor on gfx950).  The compute runs in the HIP library ``libfz.so``
(built from ``csrc/``); ``fz`` is its thin ctypes binding."""
