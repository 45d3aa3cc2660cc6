"""Build libfz.so (HIP, gfx950) in-tree with hipcc.

Run as ``python -m smith_waterman_dp_amd.build``; ``__graft_entry__.build()``
calls ``build()``.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfz.so")
PROBE_LIB = os.path.join(HERE, "libfz_probe.so")
ARCH = os.environ.get("FZ_OFFLOAD_ARCH", "gfx950")

SOURCES = ["fz_lib.hip"]
PROBE_SOURCES = ["fz_probe.hip"]
HEADERS = ["fz_device.hpp", "fz_extend.hpp", "fz_aux.hpp", "fz_local.hpp", "fz_seeds.hpp", "fz_rounds.hpp",
           "fz_sort.hpp", "fz_packed.hpp"]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "--offload-arch=" + ARCH,
    # packed fp32 ops stay off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc():
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if p and (os.path.sep not in p or os.path.exists(p)):
            return p
    return "hipcc"


def _compile(srcs, lib, verbose, extra):
    tmp = lib + ".tmp"
    cmd = [hipcc()] + FLAGS + list(extra) + ["-I", os.path.join(HERE, "..", "include")] + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)


def build(verbose=False, extra=()):
    """libfz.so (the library) and libfz_probe.so (the VALU-rate probe the
    benchmark reports beside the peak from unit counts)."""
    _compile([os.path.join(CSRC, s) for s in SOURCES], LIB, verbose, extra)
    _compile([os.path.join(CSRC, s) for s in PROBE_SOURCES], PROBE_LIB, verbose, extra)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
    print(LIB)
