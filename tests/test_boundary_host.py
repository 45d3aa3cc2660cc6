"""Host-only checks of the C-ABI boundary: the library loads, exports every
symbol include/fz.h declares, and rejects bad calls without touching a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

from smith_waterman_dp_amd import fz

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "fz.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fz_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(fz.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = fz.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_struct_sizes_match_header():
    # fz_seed is 7 int64, fz_hit is 12 int64 (the binding's tensor views rely on it)
    assert len(fz.SEED_FIELDS) == 7
    assert len(fz.HIT_FIELDS) == 12
    assert ctypes.sizeof(fz.fz_scoring) == 20
    assert ctypes.sizeof(fz.fz_matrix) == 17 * 4           # sub[4][4] and n_score
    assert ctypes.sizeof(fz.fz_seed_stats) == 11 * 4       # eleven float phase times
    # fz_stats: 22 uint64 counters (bin_hist holds 8), eight float times
    assert ctypes.sizeof(fz.fz_stats) == 22 * 8 + 8 * 4


def test_struct_sizes_match_c_compiler(tmp_path):
    # the binding's structs against the header as a C compiler lays it out
    src = tmp_path / "sizes.c"
    src.write_text('#include <stdio.h>\n#include "fz.h"\n'
                   'int main(void) { printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(fz_seed), sizeof(fz_hit), '
                   'sizeof(fz_scoring), sizeof(fz_matrix), sizeof(fz_stats), sizeof(fz_seed_stats)); return 0; }\n')
    exe = tmp_path / "sizes"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run(["gcc", "-std=c99", "-I", inc, str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    assert got == [7 * 8, 12 * 8, ctypes.sizeof(fz.fz_scoring), ctypes.sizeof(fz.fz_matrix),
                   ctypes.sizeof(fz.fz_stats), ctypes.sizeof(fz.fz_seed_stats)]


def test_null_context_is_rejected():
    lib = fz.load_library()
    sc = fz.fz_scoring(91, -31, -123, 400, 30)
    rc = lib.fz_extend_batch(None, None, 0, None, 0, None, 0, ctypes.byref(sc), None, 9400, 0, 0, None,
                             None, None, None, None)
    assert rc == fz.FZ_EINVAL
    assert lib.fz_set_pointer_workspace(None, 0) == fz.FZ_EINVAL
    assert lib.fz_copy_cigar(None, None, 0, None) == fz.FZ_EINVAL
    assert lib.fz_extend_rounds(None, None, 0, None, 0, None, 0, ctypes.byref(sc), None, 9400, 0,
                                fz.FZ_TRACEBACK, 16, None, None, None, None, None) == fz.FZ_EINVAL
    n = ctypes.c_uint64(7)
    assert lib.fz_find_seeds(None, None, 0, None, 0, 19, 0, 0, None, ctypes.byref(n), None, None, None) == fz.FZ_EINVAL
    assert lib.fz_copy_seeds(None, None, 0, None) == fz.FZ_EINVAL
    assert lib.fz_debug_set(None, fz.FZ_DEBUG_SHRINK_ROWS, 1) == fz.FZ_EINVAL
    assert lib.fz_extend_batch_noalloc(None, None, 0, None, 0, None, 0, ctypes.byref(sc), None, 9400, 0, None,
                                       None, None) == fz.FZ_EINVAL
    lib.fz_destroy(None)


def test_create_bad_device_fails_cleanly():
    lib = fz.load_library()
    h = ctypes.c_void_p()
    assert lib.fz_create(ctypes.byref(h), 10_000, 0) != fz.FZ_OK
    assert not h.value


def test_build_lists_every_source():
    from smith_waterman_dp_amd import build
    csrc = os.path.join(ROOT, "smith_waterman_dp_amd", "csrc")
    have = sorted(f for f in os.listdir(csrc) if f.endswith(".hpp"))
    assert sorted(build.HEADERS) == have
    assert sorted(build.SOURCES + build.PROBE_SOURCES) == sorted(f for f in os.listdir(csrc) if f.endswith(".hip"))
