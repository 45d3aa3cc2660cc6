"""The wave-per-side kernels keep every loop under scalar (wave-uniform)
control.

The first extension kernel of this library was a persistent grid: each wave
took its next side from an atomic counter in lane 0 and broadcast it with
readfirstlane.  Its compiled code split the wave at the end of a side: lane 0
went on to store the result and bump the counter, while lanes 1..63 took the
loop's back edge straight to the readfirstlane of the side index, read lane
1's index (0) and re-ran side 0; the loop's exit mask on that path held lane
0 only, so those lanes never left it and the kernel never finished.  The
compiled form of such a split is a loop whose exit is taken per lane by
masking EXEC ("s_andn2_b64 exec, exec, ...").

The kernels now take their side from blockIdx (one wave per side), so no
loop carries a side index; this test compiles the device code and checks
that none of the inspector, executor or walker instantiations contains a
per-lane loop exit at all.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "smith_waterman_dp_amd", "csrc")

pytestmark = pytest.mark.slow

WAVE_KERNELS = re.compile(r"^_ZN2fz(13extend_kernel|16walk_wave_kernel)\w*:", re.M)


def hipcc():
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if p and os.path.exists(p):
            return p
    return shutil.which("hipcc")


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    cc = hipcc()
    if not cc:
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("isa") / "fz_lib.s")
    from smith_waterman_dp_amd import build as b
    cmd = [cc] + [f for f in b.FLAGS if f not in ("-shared", "-fPIC")] + [
        "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"),
        os.path.join(CSRC, "fz_lib.hip"), "-o", out]
    subprocess.check_call(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    return open(out).read()


def kernel_bodies(asm):
    """{symbol: text} of every wave-per-side kernel in the assembly."""
    out = {}
    for m in WAVE_KERNELS.finditer(asm):
        start = m.end()
        end = asm.find("s_endpgm", start)
        out[m.group(0)[:-1]] = asm[start:end]
    return out


def test_wave_kernels_have_no_per_lane_loop_exits(device_asm):
    bodies = kernel_bodies(device_asm)
    # inspector and executor at both window widths and three scoring modes,
    # walker at both widths
    assert len(bodies) >= 14, sorted(bodies)
    for name, text in bodies.items():
        assert not re.search(r"s_andn2_b64 exec, exec,", text), name
