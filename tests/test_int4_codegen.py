"""Host-side check of the compiled INT4 wide kernel's waits (no GPU needed).

int4_gemv_wide_kernel loads x straight into LDS and ends every step with a
hand-written `s_waitcnt vmcnt(N)` + `s_barrier`: N counts the weight and
scale loads issued after the step's LDS loads, so that the LDS loads are
complete before any wave reads the buffer.  That count is right only if the
compiler keeps those loads where the source puts them.  This test compiles
the kernel to gfx950 assembly and checks, for every barrier of every
instantiation, that at least N vector-memory loads follow the last LDS load
before it (so vmcnt(N) covers all LDS loads), and that a barrier waits for
every load before the LDS is reused for the final sums.
"""
import os
import re
import shutil
import subprocess

import pytest

from paged_attention_fp8_amd import build as B

SRC = os.path.join(B.CSRC, "int4_gemv.hip")


def _asm(tmp_path):
    hipcc = B.hipcc()
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    out = tmp_path / "int4_gemv.s"
    subprocess.run([hipcc, *B.common_flags(), "--cuda-device-only", "-S", "-o", str(out), SRC],
                   check=True, stderr=subprocess.DEVNULL)
    return out.read_text()


def _kernels(asm):
    """{symbol: body} of every int4_gemv_wide_kernel instantiation."""
    res = {}
    for m in re.finditer(r"^(_Z\S*int4_gemv_wide_kernel\S*?):", asm, re.M):
        end = asm.index("s_endpgm", m.end())
        res[m.group(1)] = asm[m.end():end]
    return res


def _check_barriers(body):
    """[(vmcnt, loads issued after the last LDS load, or None when no LDS
    load is outstanding)] for every barrier preceded by a vmcnt wait."""
    res = []
    lds_pending, after = False, 0
    lines = [ln.split(";")[0].strip() for ln in body.splitlines()]
    for i, ln in enumerate(lines):
        if ln.startswith(("buffer_load", "global_load")):
            if ln.split()[-1] == "lds":
                lds_pending, after = True, 0
            else:
                after += 1
        elif ln.startswith("s_barrier"):
            m = re.match(r"s_waitcnt vmcnt\((\d+)\)", lines[i - 1] if i else "")
            if m is None:
                continue                      # a barrier for LDS stores alone
            res.append((int(m.group(1)), after if lds_pending else None))
            lds_pending = False               # (asserted below: the wait covered them)
    return res


def test_wide_kernel_waits_cover_lds_loads(tmp_path):
    kernels = _kernels(_asm(tmp_path))
    assert kernels, "no int4_gemv_wide_kernel instantiation found"
    for name, body in kernels.items():
        checks = _check_barriers(body)
        assert len(checks) >= 3, (name, checks)      # prologue, a step, the end
        for n, after in checks:
            if after is None:
                continue                              # no LDS load since the last barrier
            assert n <= after, (name, "vmcnt(%d) with only %d loads after the LDS loads" % (n, after))
        assert any(n == 0 for n, _ in checks), (name, "no barrier waits for every load")
