"""Structure of the compiled GEMV kernels (host-only: hipcc cross-compiles gfx950).

Every gemv_kernel<P, FUSED> must issue all P of a wavefront's weight loads
(the non-temporal 16-byte loads) before its first wait on vector memory:
the waits count loads in issue order, so a weight load issued after the
first wait is held back by a full memory latency.  The compiler is free to
schedule otherwise, so this is checked on the assembly it produces.
"""
import os
import re
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "bit_gemv_bitlinear_amd", "csrc")


@pytest.fixture(scope="module")
def gemv_asm(tmp_path_factory):
    from bit_gemv_bitlinear_amd import build
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "gemv.s"
    flags = [f for f in build.FLAGS if f != "-fPIC"]
    cmd = [build.HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, "gemv.hip"),
           "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def test_weight_loads_issued_before_first_wait(gemv_asm):
    kernels = list(re.finditer(r"^(_ZN\S*gemv_kernelILi(\d+)ELb([01])E\S*):", gemv_asm, re.M))
    assert len(kernels) == 40   # P = 1..20, int8 and bf16 input
    late = []
    for m in kernels:
        P = int(m.group(2))
        body = gemv_asm[m.end():gemv_asm.index("s_endpgm", m.end())]
        first_wait = body.index("s_waitcnt vmcnt")
        issued = len(re.findall(r"global_load_dwordx4 [^\n]* nt\b", body[:first_wait]))
        if issued != P:
            late.append((P, m.group(3), issued))
    assert not late, f"(P, fused, weight loads before the first wait): {late}"
