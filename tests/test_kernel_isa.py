"""Structure of the compiled kernels (host-only: hipcc cross-compiles gfx950).

Every gemv_kernel<P, FUSED, C> and gemv_local_kernel<P> must issue all P of
a wavefront's weight loads (the non-temporal 16-byte loads) before its first
wait on vector memory, and
every gemm_mfma_kernel<MT, PS> all 4 * PS of its weight words (non-temporal
4-byte loads) and all PS * MT of its activation operands: the waits count
loads in issue order, so a load issued after the first wait is held back by
a full memory latency.  The compiler is
free to schedule otherwise, so this is checked on the assembly it produces.
"""
import os
import re
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "bit_gemv_bitlinear_amd", "csrc")


def _asm(tmp_path_factory, source):
    from bit_gemv_bitlinear_amd import build
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / source.replace(".hip", ".s")
    flags = [f for f in build.flags_for(source) if f != "-fPIC"]
    cmd = [build.HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, source),
           "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


@pytest.fixture(scope="module")
def gemv_asm(tmp_path_factory):
    return _asm(tmp_path_factory, "gemv.hip")


@pytest.fixture(scope="module")
def local_asm(tmp_path_factory):
    return _asm(tmp_path_factory, "gemv_local.hip")


@pytest.fixture(scope="module")
def norm_asm(tmp_path_factory):
    return _asm(tmp_path_factory, "gemv_norm.hip")


@pytest.fixture(scope="module")
def mfma_asm(tmp_path_factory):
    return _asm(tmp_path_factory, "gemm_mfma.hip")


@pytest.fixture(scope="module")
def prefill_asm(tmp_path_factory):
    return _asm(tmp_path_factory, "gemm_prefill.hip")


def test_weight_loads_issued_before_first_wait(gemv_asm):
    kernels = list(re.finditer(r"^(_ZN\S*gemv_kernelILi(\d+)ELb([01])ELi(\d)ELb([01])E\S*):", gemv_asm,
                               re.M))
    # P = 1..15: int8 input with C = 1, 2, 4 cached chunks, and also with one
    # wavefront per band finishing its own rows; bf16 input with C = 1, 2
    assert len(kernels) == 120
    late = []
    for m in kernels:
        P = int(m.group(2))
        body = gemv_asm[m.end():gemv_asm.index("s_endpgm", m.end())]
        first_wait = body.index("s_waitcnt vmcnt")
        issued = len(re.findall(r"global_load_dwordx4 [^\n]* nt\b", body[:first_wait]))
        if issued != P:
            late.append((P, m.group(3), issued))
    assert not late, f"(P, fused, weight loads before the first wait): {late}"


def test_gemv_arguments_preloaded(gemv_asm):
    # gemv.hip is built with its kernels' first 14 argument dwords preloaded
    # into SGPRs: after the compatibility prologue (which loads them the usual
    # way and jumps over 256 bytes), no kernel-argument load may come before
    # the weight loads have been issued
    kernels = list(re.finditer(r"^(_ZN\S*gemv_kernelILi(\d+)ELb([01])ELi(\d)ELb([01])E\S*):", gemv_asm,
                               re.M))
    assert len(kernels) == 120
    late = []
    for m in kernels:
        name = m.group(1)
        assert _meta(gemv_asm, name, "amdhsa_user_sgpr_kernarg_preload_length") == 14, name
        body = gemv_asm[m.end():gemv_asm.index("s_endpgm", m.end())]
        main = body[body.index("s_branch"):]
        first_wait = main.index("s_waitcnt vmcnt")
        if "s_load_" in main[:first_wait]:
            late.append(name)
    assert not late, f"kernel-argument loads ahead of the weight loads: {late}"


def test_local_weight_loads_issued_before_first_wait(local_asm):
    kernels = list(re.finditer(r"^(_ZN\S*gemv_local_kernelILi(\d+)E\S*):", local_asm, re.M))
    assert sorted(int(m.group(2)) for m in kernels) == list(range(1, 13))
    late = []
    for m in kernels:
        P = int(m.group(2))
        body = local_asm[m.end():local_asm.index("s_endpgm", m.end())]
        first_wait = body.index("s_waitcnt vmcnt")
        weights = len(re.findall(r"global_load_dwordx4 [^\n]* nt\b", body[:first_wait]))
        acts = len(re.findall(r"global_load_dwordx2 ", body[:first_wait]))
        if weights != P or acts != P:
            late.append((P, weights, acts))
    assert not late, f"(P, weight loads, activation loads before the first wait): {late}"


def test_mfma_operand_loads_issued_before_first_wait(mfma_asm):
    kernels = list(re.finditer(r"^(_ZN\S*gemm_mfma_kernelILi(\d+)ELi(\d+)E\S*):", mfma_asm, re.M))
    # MT = 1..4 m tiles, PS = 1..min(16, 20 / MT) steps
    assert sorted((int(m.group(2)), int(m.group(3))) for m in kernels) == \
        [(mt, ps) for mt in range(1, 5) for ps in range(1, min(16, 20 // mt) + 1)]
    late = []
    for m in kernels:
        MT, PS = int(m.group(2)), int(m.group(3))
        body = mfma_asm[m.end():mfma_asm.index("s_endpgm", m.end())]
        # from the first operand load of the main loop (the compiler may
        # rotate the loop, placing its waits above its loads in the text)
        first_load = re.search(r"global_load_dwordx4 |global_load_dword [^\n]* nt\b", body).start()
        first_wait = body.index("s_waitcnt vmcnt", first_load)
        chunk = body[first_load:first_wait]
        weights = len(re.findall(r"global_load_dword [^\n]* nt\b", chunk))
        acts = len(re.findall(r"global_load_dwordx4 ", chunk))
        if weights != 4 * PS or acts != PS * MT:
            late.append((MT, PS, weights, acts))
    assert not late, f"(MT, PS, weight words, A operands before the first wait): {late}"


def _meta(asm, name, key):
    k = asm.index(".amdhsa_kernel " + name)
    block = asm[k:asm.index(".end_amdhsa_kernel", k)]
    return int(re.search(r"\." + key + r"\s+(\d+)", block).group(1))


def test_no_scratch_and_declared_lds_only(gemv_asm, local_asm, mfma_asm):
    # No kernel spills to scratch, and each uses exactly the LDS it declares:
    # a private array that the compiler moves into LDS (it does so for arrays
    # indexed at run time) once made the MFMA kernel twice as slow.
    for m in re.finditer(r"^(_ZN\S*gemv_kernelILi(\d+)ELb([01])ELi(\d)ELb([01])E\S*):", gemv_asm,
                         re.M):
        name, fused, own = m.group(1), m.group(3) == "1", m.group(5) == "1"
        assert _meta(gemv_asm, name, "amdhsa_private_segment_fixed_size") == 0, name
        # part_sh[16][64] (not when each wavefront finishes its own rows) +
        # xsum_sh[16], + amax_sh[16] when fused (the activation row itself is
        # dynamic LDS)
        want = (0 if own else 16 * 64 * 4) + 16 * 4 + (16 * 4 if fused else 0)
        assert _meta(gemv_asm, name, "amdhsa_group_segment_fixed_size") == want, name
    for m in re.finditer(r"^(_ZN\S*gemv_local_kernelILi(\d+)E\S*):", local_asm, re.M):
        name = m.group(1)
        assert _meta(local_asm, name, "amdhsa_private_segment_fixed_size") == 0, name
        # part_sh[16][64] + amax_sh[16] (the quantised words are dynamic LDS)
        assert _meta(local_asm, name, "amdhsa_group_segment_fixed_size") == 16 * 64 * 4 + 16 * 4, name
    for m in re.finditer(r"^(_ZN\S*gemm_mfma_kernelILi(\d+)ELi(\d+)E\S*):", mfma_asm, re.M):
        name, MT = m.group(1), int(m.group(2))
        assert _meta(mfma_asm, name, "amdhsa_private_segment_fixed_size") == 0, name
        # red[16 MT][68] int32 + inv_s_sh[16 MT] fp64 + s_sh[16 MT] fp32
        # + the A staging slots, 8 wavefronts x MT x 1 KiB
        want = 16 * MT * (68 * 4 + 8 + 4) + 8 * MT * 1024
        assert _meta(mfma_asm, name, "amdhsa_group_segment_fixed_size") == want, name


def test_prefill_no_scratch_and_declared_lds(prefill_asm):
    # gemm_prefill_kernel<WN, WMW, MTW>: tile 64 WN weight rows x 16 MTW WMW
    # activation rows; two LDS buffers of the activation tile (pitch 272)
    # and the 4 WN weight tiles (1152 bytes each), nothing else.
    kernels = list(re.finditer(r"^(_ZN\S*gemm_prefill_kernelILi(\d+)ELi(\d+)ELi(\d+)E\S*):",
                               prefill_asm, re.M))
    assert sorted((int(m.group(2)), int(m.group(3)), int(m.group(4))) for m in kernels) == \
        [(1, 4, 1), (2, 4, 1), (4, 2, 2), (4, 2, 4)]
    for m in kernels:
        name = m.group(1)
        WN, WMW, MTW = int(m.group(2)), int(m.group(3)), int(m.group(4))
        BM, BN = 16 * MTW * WMW, 64 * WN
        assert _meta(prefill_asm, name, "amdhsa_private_segment_fixed_size") == 0, name
        want = 2 * (BM * 272 + BN // 16 * 1152)
        assert _meta(prefill_asm, name, "amdhsa_group_segment_fixed_size") == want, name
        body = prefill_asm[m.end():prefill_asm.index("s_endpgm", m.end())]
        # one K tile in the loop body: 4 steps x 4 bands x MTW m tiles
        assert body.count("v_mfma_i32_16x16x64_i8") == 16 * MTW, name


@pytest.mark.parametrize("kind,modes", [("gemv_norm_kernel", 3), ("gemv_norm_group_kernel", 2)])
def test_norm_kernels_issue_all_loads_first(norm_asm, kind, modes):
    # gemv_norm_kernel<P, C, MODE> (one projection; MODE 0 the row x, 1 its
    # GLU with x_up, 2 a handed-off row with its partial statistics) and
    # gemv_norm_group_kernel (several, one work record per workgroup; modes 0
    # and 1): the row's C chunks of x, gamma (and x_up), the four 16-byte
    # partial loads of mode 2, all buffer loads, and all P weight tiles are
    # issued before the first wait, without scratch.  Before the first of
    # those loads: no branch, and one round of argument reads (the work
    # record's address, then the record, for the grouped kernel) -- a branch
    # there had split the reads into rounds, each waiting for the last.
    kernels = list(re.finditer(r"^(_ZN\S*" + kind + r"ILi(\d+)ELi(\d)ELi([012])E\S*):", norm_asm, re.M))
    assert len(kernels) == 32 * modes    # P = 1..16, C = 1, 2, each mode
    assert {int(m.group(4)) for m in kernels} == set(range(modes))
    late = []
    for m in kernels:
        name, P, C, mode = m.group(1), int(m.group(2)), int(m.group(3)), int(m.group(4))
        body = norm_asm[m.end():norm_asm.index("s_endpgm", m.end())]
        first_wait = body.index("s_waitcnt vmcnt")
        weights = len(re.findall(r"global_load_dwordx4 [^\n]* nt\b", body[:first_wait]))
        # (the partials' unused fourth words make them dwordx3 loads)
        rows = len(re.findall(r"buffer_load_dwordx[34] ", body[:first_wait]))
        if weights != P or rows != C * (3 if mode == 1 else 2) + (4 if mode == 2 else 0):
            late.append((P, C, mode, weights, rows))
        pre = body[:min(body.index(k) for k in ("global_load", "buffer_load"))]
        rounds = pre.count("s_waitcnt lgkmcnt")
        if "s_cbranch" in pre or rounds != (2 if kind == "gemv_norm_group_kernel" else 1):
            late.append((P, C, mode, "argument rounds", rounds, "branches", pre.count("s_cbranch")))
        assert _meta(norm_asm, name, "amdhsa_private_segment_fixed_size") == 0, name
    assert not late, f"(P, C, mode, weight loads, row loads before the first wait): {late}"


@pytest.fixture(scope="module")
def lut_asm(tmp_path_factory):
    return _asm(tmp_path_factory, "gemv_lut.hip")


def test_lut_kernels_issue_all_loads_first(lut_asm):
    # gemv_lut_kernel<P>: all P weight tiles (after the activation chunk it
    # builds tables from) are issued before the first wait, without scratch
    kernels = list(re.finditer(r"^(_ZN\S*gemv_lut_kernelILi(\d+)E\S*):", lut_asm, re.M))
    # runs of <= 4 steps, or whole rows of <= 10 steps on wide matrices
    assert sorted(int(m.group(2)) for m in kernels) == list(range(1, 11))
    late = []
    for m in kernels:
        name, P = m.group(1), int(m.group(2))
        body = lut_asm[m.end():lut_asm.index("s_endpgm", m.end())]
        first_wait = body.index("s_waitcnt vmcnt")
        weights = len(re.findall(r"global_load_dwordx4 [^\n]* nt\b", body[:first_wait]))
        if weights != P:
            late.append((P, weights))
        assert _meta(lut_asm, name, "amdhsa_private_segment_fixed_size") == 0, name
    assert not late, f"(P, weight loads before the first wait): {late}"


@pytest.fixture(scope="module")
def band_asm(tmp_path_factory):
    return _asm(tmp_path_factory, "gemm_band.hip")


def test_band_kernels_issue_rows_then_weights(band_asm):
    # gemm_band_kernel<MT, P, BW>: every activation load (buffer loads: P
    # chunks per thread for one m tile, 4 ceil(P / 2) for two), then all BW P
    # weight tiles (non-temporal 16-byte loads), before the first wait on
    # vector memory -- the rows first, since a wait for them counts every
    # load issued before them; no scratch, and the static LDS is the rows'
    # scales and sums (fp64 + fp32 + int32 per row)
    kernels = list(re.finditer(r"^(_ZN\S*gemm_band_kernelILi(\d)ELi(\d+)ELi(\d)E\S*):", band_asm, re.M))
    assert sorted((int(m.group(2)), int(m.group(4)), int(m.group(3))) for m in kernels) == \
        [(mt, bw, p) for mt, bw in ((1, 1), (2, 1), (2, 2)) for p in range(1, 11)]
    late = []
    for m in kernels:
        name, MT, P, BW = m.group(1), int(m.group(2)), int(m.group(3)), int(m.group(4))
        body = band_asm[m.end():band_asm.index("s_endpgm", m.end())]
        first_wait = body.index("s_waitcnt vmcnt")
        head = body[:first_wait]
        rows = len(re.findall(r"buffer_load_dwordx4 ", head))
        weights = [w.start() for w in re.finditer(r"global_load_dwordx4 [^\n]* nt\b", head)]
        last_row = max(r.start() for r in re.finditer(r"buffer_load_dwordx4 ", head))
        want_rows = P if MT == 1 else 4 * ((P + 1) // 2)
        if rows != want_rows or len(weights) != BW * P or min(weights) < last_row:
            late.append((MT, P, BW, rows, len(weights)))
        assert _meta(band_asm, name, "amdhsa_private_segment_fixed_size") == 0, name
        assert _meta(band_asm, name, "amdhsa_group_segment_fixed_size") == 16 * MT * (8 + 4 + 4), name
    assert not late, f"(MT, P, BW, row loads, weight loads before the first wait, rows first): {late}"
