"""The allocation-free entry point ternarize_weights_absmean_noalloc (its
histogram lives in a library-held device array) against the entry point that
takes a caller workspace, ternarize_weights_absmean: the packed bytes and the
three bf16 scales must be identical, call after call.  Two calls in a row,
the second on a smaller matrix with other values, so a histogram left over
from the first call would show; the smaller one is also checked against the
oracle.  Called through the C ABI."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import bf16_dev, host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bit_gemv_bitlinear_amd as m
    return m


def run_both(bl, w_bits):
    import torch
    N, K = w_bits.shape
    lib = bl.lib()
    st = torch.cuda.current_stream().cuda_stream
    w = bf16_dev(w_bits)
    outs = []
    for noalloc in (False, True):
        packed = torch.full((bl.bl_packed_bytes(N, K),), 0xA5, dtype=torch.uint8, device="cuda")
        scales = torch.full((3,), float("nan"), dtype=torch.bfloat16, device="cuda")
        if noalloc:
            rc = lib.ternarize_weights_absmean_noalloc(w.data_ptr(), packed.data_ptr(),
                                                       scales.data_ptr(), N, K, st)
        else:
            work = torch.full((bl.TERNARIZE_WORKSPACE_BYTES,), 0x5A, dtype=torch.uint8, device="cuda")
            rc = lib.ternarize_weights_absmean(w.data_ptr(), packed.data_ptr(), scales.data_ptr(),
                                               work.data_ptr(), N, K, st)
        assert rc == 0, (noalloc, rc)
        torch.cuda.synchronize()
        outs.append((packed.cpu().numpy(), host_bits(scales)))
    return outs


def test_noalloc_matches_workspace_entry(bl):
    g = synth.rng(synth.seed_for(9, 7, 0))
    big = synth.weights_bf16(g, 3840, 2560, sigma=0.05)
    small = synth.weights_bf16(g, 640, 512, sigma=0.002)
    for name, w in (("3840x2560", big), ("640x512", small)):
        print(f"noalloc ternarize {name}", flush=True)
        (p_ws, s_ws), (p_na, s_na) = run_both(bl, w)
        np.testing.assert_array_equal(p_na, p_ws, err_msg=name)
        np.testing.assert_array_equal(s_na, s_ws, err_msg=name)
    # the second, smaller call against the oracle as well
    N, K = small.shape
    q, mean, s, ws = oracle.ternarize_absmean(small)
    assert (int(s_na[0]), int(s_na[1]), int(s_na[2])) == (ws, s, mean)
    np.testing.assert_array_equal(oracle.unpack_tiles(p_na, N, K), q)


def test_noalloc_rejects_bad_arguments(bl):
    import torch
    lib = bl.lib()
    st = torch.cuda.current_stream().cuda_stream
    packed = torch.empty(bl.bl_packed_bytes(16, 256), dtype=torch.uint8, device="cuda")
    scales = torch.empty(3, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((16, 256), dtype=torch.bfloat16, device="cuda")
    assert lib.ternarize_weights_absmean_noalloc(None, packed.data_ptr(), scales.data_ptr(),
                                                 16, 256, st) == bl.BL_ERR_NULL
    assert lib.ternarize_weights_absmean_noalloc(w.data_ptr(), packed.data_ptr(), scales.data_ptr(),
                                                 16, 250, st) == bl.BL_ERR_SHAPE
    assert lib.ternarize_weights_absmean_noalloc(w.data_ptr(), packed.data_ptr(), scales.data_ptr(),
                                                 (1 << 24) + 1, 256, st) == bl.BL_ERR_SHAPE
