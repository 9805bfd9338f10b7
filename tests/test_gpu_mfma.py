"""GPU parity of the batched (M >= 2) path on int8 MFMA against the oracle.

The batched workload of the pages' model shapes (M in {16, 32, 64},
N=13824, K=2560, per-row absmax quantisation of x ~ N(0,1) on the device),
plus M that are not multiples of 16 or exceed one 64-row workgroup column,
and ragged N and K.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev, bf16_dev, host_bits, assert_bf16_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bit_gemv_bitlinear_amd as m
    return m


def check(bl, name, w, xq, s, ws_bits, ws_num):
    import torch
    M, K = xq.shape
    N = w.shape[0]
    print(f"mfma {name} M={M} N={N} K={K}", flush=True)
    packed = bl.pack_ternary_weights(dev(w))
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y = bl.bitlinear_i8xi2(dev(xq), packed, dev(s), bf16_dev(ws_bits), N, ws_num, acc=acc)
    torch.cuda.synchronize()
    acc_o, y_o = oracle.bitlinear_i8(xq, w, s, ws_bits, ws_num)
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_o)
    assert assert_bf16_close(host_bits(y), y_o, max_ulp=1) == 0


@pytest.mark.parametrize("M", synth.BATCHED_M)
def test_batched_model_shape(bl, M):
    import torch
    c = synth.batched(M)
    print(f"batched M={M}: quantise on the device", flush=True)
    q, s = bl.quantize_act_absmax_i8(dev(c.x))
    torch.cuda.synchronize()
    qo, so = oracle.quant_absmax_i8(c.x)
    np.testing.assert_array_equal(q.cpu().numpy(), qo)
    np.testing.assert_array_equal(s.cpu().numpy(), so)
    check(bl, c.name, c.w, qo, so, c.ws, c.ws_num)


@pytest.mark.parametrize("M,N,K", [(2, 64, 64), (15, 100, 208), (16, 64 * 3, 2560), (17, 130, 80),
                                   (33, 640, 6912), (64, 256, 1024), (65, 192, 144),
                                   (130, 70, 272), (64, 2560, 13824),
                                   (2, 2560, 6912), (16, 2560, 6912), (7, 130, 2576), (12, 4000, 5120)])
def test_shapes(bl, M, N, K):
    # M <= 16 with K > 2560 (the last four) runs the streaming kernel with one
    # m tile: the down projection of a decode batch, K just past the band
    # kernel's range with N ragged, and a K = 5120 layer
    c = synth.make_int8_gemv(f"m{M}", M, N, K, 1, synth.seed_for(8, 0, M + N % 89))
    check(bl, c.name, c.w, c.xq, c.s, c.ws, c.ws_num)


@pytest.mark.parametrize("M,N,K,ws_num", [(3, 16, 16, 1), (2, 1, 2560, 1), (31, 1000, 2304, 4),
                                          (32, 13824, 2560, 2), (20, 100, 2560, 4), (9, 4096, 256, 8),
                                          (24, 48, 1040, 3),
                                          (33, 13824, 2560, 2), (47, 1030, 2304, 2), (64, 2432, 272, 1),
                                          (40, 24, 1040, 3), (64, 2048, 2560, 4), (50, 128, 16, 1)])
def test_band_kernel_shapes(bl, M, N, K, ws_num):
    # 2 <= M <= 64 with K <= 2560 runs the band kernel: one 256-K tile or ten,
    # a single output row, rows not filling the last workgroup, weight-scale
    # segments that split bands, K not a multiple of 256.  M = 33 .. 64 takes
    # two bands per wavefront and two groups of 32 rows, whose workgroup ids
    # are 8 apart within runs of 8 band groups: whole runs (2048 rows), runs
    # and a tail of 1 .. 7 groups (1030: 9 groups; 2432: 19), only a tail (24,
    # 128 rows), and a second group of 1 .. 31 rows (33, 47, 50)
    c = synth.make_int8_gemv(f"band_m{M}", M, N, K, ws_num, synth.seed_for(8, 1, M + N % 97))
    check(bl, c.name, c.w, c.xq, c.s, c.ws, c.ws_num)


@pytest.mark.parametrize("M,N", [(64, 13824), (33, 1030), (20, 13824)])
def test_band_kernel_without_acc(bl, M, N):
    # y alone (no int32 output), as the bench and most callers run it; the
    # rows of both row groups and a ragged last band
    import torch
    K = 2560
    c = synth.make_int8_gemv(f"band_y_m{M}", M, N, K, 2, synth.seed_for(8, 2, M + N % 89))
    print(f"mfma band y only M={M} N={N}", flush=True)
    packed = bl.pack_ternary_weights(dev(c.w))
    y = bl.bitlinear_i8xi2(dev(c.xq), packed, dev(c.s), bf16_dev(c.ws), N, 2)
    torch.cuda.synchronize()
    _, y_o = oracle.bitlinear_i8(c.xq, c.w, c.s, c.ws, 2)
    assert assert_bf16_close(host_bits(y), y_o, max_ulp=1) == 0


@pytest.mark.parametrize("M", [32, 64])
def test_extremes_and_segments(bl, M):
    # the largest sums of either sign in both row groups (M = 64: rows 32 .. 34)
    g = synth.rng(515)
    N, K = 64 * 4, 2560
    w = synth.ternary_uniform(g, N, K)
    w[:64] = 1
    w[64:128] = -1
    xq = synth.int8_uniform(g, M, K, -128, 127)
    for r0 in range(0, M, 32):
        xq[r0] = -128
        xq[r0 + 1] = 127
        xq[r0 + 2] = 0
    s = synth.act_scale(g, M)
    check(bl, f"extremes_ws4_m{M}", w, xq, s, synth.ws_bits(g, 4), 4)


@pytest.mark.parametrize("M,N,K", [(48, 640, 2560), (16, 1000, 2560), (32, 13824, 2560),
                                   (40, 640, 4096)])
def test_bf16_entry_with_staging(bl, M, N, K):
    # the bf16 entry quantises into q_out / s_out, then runs the layer kernel
    # for M >= 2: the band kernel for K <= 2560 (M = 48: two row groups), the
    # streaming kernel for K = 4096
    import torch
    c = synth.make_float_gemv(f"bf16_m{M}", M, N, K, 2, 2718 + M, bf16=True)
    print(f"mfma bf16 entry M={M}", flush=True)
    packed = bl.pack_ternary_weights(dev(c.w))
    q = torch.empty((M, K), dtype=torch.int8, device="cuda")
    s = torch.empty((M,), dtype=torch.float32, device="cuda")
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y = bl.bitlinear_bf16_i8xi2(bf16_dev(c.x), packed, bf16_dev(c.ws), N, 2, q_out=q, s_out=s,
                                acc=acc)
    torch.cuda.synchronize()
    qo, so, acc_o, y_o = oracle.bitlinear_bf16(c.x, c.w, c.ws, 2)
    np.testing.assert_array_equal(q.cpu().numpy(), qo)
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_o)
    np.testing.assert_array_equal(host_bits(y), y_o)
