"""GPU parity of the prompt-processing path (many activation rows, wide layers,
the LDS-tiled MFMA kernel) against the oracle.

The gate+up layer of the pages' 2B model (N=13824, K=2560, two weight
scales) at prompt lengths 128, 256 and 512, activations x ~ N(0,1)
quantised per row on the device: the device quantiser is checked against
the oracle on every row and the layer on sampled rows (each output row
depends only on its own activation row, so the rows the oracle computes
one by one are exact references for the full-size launch).  Smaller
shapes compare every output: M, N and K not multiples of the kernel's
tiles, weight-scale segments that split bands, activation scales from
1e-30 to 3e20, and the bf16 entry point.  int32 accumulators must match exactly; bf16 outputs too
(the bar is 1 ulp; the kernel rounds the exact quotient).
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


def run_i8(bl, w, xq, s, ws_bits, ws_num):
    import torch
    M, K = xq.shape
    N = w.shape[0]
    packed = bl.pack_ternary_weights(dev(w))
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y = bl.bitlinear_i8xi2(dev(xq), packed, dev(s), bf16_dev(ws_bits), N, ws_num, acc=acc)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), host_bits(y)


def check_rows(acc, y, w, xq, s, ws_bits, ws_num, rows):
    acc_o, y_o = oracle.bitlinear_i8(xq[rows], w, s[rows], ws_bits, ws_num)
    np.testing.assert_array_equal(acc[rows], acc_o)
    assert assert_bf16_close(y[rows], y_o, max_ulp=1) == 0


@pytest.mark.parametrize("M", (128, 256, 512))
def test_prefill_gate_up(bl, M):
    import torch
    c = synth.batched(M)   # 13824 x 2560, ws_num = 2, x ~ N(0,1)
    print(f"prefill gate+up M={M}: quantise on the device", flush=True)
    q, s = bl.quantize_act_absmax_i8(dev(c.x))
    torch.cuda.synchronize()
    qo, so = oracle.quant_absmax_i8(c.x)
    np.testing.assert_array_equal(q.cpu().numpy(), qo)
    np.testing.assert_array_equal(s.cpu().numpy(), so)
    print(f"prefill gate+up M={M}: layer", flush=True)
    acc, y = run_i8(bl, c.w, qo, so, c.ws, c.ws_num)
    g = synth.rng(9000 + M)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, M - 1],
                                     g.choice(M, size=10, replace=False)]))
    check_rows(acc, y, c.w, qo, so, c.ws, c.ws_num, rows)


@pytest.mark.parametrize("M,N,K", [(130, 8240, 528), (257, 8192, 272), (128, 8256, 2560), (65, 8256, 528),
                                   (100, 13824, 1024)])
def test_prefill_ragged(bl, M, N, K):
    c = synth.make_int8_gemv(f"p{M}", M, N, K, 1, synth.seed_for(9, 0, M + K))
    print(f"prefill ragged M={M} N={N} K={K}", flush=True)
    acc, y = run_i8(bl, c.w, c.xq, c.s, c.ws, c.ws_num)
    check_rows(acc, y, c.w, c.xq, c.s, c.ws, c.ws_num, np.arange(M))


def test_prefill_segments_and_extremes(bl):
    g = synth.rng(9517)
    M, N, K = 160, 8200, 512           # four weight-scale segments of 2050 rows (not band-aligned)
    w = synth.ternary_uniform(g, N, K)
    w[:300] = 1
    w[300:600] = -1
    xq = synth.int8_uniform(g, M, K, -128, 127)
    xq[0] = -128
    xq[1] = 127
    xq[2] = 0
    s = synth.act_scale(g, M)
    # activation scales far from 1 (their reciprocals beyond 2^45 and below
    # 2^-50): the epilogue's fp64 product and its rounding through fp32 must
    # hold there too
    s[3] = np.float32(1e-30)
    s[4] = np.float32(3e20)
    s[5] = np.float32(2.5e-14)
    ws = synth.ws_bits(g, 4)
    print(f"prefill segments/extremes M={M} N={N} K={K}", flush=True)
    acc, y = run_i8(bl, w, xq, s, ws, 4)
    check_rows(acc, y, w, xq, s, ws, 4, np.arange(M))


def test_prefill_bf16_entry(bl):
    import torch
    M, N, K = 136, 8448, 512
    c = synth.make_float_gemv("bf16_prefill", M, N, K, 2, 31415, bf16=True)
    print(f"prefill bf16 entry M={M} N={N} K={K}", flush=True)
    packed = bl.pack_ternary_weights(dev(c.w))
    q = torch.empty((M, K), dtype=torch.int8, device="cuda")
    s = torch.empty((M,), dtype=torch.float32, device="cuda")
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y = bl.bitlinear_bf16_i8xi2(bf16_dev(c.x), packed, bf16_dev(c.ws), N, 2, q_out=q, s_out=s,
                                acc=acc)
    torch.cuda.synchronize()
    qo, so, acc_o, y_o = oracle.bitlinear_bf16(c.x, c.w, c.ws, 2)
    np.testing.assert_array_equal(q.cpu().numpy(), qo)
    np.testing.assert_array_equal(s.cpu().numpy(), so)
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_o)
    np.testing.assert_array_equal(host_bits(y), y_o)
