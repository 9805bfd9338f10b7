"""GPU parity at the largest shapes the library accepts, against the oracle.

N = 2^24 output rows (the limit) at K = 16 with 64 weight-scale segments:
the row-to-segment multiply-shift over its whole range (n up to 2^24 - 1),
2^20 bands, a 1 GiB packed matrix, through the int8 GEMV and the fused bf16
one.  Many activation rows: M = 8192 on the streaming MFMA kernel (a narrow
layer, 128 workgroup rows), M = 4096 on the LDS-tiled one (N = 8192), and the
per-token quantiser over 65536 rows.  Every int32 and bf16 output, and every
quantised value and scale, must equal the oracle's.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev, bf16_dev, host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bit_gemv_bitlinear_amd as m
    return m


def check_layer(bl, name, w, xq, s, ws_bits, ws_num):
    import torch
    M, K = xq.shape
    N = w.shape[0]
    print(f"limits {name}: M={M} N={N} K={K} ws_num={ws_num}", flush=True)
    packed = bl.pack_ternary_weights(dev(w))
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y = bl.bitlinear_i8xi2(dev(xq), packed, dev(s), bf16_dev(ws_bits), N, ws_num, acc=acc)
    torch.cuda.synchronize()
    acc_o, y_o = oracle.bitlinear_i8(xq, w, s, ws_bits, ws_num)
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_o, err_msg=f"{name}: acc")
    np.testing.assert_array_equal(host_bits(y), y_o, err_msg=f"{name}: y")
    return packed


@pytest.mark.parametrize("fused", [False, True])
def test_gemv_at_the_row_limit(bl, fused):
    import torch
    N, K, ws_num = 1 << 24, 16, 64
    g = synth.rng(2424)
    w = synth.ternary_uniform(g, N, K)
    ws = synth.ws_bits(g, ws_num)
    if not fused:
        xq = synth.int8_uniform(g, 1, K)
        check_layer(bl, "gemv", w, xq, synth.act_scale(g, 1), ws, ws_num)
        return
    x = synth.normal_bf16_bits(g, 1, K)
    print(f"limits fused gemv: N={N} K={K} ws_num={ws_num}", flush=True)
    packed = bl.pack_ternary_weights(dev(w))
    acc = torch.empty((1, N), dtype=torch.int32, device="cuda")
    y = bl.bitlinear_bf16_i8xi2(bf16_dev(x), packed, bf16_dev(ws), N, ws_num, acc=acc)
    torch.cuda.synchronize()
    qo, so = oracle.quant_absmax_i8(x, bf16=True)
    acc_o, y_o = oracle.bitlinear_i8(qo, w, so, ws, ws_num)
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_o, err_msg="fused: acc")
    np.testing.assert_array_equal(host_bits(y), y_o, err_msg="fused: y")


def test_many_rows_streaming_mfma(bl):
    c = synth.make_int8_gemv("tall_narrow", 8192, 64, 32, 2, synth.seed_for(11, 0, 1))
    check_layer(bl, c.name, c.w, c.xq, c.s, c.ws, c.ws_num)


def test_many_rows_tiled_mfma(bl):
    c = synth.make_int8_gemv("tall_wide", 4096, 8192, 16, 4, synth.seed_for(11, 0, 2))
    check_layer(bl, c.name, c.w, c.xq, c.s, c.ws, c.ws_num)


def test_quantiser_many_rows(bl):
    import torch
    g = synth.rng(6553)
    x = synth.normal_bf16_bits(g, 65536, 32)
    print("limits quantiser: M=65536 K=32", flush=True)
    q, s = bl.quantize_act_absmax_i8(bf16_dev(x))
    torch.cuda.synchronize()
    qo, so = oracle.quant_absmax_i8(x, bf16=True)
    np.testing.assert_array_equal(q.cpu().numpy(), qo)
    np.testing.assert_array_equal(s.cpu().numpy(), so)
