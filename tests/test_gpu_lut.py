"""GPU parity of the table-lookup GEMV (bitlinear_lut_i8xi2) against the oracle,
and against the dot-product GEMV it cross-checks.

The lookup kernel computes the same exact int32 sums by another route (a table
of the 16 sums of every activation pair, indexed by the 4-bit code pairs of the
packed words), so the oracle is the layer's definition: int32 accumulators and
bf16 outputs bit-exact, and identical to bitlinear_i8xi2's.  Shapes: the 2B
layer set (qkv, o, gate+up, down: K = 2560 and 6912, within the kernel's
K <= 8192), ragged N and K, the smallest and the largest K, rows of all +1,
all -1 and all 0 weights against activations at -128 and 127, and
weight-scale segments.
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


def check_lut(bl, name, w, xq, s, ws_bits, ws_num):
    import torch
    N, K = w.shape
    print(f"gemv_lut {name} N={N} K={K} ws_num={ws_num}", flush=True)
    packed = bl.pack_ternary_weights(dev(w))
    acc = torch.empty((N,), dtype=torch.int32, device="cuda")
    y = bl.bitlinear_lut_i8xi2(dev(xq.reshape(-1)), packed, dev(s), bf16_dev(ws_bits), N, ws_num,
                               acc=acc)
    acc_d = torch.empty((1, N), dtype=torch.int32, device="cuda")
    y_d = bl.bitlinear_i8xi2(dev(xq.reshape(1, -1)), packed, dev(s), bf16_dev(ws_bits), N, ws_num,
                             acc=acc_d)
    torch.cuda.synchronize()
    acc_o, y_o = oracle.bitlinear_i8(xq.reshape(1, -1), w, s, ws_bits, ws_num)
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_o.reshape(-1), err_msg=f"{name}: acc")
    np.testing.assert_array_equal(host_bits(y).reshape(-1), y_o.reshape(-1), err_msg=f"{name}: y")
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_d.cpu().numpy().reshape(-1))
    np.testing.assert_array_equal(host_bits(y).reshape(-1), host_bits(y_d).reshape(-1))


@pytest.mark.parametrize("idx", range(len(synth.LAYER_SET)))
def test_lut_layer_set(bl, idx):
    c = synth.layer_set()[idx]
    check_lut(bl, c.name, c.w, c.xq, c.s, c.ws, c.ws_num)


# (12816, 2320): a wide matrix (801 bands) with a ragged row of 10 steps, one
# wavefront per band; the others split each band's steps over wavefronts
@pytest.mark.parametrize("N,K,ws_num", [(100, 272, 2), (1, 16, 1), (17, 8192, 1), (3000, 4096, 4),
                                        (8200, 512, 1), (64, 8176, 2), (12816, 2320, 2)])
def test_lut_ragged(bl, N, K, ws_num):
    c = synth.make_int8_gemv(f"lut{N}x{K}", 1, N, K, ws_num, synth.seed_for(10, 0, N + K))
    check_lut(bl, c.name, c.w, c.xq, c.s, c.ws, c.ws_num)


def test_lut_extremes(bl):
    g = synth.rng(1201)
    N, K = 2048, 2304        # four weight-scale segments of 512 rows
    w = synth.ternary_uniform(g, N, K)
    w[:64] = 1
    w[64:128] = -1
    w[128:192] = 0
    xq = synth.int8_uniform(g, 1, K, -128, 127)
    xq[0, : K // 2] = -128
    xq[0, K // 2:] = 127
    s = synth.act_scale(g, 1)
    ws = synth.ws_bits(g, 4)
    check_lut(bl, "extremes", w, xq, s, ws, 4)
