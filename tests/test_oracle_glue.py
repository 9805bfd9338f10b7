"""Pins of the oracle's glue between a block's projections: RMSNorm, the
squared-ReLU GLU and the residual add (readings of the model [W2A8] §4.1
names; see oracle.c).

Each is checked against something other than the oracle itself: exact
rational arithmetic (Python Fractions, with bf16 round-to-nearest-even
written out from the format's definition here), torch's fp64 rms_norm as a
library reference, and closed forms / invariants.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from exact_bf16 import bf16_bits_of_exact, bits_to_fraction, rmsnorm_exact


def rand_bf16(g, n, scale=1.0):
    return oracle.bf16_rne(g.normal(size=n) * scale)


@pytest.mark.parametrize("K,scale", [(1, 1.0), (7, 3.0), (64, 1.0), (300, 0.01), (2560, 1.0)])
def test_rmsnorm_against_exact(K, scale):
    g = np.random.default_rng(100 + K)
    x = rand_bf16(g, K, scale)
    w = oracle.bf16_rne(1.0 + 0.1 * g.normal(size=K))
    np.testing.assert_array_equal(oracle.rmsnorm_bf16(x, w), rmsnorm_exact(x, w))


def test_rmsnorm_wide_range_against_exact():
    g = np.random.default_rng(7)
    x = oracle.bf16_rne(g.normal(size=200) * np.exp2(g.integers(-40, 20, size=200)))
    x[:3] = [0, 0x8000, 0x3F80]      # +0, -0, 1.0
    w = oracle.bf16_rne(g.normal(size=200))
    np.testing.assert_array_equal(oracle.rmsnorm_bf16(x, w), rmsnorm_exact(x, w))


def test_rmsnorm_against_torch_fp64():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(11)
    K = 6912
    x = rand_bf16(g, K)
    w = oracle.bf16_rne(1.0 + 0.2 * g.normal(size=K))
    xt = torch.from_numpy(oracle.bf16_to_f32(x).astype(np.float64))
    wt = torch.from_numpy(oracle.bf16_to_f32(w).astype(np.float64))
    ref = torch.nn.functional.rms_norm(xt, (K,), weight=wt, eps=float(np.float32(1e-5)))
    np.testing.assert_array_equal(oracle.rmsnorm_bf16(x, w), oracle.bf16_rne(ref.numpy()))


def test_rmsnorm_closed_forms():
    one = np.full(16, 0x3F80, dtype=np.uint16)
    # constant row c with weight 1: c / sqrt(c^2 + eps) = 0.999995 -> 1.0 for c = 1
    np.testing.assert_array_equal(oracle.rmsnorm_bf16(one, one), one)
    # zero row -> zeros; zero weight -> zeros
    zero = np.zeros(16, dtype=np.uint16)
    np.testing.assert_array_equal(oracle.rmsnorm_bf16(zero, one), zero)
    g = np.random.default_rng(3)
    x = rand_bf16(g, 16)
    assert not np.any(oracle.rmsnorm_bf16(x, zero) & 0x7FFF)
    # without eps the norm is invariant under scaling by a power of two
    w = oracle.bf16_rne(g.normal(size=16))
    x2 = oracle.bf16_rne(oracle.bf16_to_f32(x).astype(np.float64) * 2.0 ** 9)
    np.testing.assert_array_equal(oracle.rmsnorm_bf16(x, w, eps=0.0), oracle.rmsnorm_bf16(x2, w, eps=0.0))
    # a single element: x / sqrt(x^2 + eps) -> sign(x) * w for |x| >> sqrt(eps)
    np.testing.assert_array_equal(
        oracle.rmsnorm_bf16(np.array([0xC080], np.uint16), np.array([0x4000], np.uint16)),
        np.array([0xC000], np.uint16))


def exact_glu(gb, ub):
    gv, uv = bits_to_fraction(gb), bits_to_fraction(ub)
    r = gv if gv > 0 else Fraction(0)
    v = r * r * uv
    if v == 0:
        # fp64: (+0) * up keeps up's sign
        return 0x8000 if (int(ub) & 0x8000) else 0
    return bf16_bits_of_exact(v)


def test_relu2_glu_against_exact():
    g = np.random.default_rng(5)
    gate = rand_bf16(g, 500, 2.0)
    up = rand_bf16(g, 500, 2.0)
    gate[:4] = [0, 0x8000, 0x3F80, 0xBF80]   # +0, -0, 1, -1
    up[:4] = [0xBF80, 0x3F80, 0xC040, 0x4040]
    want = np.array([exact_glu(a, b) for a, b in zip(gate, up)], dtype=np.uint16)
    np.testing.assert_array_equal(oracle.relu2_glu_bf16(gate, up), want)


def test_relu2_glu_closed_forms():
    # negative gate -> signed zero; gate 2, up 3 -> 12; overflow -> inf
    gate = np.array([0xC000, 0x4000, 0x7100], dtype=np.uint16)     # -2, 2, 2^99
    up = np.array([0x4040, 0x4040, 0x7100], dtype=np.uint16)       # 3, 3, 2^99
    np.testing.assert_array_equal(oracle.relu2_glu_bf16(gate, up),
                                  np.array([0x0000, 0x4140, 0x7F80], dtype=np.uint16))


def test_add_against_exact():
    g = np.random.default_rng(9)
    a = rand_bf16(g, 1000)
    b = oracle.bf16_rne(g.normal(size=1000) * np.exp2(g.integers(-60, 8, size=1000)))
    b[:3] = [a[0] ^ 0x8000, 0, 0x8000]       # cancellation -> +0, and signed zeros
    want = []
    for x, y in zip(a, b):
        v = bits_to_fraction(x) + bits_to_fraction(y)
        if v == 0:
            both_neg = (int(x) & 0x8000) and (int(y) & 0x8000)
            want.append(0x8000 if both_neg else 0)
        else:
            want.append(bf16_bits_of_exact(v))
    np.testing.assert_array_equal(oracle.add_bf16(a, b), np.array(want, dtype=np.uint16))


def test_rmsnorm_midpoint_closed_form():
    # K = 16: four values 1.5, seven 1.0, five 0 -> sum of squares 16, mean 1;
    # gamma = 129/128.  With eps = 0, inv = 1 and 1.5 * 129/128 = 193.5/128 is
    # a bf16 midpoint: ties to even -> 194/128 (0x3FC2).  With eps = 2^-28,
    # inv = 1/sqrt(1 + 2^-28) sits just below 1, so the value falls just below
    # the midpoint -> 193/128 (0x3FC1), although its nearest fp32 is the
    # midpoint itself (a rounding through fp32 would give 0x3FC2).  The ones
    # give 129/128 (0x3F81) either way.
    x = np.array([0x3FC0] * 4 + [0x3F80] * 7 + [0] * 5, dtype=np.uint16)
    g = np.full(16, 0x3F81, dtype=np.uint16)
    want0 = np.array([0x3FC2] * 4 + [0x3F81] * 7 + [0] * 5, dtype=np.uint16)
    want1 = np.array([0x3FC1] * 4 + [0x3F81] * 7 + [0] * 5, dtype=np.uint16)
    np.testing.assert_array_equal(oracle.rmsnorm_bf16(x, g, eps=0.0), want0)
    np.testing.assert_array_equal(oracle.rmsnorm_bf16(x, g, eps=np.float32(2.0 ** -28)), want1)
