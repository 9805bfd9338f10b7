"""Pins of the oracle's weight ternariser ([W2A8] §4.2: s = 1/mean|W|, Wt = clamp(round(W*s), -1, 1), ws = 1/s).

Checked against things other than itself: a second exact rounding routine
(fp64-based, for values fp64 holds exactly), Fraction brute force for the
mean, the page's own torch code on inputs where its fp32 accumulation is
exact, closed forms, ties, the zero matrix and power-of-two scaling.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def bits_of(values):
    """fp32-representable bf16 values -> uint16 bit patterns (exact)."""
    a = np.asarray(values, dtype=np.float32)
    u = a.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "values must be bf16-exact"
    return (u >> 16).astype(np.uint16)


def f32(bits):
    return oracle.bf16_to_f32(np.asarray(bits, dtype=np.uint16))


def test_ratio_rounding_matches_fp64_rounding():
    # values num / 2^k that fp64 holds exactly: the integer routine and the
    # fp64 routine (a different implementation of the same definition) agree
    g = np.random.default_rng(7)
    for _ in range(3000):
        k = int(g.integers(0, 200))
        num = int(g.integers(1, 1 << 52))
        want = int(oracle.bf16_rne(np.array([num / 2.0 ** k]))[0]) if k < 1000 else None
        assert oracle.bf16_rne_ratio(num, 1 << k) == want


@pytest.mark.parametrize("num,den,want", [
    (1, 1, 0x3F80),                       # 1.0
    (3, 2, 0x3FC0),                       # 1.5
    ((256 + 1), 256, 0x3F80),             # 1 + 2^-8: a tie below even 1.0 -> 1.0
    ((256 + 3), 256, 0x3F82),             # 1 + 3*2^-8: a tie -> even 1 + 2^-6
    ((512 + 3), 512, 0x3F81),             # 1 + 0.75 * 2^-7: above the tie -> 1 + 2^-7
    (1, 3, 0x3EAB),                       # 1/3
    (1, 1 << 133, 0x0001),                # smallest subnormal
    (1, 1 << 134, 0x0000),                # half of it: a tie to even 0
    (3, 1 << 135, 0x0001),                # 0.75 of it -> 1
    ((1 << 8) - 1, 1 << 7, 0x3FFF),       # 1 + 127/128 is a bf16 value
    ((1 << 9) - 1, 1 << 8, 0x4000),       # 1 + 255/256: a tie -> even 2.0 (carry into the exponent)
    (1 << 128, 1, 0x7F80),                # 2^128 -> inf
])
def test_ratio_rounding_cases(num, den, want):
    assert oracle.bf16_rne_ratio(num, den) == want


def test_mean_matches_fraction_brute_force():
    g = np.random.default_rng(11)
    for trial in range(40):
        n = int(g.integers(1, 300))
        # magnitudes over a wide range, including subnormals and zeros
        e = g.integers(-140, 20, size=n).astype(np.float64)
        v = (g.standard_normal(n) * np.exp2(e)).astype(np.float32)
        b = (v.view(np.uint32) >> 16).astype(np.uint16)
        b[g.random(n) < 0.1] = 0
        exact = sum((Fraction(float(x)) for x in np.abs(f32(b)).astype(np.float64)), Fraction(0)) / n
        assert oracle.absmean_bf16(b) == oracle.bf16_rne_ratio(exact.numerator, exact.denominator)


def test_constant_magnitude_closed_form():
    # |w| = 0.25 everywhere: mean 0.25, s = 4, ws = 0.25, Wt = sign(W)
    g = np.random.default_rng(3)
    sign = np.where(g.random((16, 48)) < 0.5, -1.0, 1.0)
    q, mean, s, ws = oracle.ternarize_absmean(bits_of(0.25 * sign))
    assert (mean, s, ws) == (0x3E80, 0x4080, 0x3E80)
    np.testing.assert_array_equal(q, sign.astype(np.int8))


def test_ties_round_half_to_even():
    # mean exactly 0.25 -> s = 4; w*s = 0.5 -> 0, 1.5 -> 2 -> clamp 1, 0.75 -> 1, 0.25 -> 0
    w = np.array([[0.125, 0.375, -0.125, -0.375, 0.1875, 0.3125, 0.0625, 0.4375]], dtype=np.float32)
    q, mean, s, ws = oracle.ternarize_absmean(bits_of(w))
    assert f32([mean])[0] == 0.25 and f32([s])[0] == 4.0
    np.testing.assert_array_equal(q[0], [0, 1, 0, -1, 1, 1, 0, 1])


def test_zero_matrix_uses_the_floor():
    q, mean, s, ws = oracle.ternarize_absmean(np.zeros((4, 32), dtype=np.uint16))
    floor = int(oracle.bf16_rne(np.array([np.float32(1e-5)], dtype=np.float64))[0])
    assert mean == 0
    want_s = int(oracle.bf16_rne(np.array([np.float32(1.0) / f32([floor])[0]], dtype=np.float64))[0])
    assert s == want_s
    assert not q.any()


def test_power_of_two_scaling():
    g = np.random.default_rng(5)
    v = (g.standard_normal((32, 64)) * 0.02).astype(np.float32)
    b = (v.view(np.uint32) >> 16).astype(np.uint16)
    q0, m0, s0, ws0 = oracle.ternarize_absmean(b)
    for j in (-3, 4):
        v2 = f32(b) * np.float32(2.0 ** j)
        q1, m1, s1, ws1 = oracle.ternarize_absmean(bits_of(v2))
        np.testing.assert_array_equal(q1, q0)
        assert f32([m1])[0] == f32([m0])[0] * 2.0 ** j
        assert f32([s1])[0] == f32([s0])[0] * 2.0 ** -j
        assert f32([ws1])[0] == f32([ws0])[0] * 2.0 ** j


def test_matches_the_pages_torch_code_where_its_sum_is_exact():
    # The page's converter, run as written on bf16 tensors.  Inputs are
    # multiples of 2^-8 in [-1, 1] and n = 4096, so torch's fp32 sum and its
    # division by n are exact and its mean is the exact mean, rounded to bf16.
    torch = pytest.importorskip("torch")

    def quant_weight_int8(weight):          # [W2A8] §4.2, as printed on the page
        s = 1.0 / weight.abs().mean().clamp_(min=1e-5)
        new_weight = (weight * s).round().clamp(-1, 1).to(torch.int8)
        new_scale = (1.0 / s).to(torch.bfloat16)
        return new_weight, new_scale.reshape(1)

    g = np.random.default_rng(9)
    for trial in range(20):
        v = (g.integers(-256, 257, size=(64, 64)) / 256.0).astype(np.float32)
        v *= (g.random((64, 64)) < 0.8)
        b = bits_of(v)
        wt, ws_t = quant_weight_int8(torch.from_numpy(v).to(torch.bfloat16))
        q, mean, s, ws = oracle.ternarize_absmean(b)
        np.testing.assert_array_equal(q, wt.numpy())
        assert ws == int(ws_t.view(torch.int16).numpy()[0]) & 0xFFFF


def test_mean_exactly_on_a_tie_and_one_subnormal_above():
    # 256 entries summing to 257 plus 256 zeros: mean = 0.5 * (1 + 2^-8), a bf16
    # tie that rounds to even 0.5; one zero raised to 2^-133 puts the mean just
    # above it (rounds up to 0.5 + 2^-8).  Only an exact sum sees the difference.
    v = np.zeros(512, dtype=np.float32)
    v[0:512:2][:255] = 1.0
    v[510] = 2.0
    b = bits_of(v).reshape(16, 32)
    assert oracle.absmean_bf16(b) == 0x3F00
    b[0, 1] = 0x0001
    assert oracle.absmean_bf16(b) == 0x3F01
