"""Pins of the oracle's weight ternariser ([W2A8] §4.2: s = 1/mean|W|, Wt = clamp(round(W*s), -1, 1), ws = 1/s).

Checked against things other than itself: a second exact rounding routine
(fp64-based, for values fp64 holds exactly), Fraction brute force for the
mean, the whole definition evaluated in exact rational arithmetic with every
rounding written out, closed forms, ties, the zero matrix and power-of-two
scaling.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from exact_bf16 import bf16_bits, bits_to_fraction, r32


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


def ternarize_by_definition(w_bits):
    """[W2A8] §4.2 in exact arithmetic: the mean of |W| (exact, rounded once to bf16), the
    multiplier s = 1 / max(mean, 1e-5) and the weight scale ws = 1 / s (each an fp32
    operation rounded to bf16), Wt = clamp(round(bf16(fl32(w * s))), -1, 1) with ties to
    even.  Every rounding is written out on Fractions (tests/exact_bf16.py)."""
    vals = [bits_to_fraction(b) for b in np.asarray(w_bits, dtype=np.uint16).reshape(-1)]
    mean = sum(abs(v) for v in vals) / len(vals)
    mean_b = bf16_bits(mean)
    m = bits_to_fraction(mean_b)
    floor = r32(Fraction(1, 100000))                  # 1e-5 as fp32
    if m < floor:
        m = bits_to_fraction(bf16_bits(floor))
    s_b = bf16_bits(r32(1 / m))
    s = bits_to_fraction(s_b)
    ws_b = bf16_bits(r32(1 / s))
    q = [max(-1, min(1, round(bits_to_fraction(bf16_bits(r32(v * s)))))) for v in vals]
    return np.array(q, dtype=np.int8).reshape(np.shape(w_bits)), mean_b, s_b, ws_b


@pytest.mark.parametrize("trial", range(12))
def test_matches_the_definition_in_exact_arithmetic(trial):
    # random bf16 matrices over a range of magnitudes (some rows of zeros, some
    # outliers), against the definition evaluated in exact rational arithmetic
    g = np.random.default_rng(100 + trial)
    N, K = 16, 48
    scale = 2.0 ** int(g.integers(-20, 10))
    v = (g.standard_normal((N, K)) * scale).astype(np.float32)
    v[int(g.integers(0, N))] = 0.0
    v[int(g.integers(0, N)), int(g.integers(0, K))] *= 50.0
    b = (v.view(np.uint32) >> 16).astype(np.uint16)     # cut to bf16
    want = ternarize_by_definition(b)
    got = oracle.ternarize_absmean(b)
    np.testing.assert_array_equal(got[0], want[0])
    assert tuple(int(x) for x in got[1:]) == tuple(int(x) for x in want[1:])


def test_closed_forms():
    # all |w| equal to c: the mean is c, every w * s is about +-1 -> Wt = sign(w)
    for c in (1.0, 0.375, 2.0 ** -9, 3.0):
        v = np.full((16, 32), c, dtype=np.float32)
        v[::3] *= -1.0
        v[5] = 0.0
        b = bits_of(v)
        q, mean, s, ws = oracle.ternarize_absmean(b)
        np.testing.assert_array_equal(q, np.sign(v).astype(np.int8))
        # mean over 512 entries, a row of 32 of them zero: c * 15 / 16 (a bf16 value)
        assert mean == int(bits_of([np.float32(c * 15 / 16)])[0])
    # a matrix of zeros: mean 0 < 1e-5 -> s = bf16(1 / bf16(1e-5)), Wt = 0
    q, mean, s, ws = oracle.ternarize_absmean(np.zeros((16, 32), dtype=np.uint16))
    assert mean == 0 and not q.any()
    assert s == bf16_bits(r32(1 / bits_to_fraction(bf16_bits(r32(Fraction(1, 100000))))))


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
