"""Pins of the oracle's epilogue (W2A8 page §5.3): y = bf16_rne(acc * ws[seg(n)] / s[m]).

The bf16 rounding is checked against torch's fp32 -> bf16 conversion and
against an exact rational-arithmetic rounding written here with fractions;
the epilogue against closed forms (zero, exact small integers, power-of-two
scales, the N-segment that picks each weight scale).
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _bf16_value(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _exact_rne_bf16(v) -> int:
    """Round v (a float or an exact Fraction) to bf16 by comparing exact distances
    to its two bf16 neighbours."""
    if v == 0:
        return 0x8000 if isinstance(v, float) and math.copysign(1.0, v) < 0 else 0
    sign = 0x8000 if v < 0 else 0
    a = abs(Fraction(v))
    # largest finite bf16 magnitude pattern is 0x7F7F; search the monotone bit patterns
    lo, hi = 0, 0x7F7F
    while lo < hi:                      # last pattern whose value <= a
        mid = (lo + hi + 1) // 2
        if Fraction(_bf16_value(mid)) <= a:
            lo = mid
        else:
            hi = mid - 1
    below = lo
    if Fraction(_bf16_value(below)) == a:
        return sign | below
    above = below + 1                  # 0x7F80 is +inf: the "next value" past the max
    vb = Fraction(_bf16_value(below))
    va = Fraction(2) ** 128 if above == 0x7F80 else Fraction(_bf16_value(above))
    db, da = a - vb, va - a
    if db < da or (db == da and below % 2 == 0):
        return sign | below
    return sign | above


def test_matches_torch_on_fp32_values():
    g = np.random.Generator(np.random.PCG64(31))
    bits = g.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ours = oracle.bf16_rne(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_matches_exact_rational_rounding():
    g = np.random.Generator(np.random.PCG64(32))
    vals = list(g.standard_normal(300) * 10.0 ** g.integers(-40, 39, 300))
    # ties and near-ties of bf16 at several magnitudes, and values near the overflow point
    for base in (1.0, 3.0, 2.0 ** -130, 2.0 ** 100, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8):
        vals += [base, base * (1 + 2 ** -40), base * (1 - 2 ** -40)]
    vals += [3.3895313892515355e38, 3.3961775292304957e38, 3.4e38, -3.4e38, 1e-45, -9.2e-41]
    ours = oracle.bf16_rne(np.array(vals, dtype=np.float64))
    for v, b in zip(vals, ours):
        assert int(b) == _exact_rne_bf16(float(v)), v


def test_special_values():
    out = oracle.bf16_rne(np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e39, -1e39]))
    assert out[0] == 0x0000 and out[1] == 0x8000
    assert out[2] == 0x7F80 and out[3] == 0xFF80
    assert (out[4] & 0x7F80) == 0x7F80 and (out[4] & 0x007F) != 0
    assert out[5] == 0x7F80 and out[6] == 0xFF80


def _bf16(x):
    return oracle.bf16_rne(np.array([x], dtype=np.float64))[0]


def test_epilogue_closed_forms():
    acc = np.array([[0, 1, -1, 255, -256, 100, 7, -3]], dtype=np.int32)
    one = np.array([_bf16(1.0)], dtype=np.uint16)
    y = oracle.epilogue_bf16(acc, np.array([1.0], np.float32), one, 1)
    np.testing.assert_array_equal(oracle.bf16_to_f32(y), acc.astype(np.float32))
    # s = 4 divides, ws = 0.5 multiplies: y = acc * 0.5 / 4 exactly
    y2 = oracle.epilogue_bf16(acc, np.array([4.0], np.float32),
                              np.array([_bf16(0.5)], np.uint16), 1)
    np.testing.assert_array_equal(oracle.bf16_to_f32(y2), (acc / 8.0).astype(np.float32))


def test_epilogue_segments_pick_their_scale():
    N = 12
    acc = np.ones((2, N), dtype=np.int32) * 3
    ws = np.array([_bf16(1.0), _bf16(2.0), _bf16(4.0)], dtype=np.uint16)
    s = np.array([1.0, 0.5], dtype=np.float32)
    y = oracle.bf16_to_f32(oracle.epilogue_bf16(acc, s, ws, 3))
    expect_row = np.repeat([3.0, 6.0, 12.0], 4)
    np.testing.assert_array_equal(y[0], expect_row)
    np.testing.assert_array_equal(y[1], expect_row * 2)


def test_epilogue_general_value_is_rounded_quotient():
    g = np.random.Generator(np.random.PCG64(33))
    acc = g.integers(-400000, 400000, size=(3, 64)).astype(np.int32)
    s = np.array([127 / 3.7, 127 / 0.9, 127 / 1e-5], dtype=np.float32)
    ws = np.array([_bf16(1.2), _bf16(0.75)], dtype=np.uint16)
    y = oracle.epilogue_bf16(acc, s, ws, 2)
    for m in range(3):
        for n in range(64):
            wsv = float(oracle.bf16_to_f32(ws[n // 32])[0])
            exact = Fraction(int(acc[m, n])) * Fraction(wsv) / Fraction(float(s[m]))
            # the oracle rounds the fp64 quotient; it must be the bf16 nearest to the exact value
            assert int(y[m, n]) == _exact_rne_bf16(exact)
