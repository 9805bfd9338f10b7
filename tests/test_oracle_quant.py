"""Pins of the oracle's per-token absmax int8 quantiser (W2A8 page §六 item 3).

s = 127 / max(max|x|, 1e-5) in fp32; q = clamp(round_half_even(x * s), -128, 127).
Checked against numpy's float32 arithmetic (an independent IEEE implementation),
closed forms (integer rows, ties), and invariants (extremes, symmetry,
power-of-two scaling, zero rows).
"""
import numpy as np
import pytest

import oracle


def _numpy_quant(x):
    x = np.asarray(x, dtype=np.float32)
    amax = np.maximum(np.abs(x).max(axis=1), np.float32(1e-5)).astype(np.float32)
    s = (np.float32(127.0) / amax).astype(np.float32)
    prod = (x * s[:, None]).astype(np.float32)
    q = np.clip(np.rint(prod), -128, 127).astype(np.int8)
    return q, s


def test_matches_numpy_float32():
    g = np.random.Generator(np.random.PCG64(21))
    x = g.standard_normal((16, 2560), dtype=np.float32)
    x[3] *= 1e-3
    x[4] *= 1e4
    x[5] = g.uniform(-1, 1, 2560).astype(np.float32)
    q, s = oracle.quant_absmax_i8(x)
    qn, sn = _numpy_quant(x)
    np.testing.assert_array_equal(q, qn)
    np.testing.assert_array_equal(s.view(np.uint32), sn.view(np.uint32))


def test_extreme_maps_to_127():
    g = np.random.Generator(np.random.PCG64(22))
    x = g.standard_normal((64, 777), dtype=np.float32)
    q, _ = oracle.quant_absmax_i8(x)
    idx = np.abs(x).argmax(axis=1)
    ext = q[np.arange(64), idx]
    assert (np.abs(ext) == 127).all()
    assert (np.sign(ext) == np.sign(x[np.arange(64), idx])).all()
    assert (np.abs(q.astype(np.int32)) <= 127).all()


def test_odd_symmetry():
    g = np.random.Generator(np.random.PCG64(23))
    x = g.standard_normal((8, 1000), dtype=np.float32)
    q1, s1 = oracle.quant_absmax_i8(x)
    q2, s2 = oracle.quant_absmax_i8(-x)
    np.testing.assert_array_equal(q2.astype(np.int32), -q1.astype(np.int32))
    np.testing.assert_array_equal(s1, s2)


@pytest.mark.parametrize("j", [-6, -1, 1, 5])
def test_power_of_two_scaling_invariance(j):
    g = np.random.Generator(np.random.PCG64(24))
    x = g.standard_normal((8, 512), dtype=np.float32)
    q1, s1 = oracle.quant_absmax_i8(x)
    q2, s2 = oracle.quant_absmax_i8((x * np.float32(2.0 ** j)).astype(np.float32))
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(s2, (s1 * np.float32(2.0 ** -j)).astype(np.float32))


def test_integer_rows_are_fixed_points():
    # amax = 127 gives s = 1 exactly, so integer activations come back unchanged
    g = np.random.Generator(np.random.PCG64(25))
    x = g.integers(-127, 128, size=(4, 300)).astype(np.float32)
    x[:, 0] = 127
    x[1, 0] = -127
    q, s = oracle.quant_absmax_i8(x)
    assert (s == 1.0).all()
    np.testing.assert_array_equal(q, x.astype(np.int8))


def test_ties_round_to_even():
    x = np.array([[127.0, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5, 126.5]], dtype=np.float32)
    q, s = oracle.quant_absmax_i8(x)
    assert s[0] == 1.0
    assert q[0].tolist() == [127, 2, 4, -2, -4, 0, 0, 2, 126]


def test_zero_and_tiny_rows_use_the_floor():
    x = np.zeros((3, 64), dtype=np.float32)
    x[1, 5] = 5e-6           # below the 1e-5 floor
    x[2, 7] = -2e-5          # above it
    q, s = oracle.quant_absmax_i8(x)
    floor_s = np.float32(127.0) / np.float32(1e-5)
    assert s[0] == floor_s and s[1] == floor_s
    assert (q[0] == 0).all()
    assert q[1, 5] == np.clip(np.rint(np.float32(5e-6) * floor_s), -128, 127)
    assert q[2, 7] == -127


def test_bf16_input_equals_widened_fp32():
    g = np.random.Generator(np.random.PCG64(26))
    f = g.standard_normal((4, 2560), dtype=np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    widened = (bits.astype(np.uint32) << 16).view(np.float32)
    q1, s1 = oracle.quant_absmax_i8(bits, bf16=True)
    q2, s2 = oracle.quant_absmax_i8(widened)
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(s1, s2)
