"""Exact-rational references for the bf16 glue of a decode step, written from
the formats' definitions (test infrastructure; no oracle code).

bf16 and fp32 rounding (nearest, ties to even) are spelled out on Python
Fractions; RMSNorm's rounding is decided by comparing squares, so no square
root is approximated.
"""
import math
import struct
from fractions import Fraction

import numpy as np

EPS = Fraction(float(np.float32(1e-5)))


def bits_to_fraction(b):
    f = struct.unpack("<f", struct.pack("<I", int(b) << 16))[0]
    return Fraction(f)


def bf16_bits_of_exact(v: Fraction) -> int:
    """Round a rational to bf16 (nearest, ties to even) from the format's definition."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = -v if v < 0 else v
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    spacing = Fraction(2) ** (max(e, -126) - 7)
    q = a / spacing
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * spacing
    if r >= Fraction(2) ** 128:
        return sign | 0x7F80
    u = struct.unpack("<I", struct.pack("<f", float(r)))[0]
    assert u & 0xFFFF == 0
    return sign | (u >> 16)


def rmsnorm_exact(x_bits, g_bits, eps=EPS):
    """bf16 of x*g / sqrt(sum(x^2)/K + eps), decided exactly (squares compared as rationals)."""
    xs = [bits_to_fraction(b) for b in x_bits]
    gs = [bits_to_fraction(b) for b in g_bits]
    D = sum(v * v for v in xs) / len(xs) + eps
    out = []
    for xv, gv, xb, gb in zip(xs, gs, x_bits, g_bits):
        num = xv * gv
        if num == 0:
            # IEEE product of zeros: sign is the exclusive or of the signs
            out.append(0x8000 if ((int(xb) ^ int(gb)) & 0x8000) else 0)
            continue
        sign = 0x8000 if num < 0 else 0
        a = abs(num)
        approx = float(a) / math.sqrt(float(D))
        c = bf16_bits_of_exact(Fraction(approx)) & 0x7FFF
        # the exact value a/sqrt(D) against the midpoints around candidates c-1, c, c+1
        best = None
        for cand in (c - 1, c, c + 1):
            if cand < 0 or cand >= 0x7F80:
                continue
            lo = bits_to_fraction(cand - 1) if cand > 0 else Fraction(0)
            hi = bits_to_fraction(cand + 1)
            cv = bits_to_fraction(cand)
            m_lo = (lo + cv) / 2
            m_hi = (cv + hi) / 2
            # m_lo <= a/sqrt(D) <= m_hi  <=>  m_lo^2 D <= a^2 <= m_hi^2 D (all positive)
            a2 = a * a
            below = a2 < m_lo * m_lo * D
            above = a2 > m_hi * m_hi * D
            if below or above:
                continue
            if a2 == m_lo * m_lo * D and cand % 2 == 1:
                continue
            if a2 == m_hi * m_hi * D and cand % 2 == 1:
                continue
            best = cand
            break
        assert best is not None
        out.append(sign | best)
    return np.array(out, dtype=np.uint16)


def round_binary(v: Fraction, p: int, emin: int, emax: int):
    """v rounded to the binary format with p significant bits, least normal
    exponent emin and largest exponent emax (nearest, ties to even); None for
    an overflow to infinity."""
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e, emin) - (p - 1)
    n = round(a / Fraction(2) ** q)          # Fraction.__round__: half to even
    r = n * Fraction(2) ** q
    if r >= Fraction(2) ** (emax + 1):
        return None
    return r if v > 0 else -r


def r32(v):
    return round_binary(v, 24, -126, 127)


def r64(v):
    return round_binary(v, 53, -1022, 1023)


def bf16_bits(v: Fraction) -> int:
    """bf16 encoding of v rounded to bf16 (finite results only in these cases)."""
    r = round_binary(v, 8, -126, 127)
    assert r is not None
    if r == 0:
        return 0
    sign = 0x8000 if r < 0 else 0
    a = abs(r)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    if e < -126:                              # subnormal: multiple of 2^-133
        return sign | int(a / Fraction(2) ** -133)
    mant = int(a / Fraction(2) ** (e - 7)) - 128
    return sign | ((e + 127) << 7) | mant
