"""Activation rows whose quantisation separates two roundings from one.

A row holds its absmax A and then bf16 values x with |x| < A for which the
fp32 product x * s (s = fl32(127 / A)) lands exactly on a half-integer while
the exact product does not.  Quantising such x rounds the product twice (to
fp32, then to an integer, ties to even); an implementation that fuses the two
steps sees the exact product and can land one integer away.  The expected
values always come from the oracle; this module only finds the inputs.
"""
import numpy as np


def _bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def tie_values(a_bits):
    """bf16 patterns x with |x| < A whose fp32 product with 127/A is a misleading .5 tie."""
    A = _bf16_to_f32(np.array([a_bits], dtype=np.uint16))[0]
    s = np.float32(127.0) / np.float32(A)
    mags = np.arange(0, int(a_bits) & 0x7FFF, dtype=np.uint32)
    pats = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
    x = _bf16_to_f32(pats)
    p32 = (x * s).astype(np.float32)
    p64 = x.astype(np.float64) * np.float64(s)
    frac = p32.astype(np.float64) - np.floor(p32.astype(np.float64))
    return pats[(frac == 0.5) & (p64 != p32.astype(np.float64))]


def tie_rows(M, K, seed):
    """M x K bf16 patterns: each row is its absmax followed by tie values (and its negation)."""
    g = np.random.default_rng(seed)
    rows = []
    e = 0
    while len(rows) < M:
        a_bits = np.uint16(((127 + (e % 9) - 4) << 7) | int(g.integers(1, 128)))
        e += 1
        ties = tie_values(a_bits)
        if ties.size == 0:
            continue
        row = g.choice(ties, size=K)
        row[0] = a_bits
        row[K // 2] = a_bits | 0x8000
        rows.append(row)
    return np.stack(rows).astype(np.uint16)
