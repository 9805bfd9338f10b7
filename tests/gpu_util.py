"""Helpers for the GPU tests: numpy <-> device tensors and bf16 comparisons.

Marshalling only; the expected values always come from the oracle.
"""
import numpy as np


def dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def bf16_dev(bits):
    """uint16 bf16 bit patterns (numpy) -> device bfloat16 tensor."""
    import torch
    return dev(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16), torch.bfloat16)


def host_bits(t):
    """device bfloat16 tensor -> numpy uint16 bit patterns."""
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_ulp_distance(a_bits, b_bits):
    """|a - b| in units of bf16 spacing, on the monotone integer line of bf16 patterns."""
    def ordered(b):
        b = np.asarray(b, dtype=np.int64)
        mag = b & 0x7FFF
        return np.where(b & 0x8000, -mag, mag)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def assert_bf16_close(got_bits, want_bits, max_ulp=1):
    d = bf16_ulp_distance(got_bits, want_bits)
    worst = int(d.max()) if d.size else 0
    assert worst <= max_ulp, f"bf16 mismatch: worst {worst} ulp at {np.unravel_index(d.argmax(), d.shape)}"
    return int((d != 0).sum())
