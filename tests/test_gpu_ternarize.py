"""GPU parity of the weight ternariser + packer ([W2A8] §4.2, §5.2) against the oracle.

The device packs the ternary matrix directly; the oracle's unpacker reads
those bytes back, and the result must equal the oracle's ternary matrix
element for element, with the three bf16 scales (ws, s, mean) bit-exact.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import bf16_dev, host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bit_gemv_bitlinear_amd as m
    return m


def check(bl, name, w_bits, workspace=None):
    import torch
    N, K = w_bits.shape
    print(f"ternarize {name} N={N} K={K}", flush=True)
    packed, scales = bl.ternarize_weights_absmean(bf16_dev(w_bits), workspace=workspace)
    torch.cuda.synchronize()
    q, mean, s, ws = oracle.ternarize_absmean(w_bits)
    got = host_bits(scales)
    assert (int(got[0]), int(got[1]), int(got[2])) == (ws, s, mean), (got, (ws, s, mean))
    np.testing.assert_array_equal(oracle.unpack_tiles(packed.cpu().numpy(), N, K), q)
    return q


def f32_to_bits(v):
    v = np.asarray(v, dtype=np.float32)
    assert np.all((v.view(np.uint32) & 0xFFFF) == 0)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("N,K", [(64, 256), (70, 272), (1, 16), (2560, 2560), (13824, 2560),
                                 (2560, 6912), (3840, 2560)])
def test_random_weights(bl, N, K):
    g = synth.rng(synth.seed_for(9, 0, N % 97 + K % 89))
    check(bl, "normal", synth.weights_bf16(g, N, K))


def test_zero_matrix_and_tiny_weights(bl):
    q = check(bl, "zero", np.zeros((32, 64), dtype=np.uint16))
    assert not q.any()
    g = synth.rng(41)
    tiny = synth.weights_bf16(g, 32, 64, sigma=1e-7)       # mean below the 1e-5 floor
    check(bl, "tiny", tiny)


@pytest.mark.parametrize("N,K", [(96, 512), (13824, 2560)])
def test_wide_range_subnormals_and_outlier(bl, N, K):
    # magnitudes over 170 binades: most threads' spans exceed the fp64 fast
    # path's bound and take the per-weight bins, some do not; at 13824 x 2560
    # the mean pass runs 24 chunks per thread (a bound of 37 binades), at 96 x
    # 512 16 (38)
    g = synth.rng(43 + N % 7)
    e = g.integers(-140, 30, size=(N, K)).astype(np.float64)
    v = (g.standard_normal((N, K)) * np.exp2(e)).astype(np.float32)
    check(bl, "wide range", (v.view(np.uint32) >> 16).astype(np.uint16))
    w = synth.weights_bf16(g, N, K)
    w[5, 7] = np.array([1e30], dtype=np.float32).view(np.uint32)[0] >> 16   # ~1e30 in bf16
    w[N - 1, K - 1] = np.array([3e-40], dtype=np.float32).view(np.uint32)[0] >> 16   # subnormal
    check(bl, "outlier", w)


def test_mean_on_a_tie_and_just_above_it(bl):
    # 256 entries summing to 257 and 256 zeros: the exact mean 0.5 * (1 + 2^-8)
    # is a bf16 tie and rounds to even 0.5; one zero raised to the smallest
    # subnormal puts the mean just above the tie, which must round up.
    v = np.zeros(512, dtype=np.float32)
    v[:255] = 1.0
    v[255] = 2.0
    v[::2], v[1::2] = v[:256].copy(), v[256:].copy()      # interleave with the zeros
    w = f32_to_bits(v).reshape(16, 32)
    _, mean, _, _ = oracle.ternarize_absmean(w)
    assert mean == 0x3F00
    check(bl, "tie", w)
    w2 = w.copy()
    w2[0, 1] = 0x0001                                      # 2^-133
    _, mean2, _, _ = oracle.ternarize_absmean(w2)
    assert mean2 == 0x3F01
    check(bl, "above the tie", w2)


def test_products_on_half_ties(bl):
    # mean exactly 0.25 (s = 4): w*s in {+-0.5, +-1.5, +-0.75, ...}
    base = np.array([0.125, 0.375, -0.125, -0.375, 0.1875, 0.3125, 0.0625, 0.4375], dtype=np.float32)
    v = np.tile(base, (16, 8))
    check(bl, "half ties", f32_to_bits(v))


def test_workspace_reuse(bl):
    import torch
    ws_buf = torch.full((bl.TERNARIZE_WORKSPACE_BYTES,), 0xAB, dtype=torch.uint8, device="cuda")
    g = synth.rng(47)
    for N, K in ((128, 512), (64, 256)):
        check(bl, "reused workspace", synth.weights_bf16(g, N, K), workspace=ws_buf)
