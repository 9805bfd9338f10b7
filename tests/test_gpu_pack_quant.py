"""GPU parity of the weight packer and the activation quantiser against the oracle.

Packer: the device bytes must decode (oracle.unpack_tiles, written from the
layout's bit-level definition) to exactly the input matrix, padding included,
and equal the host twin byte for byte.  Quantiser: int8 values and fp32
scales bit-exact against oracle.quant_absmax_i8 (W2A8 page §六 item 3).
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


@pytest.mark.parametrize("N,K", [(64, 64), (13824, 2560), (2560, 6912), (1, 16), (70, 80),
                                 (4097, 1040), (130, 200), (3, 1)])
def test_pack_matches_definition(bl, N, K):
    import torch
    print(f"pack N={N} K={K}", flush=True)
    w = synth.ternary_uniform(synth.rng(N + 7 * K), N, K)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    packed = bl.pack_ternary_weights(dev(w), n_invalid=bad)
    torch.cuda.synchronize()
    p = packed.cpu().numpy()
    assert int(bad.item()) == 0
    np.testing.assert_array_equal(oracle.unpack_tiles(p, N, K), w)
    host, nbad = bl.bl_pack_ternary_host(w)
    assert nbad == 0
    np.testing.assert_array_equal(p, host)


def test_pack_unaligned_source_and_invalid_count(bl):
    import torch
    print("pack unaligned source", flush=True)
    N, K = 100, 96
    w = synth.ternary_sparse(synth.rng(5), N, K)
    w[7, 9] = 5
    w[99, 95] = -2
    buf = torch.zeros(N * K + 1, dtype=torch.int8, device="cuda")
    buf[1:].copy_(dev(w).reshape(-1))          # 1-byte offset: the byte-wise path
    src = buf[1:].view(N, K)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    packed = bl.pack_ternary_weights(src, n_invalid=bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == 2
    host, nbad = bl.bl_pack_ternary_host(w)
    assert nbad == 2
    np.testing.assert_array_equal(packed.cpu().numpy(), host)


def test_pack_aligned_source_invalid_values(bl):
    # the 16-byte path: codes four weights at a time and a byte-parallel count
    # of the weights outside {-1, 0, 1}; rows 3 and 40 hold every int8 value
    # once (253 invalid each), and a word with one invalid weight among valid
    # ones, all checked against the host twin byte for byte
    import torch
    print("pack aligned source, invalid values", flush=True)
    N, K = 64, 256
    w = synth.ternary_uniform(synth.rng(6), N, K)
    w[3] = np.arange(-128, 128, dtype=np.int8)
    w[40] = np.arange(127, -129, -1).astype(np.int8)
    w[10, 17] = 2
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    packed = bl.pack_ternary_weights(dev(w), n_invalid=bad)
    torch.cuda.synchronize()
    host, nbad = bl.bl_pack_ternary_host(w)
    assert nbad == 2 * 253 + 1
    assert int(bad.item()) == nbad
    np.testing.assert_array_equal(packed.cpu().numpy(), host)


def _quant_cases():
    g = synth.rng(99)
    cases = []
    x = synth.normal_f32(g, 16, 2560)
    x[1] = 0.0                                   # zero row -> the 1e-5 floor
    x[2] *= 1e-7                                 # tiny row, below the floor
    x[3] *= 3e4
    x[4, :] = np.float32(0.5)                    # all ties after scaling by 254
    x[4, 0] = np.float32(1.0)
    x[5, :] = np.arange(2560, dtype=np.float32) % 255 - 127   # integers, s = 1
    cases.append(("mixed_2560", x))
    cases.append(("ragged_k80", synth.normal_f32(g, 3, 80)))
    cases.append(("k6912", synth.normal_f32(g, 2, 6912)))
    cases.append(("k13824_m64", synth.normal_f32(g, 64, 13824)))
    cases.append(("k16", synth.normal_f32(g, 5, 16)))
    return cases


@pytest.mark.parametrize("name,x", _quant_cases(), ids=lambda v: v if isinstance(v, str) else "")
def test_quant_fp32_bit_exact(bl, name, x):
    import torch
    print(f"quant fp32 {name} {x.shape}", flush=True)
    q, s = bl.quantize_act_absmax_i8(dev(x))
    torch.cuda.synchronize()
    qo, so = oracle.quant_absmax_i8(x)
    np.testing.assert_array_equal(q.cpu().numpy(), qo)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))


@pytest.mark.parametrize("M,K", [(1, 2560), (7, 6912), (3, 80), (64, 2560)])
def test_quant_bf16_bit_exact(bl, M, K):
    import torch
    print(f"quant bf16 M={M} K={K}", flush=True)
    xb = synth.normal_bf16_bits(synth.rng(M * K), M, K)
    q, s = bl.quantize_act_absmax_i8(bf16_dev(xb))
    torch.cuda.synchronize()
    qo, so = oracle.quant_absmax_i8(xb, bf16=True)
    np.testing.assert_array_equal(q.cpu().numpy(), qo)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))


def test_quant_many_random_scales_bit_exact(bl):
    # many rows with amax spread over 20 binades: exercises the IEEE division 127 / amax
    import torch
    print("quant many scales", flush=True)
    g = synth.rng(1234)
    M, K = 4096, 64
    x = synth.normal_f32(g, M, K) * (2.0 ** g.integers(-10, 10, size=(M, 1))).astype(np.float32)
    x = x.astype(np.float32)
    q, s = bl.quantize_act_absmax_i8(dev(x))
    torch.cuda.synchronize()
    qo, so = oracle.quant_absmax_i8(x)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
    np.testing.assert_array_equal(q.cpu().numpy(), qo)


def test_quant_bf16_product_ties(bl):
    # x * s lands on an fp32 .5 tie that the exact product misses: the two
    # roundings of the definition must not be fused into one
    import torch
    from quant_cases import tie_rows
    print("quant bf16 product ties", flush=True)
    xb = tie_rows(16, 2560, seed=5)
    q, s = bl.quantize_act_absmax_i8(bf16_dev(xb))
    torch.cuda.synchronize()
    qo, so = oracle.quant_absmax_i8(xb, bf16=True)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
    np.testing.assert_array_equal(q.cpu().numpy(), qo)
