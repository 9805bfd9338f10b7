"""GPU parity of the M = 1 layer (int8 GEMV and the fused bf16 path) against the oracle.

int32 accumulators bit-exact; bf16 outputs within 1 bf16 ulp of the oracle
(the kernels evaluate the same fp64 expression and round once, so they are
expected to agree exactly; the test states the 1-ulp bar and reports the
count of differing outputs).  Shapes: the pages' workloads (small, the 2B
layer set, the large set) plus ragged N and K, the smallest legal shape and
extreme values.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev, bf16_dev, host_bits, assert_bf16_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bit_gemv_bitlinear_amd as m
    return m


def run_i8(bl, w, xq, s, ws_bits, ws_num):
    import torch
    N, K = w.shape
    packed = bl.pack_ternary_weights(dev(w))
    acc = torch.empty((xq.shape[0], N), dtype=torch.int32, device="cuda")
    y = bl.bitlinear_i8xi2(dev(xq), packed, dev(s), bf16_dev(ws_bits), N, ws_num, acc=acc)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), host_bits(y)


def check_i8(bl, name, w, xq, s, ws_bits, ws_num):
    print(f"gemv_i8 {name} M={xq.shape[0]} N={w.shape[0]} K={w.shape[1]}", flush=True)
    acc, y = run_i8(bl, w, xq, s, ws_bits, ws_num)
    acc_o, y_o = oracle.bitlinear_i8(xq, w, s, ws_bits, ws_num)
    np.testing.assert_array_equal(acc, acc_o)
    ndiff = assert_bf16_close(y, y_o, max_ulp=1)
    assert ndiff == 0, f"{ndiff} outputs 1 ulp away (within the bar, but not expected)"


def test_small(bl):
    c = synth.small()
    check_i8(bl, c.name, c.w, c.xq, c.s, c.ws, c.ws_num)


@pytest.mark.parametrize("idx", range(len(synth.LAYER_SET)), ids=[n for n, *_ in synth.LAYER_SET])
def test_layer_set(bl, idx):
    c = synth.layer_set()[idx]
    check_i8(bl, c.name, c.w, c.xq, c.s, c.ws, c.ws_num)


@pytest.mark.parametrize("idx", range(len(synth.LARGE_SET)), ids=[n for n, *_ in synth.LARGE_SET])
def test_large_set_with_device_quantiser(bl, idx):
    import torch
    c = synth.large_set()[idx]
    print(f"large {c.name}: quantise on the device", flush=True)
    q, s = bl.quantize_act_absmax_i8(dev(c.x))
    torch.cuda.synchronize()
    qo, so = oracle.quant_absmax_i8(c.x)
    np.testing.assert_array_equal(q.cpu().numpy(), qo)
    np.testing.assert_array_equal(s.cpu().numpy(), so)
    check_i8(bl, c.name, c.w, qo, so, c.ws, c.ws_num)


# (33, 61440): the GEMV's largest K (16 wavefronts per band, 15 steps each);
# (20, 61456): one step past it, which M = 1 takes through the MFMA kernel
# (6912, 2560): 432 bands, runs of 5 over two wavefronts per band; (3200, 10240)
# and (2570, 13808): narrow with long rows, at most eight wavefronts per band
RAGGED = [(1, 16), (64, 16), (65, 80), (100, 208), (64 * 3 + 7, 64 * 5 + 48), (4097, 1040),
          (127, 6912 + 16), (640, 13824), (33, 61440), (20, 61456), (6912, 2560), (3200, 10240),
          (2570, 13808)]


@pytest.mark.parametrize("N,K", RAGGED)
def test_ragged_shapes(bl, N, K):
    c = synth.make_int8_gemv(f"ragged_{N}x{K}", 1, N, K, 1, synth.seed_for(9, 0, N % 997 + K % 13))
    check_i8(bl, c.name, c.w, c.xq, c.s, c.ws, c.ws_num)


def test_segmented_weight_scales(bl):
    g = synth.rng(77)
    N, K = 64 * 6, 256
    w = synth.ternary_uniform(g, N, K)
    xq = synth.int8_uniform(g, 1, K)
    s = synth.act_scale(g, 1)
    for ws_num in (1, 2, 3, 6):
        check_i8(bl, f"ws_num={ws_num}", w, xq, s, synth.ws_bits(g, ws_num), ws_num)


def test_extreme_values(bl):
    N, K = 192, 6912
    g = synth.rng(88)
    w = np.empty((N, K), dtype=np.int8)
    w[:64] = 1
    w[64:128] = -1
    w[128:] = synth.ternary_uniform(g, 64, K)
    ws = synth.ws_bits(g, 1)
    for label, xval in (("all_-128", -128), ("all_127", 127)):
        xq = np.full((1, K), xval, dtype=np.int8)
        check_i8(bl, label, w, xq, np.array([1.0], np.float32), ws, 1)
    xq = np.where(g.integers(0, 2, size=(1, K)) == 0, -128, 127).astype(np.int8)
    check_i8(bl, "mixed_extremes", w, xq, np.array([127.0 / 3.0], np.float32), ws, 1)
    check_i8(bl, "zero_activations", w, np.zeros((1, K), np.int8),
             np.array([127.0 / 1e-5], np.float32), ws, 1)


def test_output_buffer_fully_written(bl):
    # poison the outputs first: every row of a ragged shape must be written
    import torch
    N, K = 200, 144
    c = synth.make_int8_gemv("poison", 1, N, K, 1, 4242)
    packed = bl.pack_ternary_weights(dev(c.w))
    y = torch.full((1, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    acc = torch.full((1, N), -7, dtype=torch.int32, device="cuda")
    bl.bitlinear_i8xi2(dev(c.xq), packed, dev(c.s), bf16_dev(c.ws), N, 1, y=y, acc=acc)
    torch.cuda.synchronize()
    acc_o, y_o = oracle.bitlinear_i8(c.xq, c.w, c.s, c.ws, 1)
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_o)
    np.testing.assert_array_equal(host_bits(y), y_o)


# ---------------------------------------------------------------------------
# fused bf16 path (M = 1)
# ---------------------------------------------------------------------------

FUSED = [("qkv", 3840, 2560, 1), ("o", 2560, 2560, 1), ("gate_up", 13824, 2560, 2),
         ("down", 2560, 6912, 1), ("ragged", 100, 208, 1), ("k13824", 5120, 13824, 1),
         ("tiny", 1, 16, 1), ("kmax", 48, 61440, 1), ("medium", 6912, 2560, 1),
         ("narrow_long", 3200, 10240, 1)]


@pytest.mark.parametrize("name,N,K,ws_num", FUSED)
def test_fused_bf16(bl, name, N, K, ws_num):
    import torch
    print(f"fused_bf16 {name} N={N} K={K}", flush=True)
    c = synth.make_float_gemv(name, 1, N, K, ws_num, synth.seed_for(7, 0, N % 101), bf16=True)
    packed = bl.pack_ternary_weights(dev(c.w))
    q = torch.empty((1, K), dtype=torch.int8, device="cuda")
    s = torch.empty((1,), dtype=torch.float32, device="cuda")
    acc = torch.empty((1, N), dtype=torch.int32, device="cuda")
    y = bl.bitlinear_bf16_i8xi2(bf16_dev(c.x), packed, bf16_dev(c.ws), N, ws_num,
                                q_out=q, s_out=s, acc=acc)
    torch.cuda.synchronize()
    qo, so, acc_o, y_o = oracle.bitlinear_bf16(c.x, c.w, c.ws, ws_num)
    np.testing.assert_array_equal(q.cpu().numpy(), qo)
    np.testing.assert_array_equal(s.cpu().numpy(), so)
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_o)
    assert assert_bf16_close(host_bits(y), y_o, max_ulp=1) == 0


@pytest.mark.parametrize("N,K", [(640, 2560), (13824, 2560), (2560, 6912)])
def test_fused_product_ties(bl, N, K):
    # activations whose products x * s sit on fp32 .5 ties (see quant_cases):
    # the in-kernel quantiser must round twice, as the definition does
    import torch
    from quant_cases import tie_rows
    print(f"fused product ties N={N} K={K}", flush=True)
    xb = tie_rows(1, K, seed=N + K)
    c = synth.make_int8_gemv("ties", 1, N, K, 1, synth.seed_for(8, 0, N % 101))
    packed = bl.pack_ternary_weights(dev(c.w))
    q = torch.empty((1, K), dtype=torch.int8, device="cuda")
    s = torch.empty((1,), dtype=torch.float32, device="cuda")
    acc = torch.empty((1, N), dtype=torch.int32, device="cuda")
    y = bl.bitlinear_bf16_i8xi2(bf16_dev(xb), packed, bf16_dev(c.ws), N, 1, q_out=q, s_out=s,
                                acc=acc)
    torch.cuda.synchronize()
    qo, so, acc_o, y_o = oracle.bitlinear_bf16(xb, c.w, c.ws, 1)
    np.testing.assert_array_equal(q.cpu().numpy(), qo)
    np.testing.assert_array_equal(s.cpu().numpy(), so)
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_o)
    assert assert_bf16_close(host_bits(y), y_o, max_ulp=1) == 0


def test_fused_without_optional_outputs(bl):
    import torch
    print("fused_bf16 no optional outputs", flush=True)
    c = synth.make_float_gemv("plain", 1, 2560, 2560, 1, 31337, bf16=True)
    packed = bl.pack_ternary_weights(dev(c.w))
    y = bl.bitlinear_bf16_i8xi2(bf16_dev(c.x), packed, bf16_dev(c.ws), 2560, 1)
    torch.cuda.synchronize()
    _, _, _, y_o = oracle.bitlinear_bf16(c.x, c.w, c.ws, 1)
    np.testing.assert_array_equal(host_bits(y), y_o)


def _rows_with_sums(targets, K):
    """Ternary rows whose dot product with x (x[k] = 2^(k % 7), groups of 7) equals targets[n]."""
    x = np.zeros((1, K), dtype=np.int8)
    groups = K // 7
    for g in range(groups):
        for b in range(7):
            x[0, 7 * g + b] = 1 << b
    w = np.zeros((len(targets), K), dtype=np.int8)
    for n, t in enumerate(targets):
        sign = 1 if t >= 0 else -1
        rem = abs(int(t))
        for g in range(groups):
            c = min(rem, 127)
            rem -= c
            for b in range(7):
                if (c >> b) & 1:
                    w[n, 7 * g + b] = sign
        assert rem == 0
    return w, x


@pytest.mark.parametrize("s_val", [3.0, 1.0, 7.0, 127.0 / 3.3])
def test_epilogue_rounding_boundaries(bl, s_val):
    # outputs that land exactly on (or next to) bf16 midpoints: the division-free
    # epilogue must fall back to the exact quotient there (e.g. 777 / 3 = 259 -> 260)
    K = 64 * 4
    base = [257, 259, 261, 383, 385, 511, 513, 515, 1025, 1027, 2047, 2049]
    targets = []
    for t in base:
        for d in (-1, 0, 1):
            v = int(round(t * s_val)) + d
            if abs(v) <= (K // 7) * 127:
                targets += [v, -v]
    targets = targets[:128] + [0] * max(0, 128 - len(targets))
    w, x = _rows_with_sums(targets, K)
    check_i8(bl, f"midpoints_s{s_val:.4f}", w, x, np.array([s_val], np.float32),
             np.array([0x3F80], np.uint16), 1)


@pytest.mark.parametrize("s_val", [1e-36, 3e38, 1e37])
def test_epilogue_outside_normal_range(bl, s_val):
    # outputs that overflow to +-inf (s = 1e-36) or fall into bf16 subnormals (s >= 1e37)
    K = 64 * 4
    t = [0, 1, 2, 3, 5, 100, 339, 340, 341, 500, 1000, 2000, 4000]
    targets = t + [-v for v in t if v]
    w, x = _rows_with_sums(targets, K)
    check_i8(bl, f"extreme_s{s_val:g}", w, x, np.array([s_val], np.float32),
             np.array([0x3F80], np.uint16), 1)
