"""Seeded synthetic inputs for the W2A8 ternary linear layer.

Shared by the tests, the benchmark and the smoke check; both the oracle side
and the GPU side are fed from here.  This module draws random numbers only:
it holds none of the layer's arithmetic (no quantisation, no packing, no
dot products, no rounding of results).  Values that must be bf16 (weight
scales, bf16 activations) are drawn directly on the bf16 grid by keeping the
top 16 bits of an fp32 draw.

Workloads (all shapes from the 2B-style model of the W2A8 page, "BitNet GPU
推理框架：从零构建 W2A8 的 2-bit 大模型 CUDA GEMV 内核", §一: dim 2560, ffn
6912, 20 heads / 5 KV heads, 30 layers; and its kernel table, §5.4 / §7.1):

  small      M=1, (2560, 2560)
  layer set  M=1, qkv (3840, 2560), o (2560, 2560), gate+up (13824, 2560), down (2560, 6912)
  large      M=1, (55296, 5120), (13824, 5120), (5120, 13824)
  batched    M in {16, 32, 64}, (13824, 2560)
  decode     30 layers x the layer set, bf16 activations, one graph
"""
from dataclasses import dataclass
from typing import List, Tuple

import numpy as np

BASE_SEED = 20261202

# Model width and MLP width of the pages' 2B configuration (dim 2560, intermediate 6912).
DIM = 2560
FFN = 6912
# (name, N, K, ws_num) of one transformer layer of the 2B-style model.
LAYER_SET: List[Tuple[str, int, int, int]] = [
    ("qkv", 3840, 2560, 1),
    ("o", 2560, 2560, 1),
    ("gate_up", 13824, 2560, 2),
    ("down", 2560, 6912, 1),
]
LARGE_SET: List[Tuple[str, int, int, int]] = [
    ("large_55296x5120", 55296, 5120, 1),
    ("large_13824x5120", 13824, 5120, 1),
    ("large_5120x13824", 5120, 13824, 1),
]
BATCHED_M = (16, 32, 64)
# Prompt lengths of the pages' end-to-end latency table ([W2A8] §7.2): the
# prompt-processing workload of the gate+up layer.
PREFILL_M = (64, 256, 512)
N_LAYERS = 30


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def seed_for(config: int, layer: int = 0, tensor: int = 0) -> int:
    return BASE_SEED + 1000 * config + 10 * layer + tensor


def ternary_uniform(g: np.random.Generator, N: int, K: int) -> np.ndarray:
    """Weights i.i.d. uniform over {-1, 0, +1}, int8, N x K (row n = output n)."""
    return g.integers(-1, 2, size=(N, K), dtype=np.int8)


def ternary_sparse(g: np.random.Generator, N: int, K: int) -> np.ndarray:
    """Weights with P(0) = 0.5, P(+1) = P(-1) = 0.25, int8, N x K."""
    u = g.integers(0, 4, size=(N, K), dtype=np.int8)      # 0,1,2,3 equally likely
    return np.where(u == 0, -1, np.where(u == 3, 1, 0)).astype(np.int8)


def int8_uniform(g: np.random.Generator, M: int, K: int, lo: int = -127, hi: int = 127) -> np.ndarray:
    """Activations i.i.d. uniform integers in [lo, hi], int8, M x K."""
    return g.integers(lo, hi + 1, size=(M, K), dtype=np.int8)


def normal_f32(g: np.random.Generator, M: int, K: int) -> np.ndarray:
    """x ~ N(0, 1), fp32, M x K."""
    return g.standard_normal(size=(M, K), dtype=np.float32)


def _top16(f: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(f, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def weights_bf16(g, N, K, sigma=0.02):
    """bf16 weight matrix (uint16 bit patterns): N(0, sigma^2) draws, fp32 cut to its top 16 bits."""
    v = (g.standard_normal((N, K)) * sigma).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def normal_bf16_bits(g: np.random.Generator, M: int, K: int) -> np.ndarray:
    """x ~ N(0, 1) on the bf16 grid (fp32 draw, top 16 bits kept), as uint16 bit patterns."""
    return _top16(normal_f32(g, M, K))


def ws_bits(g: np.random.Generator, ws_num: int) -> np.ndarray:
    """ws_num weight scales ~ U(0.5, 2) on the bf16 grid, as uint16 bit patterns."""
    return _top16(g.uniform(0.5, 2.0, size=(ws_num,)).astype(np.float32))


def act_scale(g: np.random.Generator, M: int) -> np.ndarray:
    """fp32 activation scales s = 127 / amax with amax ~ U(0.5, 4).

    Used where int8 activations are drawn directly: amax is then a free
    positive number, and s is an input of the layer.
    """
    amax = g.uniform(0.5, 4.0, size=(M,)).astype(np.float32)
    return (np.float32(127.0) / amax).astype(np.float32)


@dataclass
class Gemv:
    """One M x (N, K) instance of the layer with int8 activations given directly."""
    name: str
    M: int
    N: int
    K: int
    ws_num: int
    w: np.ndarray          # int8 N x K in {-1, 0, 1}
    xq: np.ndarray         # int8 M x K
    s: np.ndarray          # fp32 M
    ws: np.ndarray         # uint16 bf16 bits, ws_num


@dataclass
class GemvF:
    """One M x (N, K) instance with real-valued activations to be quantised."""
    name: str
    M: int
    N: int
    K: int
    ws_num: int
    w: np.ndarray          # int8 N x K
    x: np.ndarray          # fp32 M x K, or uint16 bf16 bits M x K
    x_is_bf16: bool
    ws: np.ndarray         # uint16 bf16 bits, ws_num


def make_int8_gemv(name, M, N, K, ws_num, seed, sparse=False) -> Gemv:
    g = rng(seed)
    w = ternary_sparse(g, N, K) if sparse else ternary_uniform(g, N, K)
    xq = int8_uniform(g, M, K)
    s = act_scale(g, M)
    ws = ws_bits(g, ws_num)
    return Gemv(name, M, N, K, ws_num, w, xq, s, ws)


def make_float_gemv(name, M, N, K, ws_num, seed, sparse=False, bf16=False) -> GemvF:
    g = rng(seed)
    w = ternary_sparse(g, N, K) if sparse else ternary_uniform(g, N, K)
    x = normal_bf16_bits(g, M, K) if bf16 else normal_f32(g, M, K)
    ws = ws_bits(g, ws_num)
    return GemvF(name, M, N, K, ws_num, w, x, bf16, ws)


def small() -> Gemv:
    """M=1, (2560, 2560): uniform ternary, uniform int8, one weight scale."""
    return make_int8_gemv("small_2560x2560", 1, 2560, 2560, 1, seed_for(1))


def layer_set() -> List[Gemv]:
    """M=1 per-layer shapes of the 2B-style model, uniform ternary, uniform int8."""
    return [make_int8_gemv(n, 1, N, K, wn, seed_for(2, 0, i))
            for i, (n, N, K, wn) in enumerate(LAYER_SET)]


def layer(name: str) -> Gemv:
    for i, (n, N, K, wn) in enumerate(LAYER_SET):
        if n == name:
            return make_int8_gemv(n, 1, N, K, wn, seed_for(2, 0, i))
    raise KeyError(name)


def large_set() -> List[GemvF]:
    """M=1 large shapes: sparse ternary weights, fp32 x ~ N(0, 1) to be quantised."""
    return [make_float_gemv(n, 1, N, K, wn, seed_for(3, 0, i), sparse=True)
            for i, (n, N, K, wn) in enumerate(LARGE_SET)]


def batched(M: int) -> GemvF:
    """M rows (BATCHED_M, PREFILL_M), (13824, 2560), ws_num=2: fp32 x ~ N(0, 1) to be
    quantised per row."""
    return make_float_gemv(f"batched_m{M}", M, 13824, 2560, 2, seed_for(4, 0, M))


def decode_step_nodes(n_layers: int = N_LAYERS) -> List[GemvF]:
    """The decode step: n_layers x the layer set, each node with its own bf16 x ~ N(0, 1)."""
    nodes = []
    for layer_i in range(n_layers):
        for i, (n, N, K, wn) in enumerate(LAYER_SET):
            nodes.append(make_float_gemv(f"L{layer_i}.{n}", 1, N, K, wn,
                                         seed_for(5, layer_i, i), bf16=True))
    return nodes


# --------------------------------------------------------------------------
# Chained decode step: one block's projections joined through the model's
# norms, MLP activation and residuals.  The attention itself is out of scope:
# each layer's attention output is a seeded bf16 N(0, 1) row, and the qkv
# projection's output is computed but feeds nothing.
# --------------------------------------------------------------------------

CHAIN_NORMS = ("attn", "attn_sub", "ffn", "ffn_sub")


@dataclass
class ChainLayer:
    w: dict          # projection name (LAYER_SET names) -> int8 ternary N x K
    ws: dict         # name -> bf16 bits [ws_num]
    ws_num: dict     # name -> int
    gamma: dict      # norm name (CHAIN_NORMS) -> bf16 bits [K of its input]
    attn_out: np.ndarray   # bf16 bits [dim]: the attention output this layer's o reads


def chained_layer(layer: int) -> ChainLayer:
    """Weights (uniform ternary), weight scales, RMSNorm weights ~ N(1, 0.1) and the
    attention output of one layer of the chained decode step."""
    w, ws, wn = {}, {}, {}
    for i, (name, N, K, ws_num) in enumerate(LAYER_SET):
        g = rng(seed_for(6, layer, i))
        w[name] = ternary_uniform(g, N, K)
        ws[name] = ws_bits(g, ws_num)
        wn[name] = ws_num
    g = rng(seed_for(6, layer, 7))
    dims = {"attn": DIM, "attn_sub": DIM, "ffn": DIM, "ffn_sub": FFN}
    gamma = {k: _top16((1.0 + 0.1 * g.standard_normal(dims[k])).astype(np.float32)) for k in CHAIN_NORMS}
    attn = normal_bf16_bits(g, 1, DIM).reshape(-1)
    return ChainLayer(w, ws, wn, gamma, attn)


def chained_h0() -> np.ndarray:
    """The residual stream entering the first layer: bf16 N(0, 1) bits [dim]."""
    return normal_bf16_bits(rng(seed_for(6, 99, 0)), 1, DIM).reshape(-1)
