"""CPU oracle for the BitNet b1.58 W2A8 ternary linear layer.

TEST INFRASTRUCTURE ONLY.  The test-suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package; the product
package (``bit_gemv_bitlinear_amd``) never does, and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C loops); this module only
marshals numpy arrays into it.  Every function states the page section it
follows.  Source page: "BitNet GPU 推理框架：从零构建 W2A8 的 2-bit 大模型
CUDA GEMV 内核" (blog.gitcode.com), cited below as [W2A8].

Pinned by tests/test_oracle_*.py against brute force, closed forms,
invariants and the values the page prints (tests/golden/).
"""
import ctypes
import os

import numpy as np

from . import pages_layout  # noqa: F401  (the page's own layout, a reading test)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

OK, ERR_ARG, ERR_RANGE, ERR_CODE, ERR_PAD = 0, -1, -2, -3, -4


class OracleError(RuntimeError):
    pass


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_bf16_rne.argtypes = [ctypes.c_double]
    lib.oracle_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_bf16_rne_array.argtypes = [P, P, ctypes.c_size_t]
    lib.oracle_bf16_rne_array.restype = None
    lib.oracle_quant_absmax_i8_f32.argtypes = [P, I, I, P, P]
    lib.oracle_quant_absmax_i8_bf16.argtypes = [P, I, I, P, P]
    lib.oracle_packed_bytes.argtypes = [I, I]
    lib.oracle_packed_bytes.restype = ctypes.c_size_t
    lib.oracle_unpack_tiles.argtypes = [P, I, I, P, P]
    lib.oracle_gemm_i32.argtypes = [P, P, I, I, I, P]
    lib.oracle_epilogue_bf16.argtypes = [P, P, P, I, I, I, P]
    lib.oracle_bitlinear_i8.argtypes = [P, P, P, P, I, I, I, I, P, P]
    lib.oracle_bitlinear_bf16.argtypes = [P, P, P, I, I, I, I, P, P, P, P]
    lib.oracle_absmean_scales.argtypes = [ctypes.c_uint16, P, P]
    lib.oracle_ternary_from_scale.argtypes = [P, ctypes.c_size_t, ctypes.c_uint16, P]
    lib.oracle_rmsnorm_bf16.argtypes = [P, P, I, ctypes.c_float, P]
    lib.oracle_relu2_glu_bf16.argtypes = [P, P, I, P]
    lib.oracle_add_bf16.argtypes = [P, P, I, P]
    for name in ("oracle_rmsnorm_bf16", "oracle_relu2_glu_bf16", "oracle_add_bf16",
                 "oracle_absmean_scales", "oracle_ternary_from_scale", "oracle_quant_absmax_i8_f32", "oracle_quant_absmax_i8_bf16", "oracle_unpack_tiles",
                 "oracle_gemm_i32", "oracle_epilogue_bf16", "oracle_bitlinear_i8",
                 "oracle_bitlinear_bf16"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != OK:
        raise OracleError(f"{what} failed with code {rc}")


# --------------------------------------------------------------------------
# bf16
# --------------------------------------------------------------------------

def bf16_rne(v) -> np.ndarray:
    """Round fp64 values to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().oracle_bf16_rne_array(_ptr(v), _ptr(out), v.size)
    return out


def bf16_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    b = _c(bits, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# Activation quantisation  ([W2A8] §六 item 3)
# --------------------------------------------------------------------------

def quant_absmax_i8(x: np.ndarray, bf16: bool = False):
    """Per-row absmax int8 quantisation.

    s = 127 / max(max|x|, 1e-5) in fp32; q = clamp(round_half_even(x * s), -128, 127).
    ``x`` is fp32 (M x K), or bf16 bit patterns (uint16, M x K) when ``bf16``.
    Returns (q int8 M x K, s fp32 M).
    """
    x = np.atleast_2d(x)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty((M,), dtype=np.float32)
    lib = _load()
    if bf16:
        xc = _c(x, np.uint16)
        rc = lib.oracle_quant_absmax_i8_bf16(_ptr(xc), M, K, _ptr(q), _ptr(s))
    else:
        xc = _c(x, np.float32)
        rc = lib.oracle_quant_absmax_i8_f32(_ptr(xc), M, K, _ptr(q), _ptr(s))
    _check(rc, "quant_absmax_i8")
    return q, s


# --------------------------------------------------------------------------
# Packed weights
# --------------------------------------------------------------------------

def packed_bytes(N: int, K: int) -> int:
    """Bytes of the tiled packed layout: ceil(N/16)*ceil(K/256)*1024."""
    return int(_load().oracle_packed_bytes(N, K))


def unpack_tiles(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """Decode packed ternary weights (layout spelled out in oracle.c) to int8 N x K.

    Raises OracleError if a real position holds code 0 or a padding position
    holds a non-zero code.
    """
    p = _c(packed, np.uint8).reshape(-1)
    if p.size != packed_bytes(N, K):
        raise OracleError(f"packed buffer has {p.size} bytes, expected {packed_bytes(N, K)}")
    w = np.empty((N, K), dtype=np.int8)
    bad = ctypes.c_int64(-1)
    rc = _load().oracle_unpack_tiles(_ptr(p), N, K, _ptr(w), ctypes.byref(bad))
    if rc == ERR_CODE:
        raise OracleError(f"code 0 at real position (flat index {bad.value})")
    if rc == ERR_PAD:
        raise OracleError(f"non-zero code in padding (byte {bad.value})")
    _check(rc, "unpack_tiles")
    return w


# --------------------------------------------------------------------------
# int32 dot products  ([W2A8] §三 item 2, §5.3)
# --------------------------------------------------------------------------

def gemm_i32(xq: np.ndarray, w: np.ndarray) -> np.ndarray:
    """acc[m][n] = sum_k xq[m][k] * w[n][k], exact, in int32 (error if it overflows)."""
    xq = _c(np.atleast_2d(xq), np.int8)
    w = _c(w, np.int8)
    M, K = xq.shape
    N, K2 = w.shape
    if K != K2:
        raise OracleError("K mismatch")
    acc = np.empty((M, N), dtype=np.int32)
    _check(_load().oracle_gemm_i32(_ptr(xq), _ptr(w), M, N, K, _ptr(acc)), "gemm_i32")
    return acc


# --------------------------------------------------------------------------
# Epilogue  ([W2A8] §5.3)
# --------------------------------------------------------------------------

def epilogue_bf16(acc: np.ndarray, s: np.ndarray, ws_bits: np.ndarray, ws_num: int) -> np.ndarray:
    """y = bf16_rne(acc * ws[n // (N // ws_num)] / s[m]) in fp64; returns uint16 bits."""
    acc = _c(np.atleast_2d(acc), np.int32)
    M, N = acc.shape
    s = _c(s, np.float32).reshape(-1)
    ws_bits = _c(ws_bits, np.uint16).reshape(-1)
    if s.size != M or ws_bits.size < ws_num:
        raise OracleError("scale sizes")
    y = np.empty((M, N), dtype=np.uint16)
    _check(_load().oracle_epilogue_bf16(_ptr(acc), _ptr(s), _ptr(ws_bits), ws_num, M, N, _ptr(y)),
           "epilogue_bf16")
    return y


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------

def bitlinear_i8(xq, w, s, ws_bits, ws_num):
    """int8 activations in -> (acc int32 M x N, y bf16 bits M x N)."""
    xq = _c(np.atleast_2d(xq), np.int8)
    w = _c(w, np.int8)
    M, K = xq.shape
    N = w.shape[0]
    s = _c(s, np.float32).reshape(-1)
    ws_bits = _c(ws_bits, np.uint16).reshape(-1)
    acc = np.empty((M, N), dtype=np.int32)
    y = np.empty((M, N), dtype=np.uint16)
    _check(_load().oracle_bitlinear_i8(_ptr(xq), _ptr(w), _ptr(s), _ptr(ws_bits), ws_num, M, N, K,
                                       _ptr(acc), _ptr(y)), "bitlinear_i8")
    return acc, y


def bitlinear_bf16(x_bits, w, ws_bits, ws_num):
    """bf16 activations in (bit patterns) -> (q, s, acc, y): quantise, then the int8 layer."""
    x_bits = _c(np.atleast_2d(x_bits), np.uint16)
    w = _c(w, np.int8)
    M, K = x_bits.shape
    N = w.shape[0]
    ws_bits = _c(ws_bits, np.uint16).reshape(-1)
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty((M,), dtype=np.float32)
    acc = np.empty((M, N), dtype=np.int32)
    y = np.empty((M, N), dtype=np.uint16)
    _check(_load().oracle_bitlinear_bf16(_ptr(x_bits), _ptr(w), _ptr(ws_bits), ws_num, M, N, K,
                                         _ptr(q), _ptr(s), _ptr(acc), _ptr(y)), "bitlinear_bf16")
    return q, s, acc, y


def decode_step(nodes):
    """A decode step: each node is (x_bits 1 x K, w N x K, ws_bits, ws_num), run in order.

    Returns the list of (q, s, acc, y) per node, in node order.
    """
    return [bitlinear_bf16(x, w, ws, wn) for (x, w, ws, wn) in nodes]


# --------------------------------------------------------------------------
# Weight ternarisation by the mean absolute value  ([W2A8] §4.2)
# --------------------------------------------------------------------------

def bf16_rne_ratio(num: int, den: int) -> int:
    """bf16 bits of num/den (num >= 0, den > 0) rounded to nearest, ties to even.

    Exact integer arithmetic from the format's definition: around a value
    whose leading bit is 2^E the spacing is 2^(E-7) (normal, E >= -126) or
    2^-133 (below); the value divided by the spacing is rounded to an integer
    r, and the encoding of r * 2^u is ((u + 133) << 7) + r, which carries into
    the exponent when r reaches 256 and is +inf (0x7F80) from 2^128 on.
    """
    if num < 0 or den <= 0:
        raise OracleError("bf16_rne_ratio needs num >= 0, den > 0")
    if num == 0:
        return 0
    E = num.bit_length() - den.bit_length()        # num/den in [2^(E-1), 2^(E+1))
    if (num << max(0, -E)) < (den << max(0, E)):
        E -= 1                                     # now 2^E <= num/den < 2^(E+1)
    u = E - 7 if E >= -126 else -133
    a, b = (num, den << u) if u >= 0 else (num << -u, den)
    r, rem = divmod(a, b)
    if 2 * rem > b or (2 * rem == b and r & 1):
        r += 1
    return min(((u + 133) << 7) + r, 0x7F80)


def absmean_bf16(w_bits) -> int:
    """bf16 bits of the exact mean of |w| over bf16 weights (given as uint16 bit patterns).

    |w| = m * 2^(E' - 134) with E' = max(E, 1) and m = f + 128 [E >= 1] (E the
    exponent field, f the fraction); the mantissas are summed per exponent
    (exact in float64: at most 255 * 2^44 < 2^53), the per-exponent sums are
    combined as Python integers, and the mean is rounded once.
    """
    b = np.asarray(w_bits, dtype=np.uint16).reshape(-1).astype(np.int64) & 0x7FFF
    if b.size == 0:
        raise OracleError("empty weight matrix")
    if np.any(b >= 0x7F80):
        raise OracleError("weights must be finite")
    E = b >> 7
    m = (b & 0x7F) + np.where(E >= 1, 128, 0)
    Ep = np.maximum(E, 1)
    per_exp = np.bincount(Ep, weights=m.astype(np.float64), minlength=256)
    total = 0                                      # sum of |w|, in units of 2^-133
    for e in range(1, 256):
        if per_exp[e]:
            total += int(per_exp[e]) << (e - 1)
    return bf16_rne_ratio(total, b.size << 133)


def ternarize_absmean(w_bits):
    """Ternarise bf16 weights (uint16 bit patterns, N x K) as the page's converter does.

    Returns (q int8 N x K in {-1, 0, 1}, mean_bits, s_bits, ws_bits): the bf16
    mean of |W|, the bf16 multiplier s = 1 / max(mean, 1e-5), and the bf16
    weight scale ws = 1 / s that goes with the ternary matrix.
    """
    w = _c(np.atleast_2d(w_bits), np.uint16)
    mean = absmean_bf16(w)
    s_b = ctypes.c_uint16()
    ws_b = ctypes.c_uint16()
    lib = _load()
    _check(lib.oracle_absmean_scales(mean, ctypes.byref(s_b), ctypes.byref(ws_b)), "absmean_scales")
    q = np.empty(w.shape, dtype=np.int8)
    _check(lib.oracle_ternary_from_scale(_ptr(w), w.size, s_b.value, _ptr(q)), "ternary_from_scale")
    return q, mean, int(s_b.value), int(ws_b.value)


# --------------------------------------------------------------------------
# Glue between a block's projections  ([W2A8] §4.1 names the norms and the
# fused projections; the formulas are readings stated in oracle.c)
# --------------------------------------------------------------------------

RMS_EPS = np.float32(1e-5)


def rmsnorm_bf16(x_bits, g_bits, eps=RMS_EPS):
    """RMSNorm of a bf16 row with a bf16 weight, fp64, rounded once to bf16 (bits)."""
    x = _c(x_bits, np.uint16).reshape(-1)
    g = _c(g_bits, np.uint16).reshape(-1)
    if x.size != g.size:
        raise OracleError("rmsnorm sizes")
    y = np.empty_like(x)
    _check(_load().oracle_rmsnorm_bf16(_ptr(x), _ptr(g), x.size, float(eps), _ptr(y)), "rmsnorm_bf16")
    return y


def relu2_glu_bf16(gate_bits, up_bits):
    """bf16(max(gate, 0)^2 * up), elementwise (bits)."""
    a = _c(gate_bits, np.uint16).reshape(-1)
    b = _c(up_bits, np.uint16).reshape(-1)
    if a.size != b.size:
        raise OracleError("glu sizes")
    m = np.empty_like(a)
    _check(_load().oracle_relu2_glu_bf16(_ptr(a), _ptr(b), a.size, _ptr(m)), "relu2_glu_bf16")
    return m


def add_bf16(a_bits, b_bits):
    """bf16(a + b), elementwise (bits)."""
    a = _c(a_bits, np.uint16).reshape(-1)
    b = _c(b_bits, np.uint16).reshape(-1)
    if a.size != b.size:
        raise OracleError("add sizes")
    out = np.empty_like(a)
    _check(_load().oracle_add_bf16(_ptr(a), _ptr(b), a.size, _ptr(out)), "add_bf16")
    return out


def norm_bitlinear(x_bits, g_bits, w, ws_bits, ws_num, up_bits=None, residual_bits=None,
                   eps=RMS_EPS):
    """One projection of a block at M = 1: [relu2-GLU of (x, up)] -> RMSNorm(g) -> per-token
    int8 quantisation -> ternary layer -> [+ residual].  Returns (xn, q, s, acc, y)."""
    m = x_bits if up_bits is None else relu2_glu_bf16(x_bits, up_bits)
    xn = rmsnorm_bf16(m, g_bits, eps)
    q, s, acc, y = bitlinear_bf16(xn.reshape(1, -1), w, ws_bits, ws_num)
    y = y.reshape(-1)
    if residual_bits is not None:
        y = add_bf16(residual_bits, y)
    return xn, q.reshape(-1), s, acc.reshape(-1), y


def chained_layer(w, ws_bits, ws_num, gamma, attn_out_bits, h_bits, eps=RMS_EPS):
    """One layer of the decode step chained through its glue (the attention itself excluded;
    ``attn_out_bits`` stands for its output):
        qkv = wqkv(RMSNorm_attn(h))
        h1  = h + wo(RMSNorm_attn_sub(attn_out))
        gu  = w13(RMSNorm_ffn(h1))                       (gate half, then up half)
        h2  = h1 + w2(RMSNorm_ffn_sub(relu(gate)^2 * up))
    ``w``, ``ws_bits``, ``ws_num`` are keyed by qkv / o / gate_up / down and ``gamma`` by
    attn / attn_sub / ffn / ffn_sub.  Returns dict(qkv, h1, gu, h2) of bf16 bits."""
    qkv = norm_bitlinear(h_bits, gamma["attn"], w["qkv"], ws_bits["qkv"], ws_num["qkv"], eps=eps)[4]
    h1 = norm_bitlinear(attn_out_bits, gamma["attn_sub"], w["o"], ws_bits["o"], ws_num["o"],
                        residual_bits=h_bits, eps=eps)[4]
    gu = norm_bitlinear(h1, gamma["ffn"], w["gate_up"], ws_bits["gate_up"], ws_num["gate_up"],
                        eps=eps)[4]
    half = gu.size // 2
    h2 = norm_bitlinear(gu[:half], gamma["ffn_sub"], w["down"], ws_bits["down"], ws_num["down"],
                        up_bits=gu[half:], residual_bits=h1, eps=eps)[4]
    return {"qkv": qkv, "h1": h1, "gu": gu, "h2": h2}
