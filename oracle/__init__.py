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
    for name in ("oracle_quant_absmax_i8_f32", "oracle_quant_absmax_i8_bf16", "oracle_unpack_tiles",
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
