"""Python binding of libbitlinear.so, the gfx950 W2A8 ternary linear layer.

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI of include/bitlinear.h.  torch provides device memory and
streams; the functions take and return torch tensors on the current HIP
device and enqueue on ``torch.cuda.current_stream()``.

The library is loaded on first use; if it has not been built, or a call is
made without a GPU, the call raises -- there is no fallback of any kind.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitlinear.so")

BL_OK, BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_HIP, BL_ERR_ARG = 0, -1, -2, -3, -4, -5
TERNARIZE_WORKSPACE_BYTES = 2048   # BL_TERNARIZE_WORKSPACE_BYTES
# Largest K the single-kernel M = 1 paths take (include/bitlinear.h); beyond it the
# bf16 entry needs staging buffers for the quantised activations.
GEMV_MAX_K = 61440
# Largest K of the projection with its glue (bitlinear_rmsnorm_i8xi2).
NORM_MAX_K = 32768
LUT_MAX_K = 8192
RMS_EPS = 1e-5

# Entry points declared in include/bitlinear.h: name -> (restype, argtypes).
_P = ctypes.c_void_p
_I = ctypes.c_int
SIGNATURES = {
    "bl_status_string": (ctypes.c_char_p, [_I]),
    "bl_abi_version": (_I, []),
    "bl_packed_bytes": (ctypes.c_size_t, [_I, _I]),
    "pack_ternary_weights": (_I, [_P, _P, _I, _I, _P, _P]),
    "bl_pack_ternary_host": (ctypes.c_int64, [_P, _P, _I, _I]),
    "ternarize_weights_absmean": (_I, [_P, _P, _P, _P, _I, _I, _P]),
    "ternarize_weights_absmean_noalloc": (_I, [_P, _P, _P, _I, _I, _P]),
    "quantize_act_absmax_i8": (_I, [_P, _I, _P, _P, _I, _I, _P]),
    "bitlinear_i8xi2": (_I, [_P, _P, _P, _P, _I, _P, _P, _I, _I, _I, _P]),
    "bitlinear_bf16_i8xi2": (_I, [_P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _P]),
    "bitlinear_lut_i8xi2": (_I, [_P, _P, _P, _P, _I, _P, _P, _I, _I, _P]),
    "bitlinear_rmsnorm_i8xi2": (_I, [_P, _P, _P, ctypes.c_float, _P, _P, _I, _P, _P, _P, _P, _P,
                                     _P, _I, _I, _P]),
    "bl_graph_create": (_I, [_P, _I, ctypes.POINTER(_P)]),
    "bl_graph_create_norm": (_I, [_P, _I, ctypes.POINTER(_P)]),
    "bl_graph_launch": (_I, [_P, _P]),
    "bl_graph_size": (_I, [_P]),
    "bl_graph_kernels": (_I, [_P]),
    "bl_graph_linked": (_I, [_P]),
    "bl_graph_destroy": (_I, [_P]),
}


class BitLinearError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class bl_gemv_desc(ctypes.Structure):
    _fields_ = [("x", _P), ("packed", _P), ("ws", _P), ("ws_num", _I), ("y", _P), ("acc", _P),
                ("N", _I), ("K", _I)]


class bl_norm_desc(ctypes.Structure):
    _fields_ = [("x", _P), ("x_up", _P), ("gamma", _P), ("eps", ctypes.c_float), ("packed", _P),
                ("ws", _P), ("ws_num", _I), ("residual", _P), ("y", _P), ("N", _I), ("K", _I)]


_lib = None


def lib():
    """The loaded C library (ctypes.CDLL), with argument types set."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run bit_gemv_bitlinear_amd/build.py "
                              "(or __graft_entry__.build())")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def status_string(status: int) -> str:
    return lib().bl_status_string(status).decode()


def _check(status, what):
    if status != BL_OK:
        raise BitLinearError(status, what)


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require(t, dtype, name, numel=None):
    """Check a tensor argument before anything reaches the library: its dtype, that it is
    contiguous and its element count when the call fixes one (an undersized buffer would be
    read or written past its end by the kernel).  Every entry point checks all of its
    tensors this way first, then that they live on the device (_on_device)."""
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, the call needs {numel}")


def _on_device(**tensors):
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")


def _optional(t, dtype, name, numel):
    if t is not None:
        _require(t, dtype, name, numel)


def _ws_num(ws, ws_num):
    """ws_num defaults to every scale of ws; an explicit one must lie within ws."""
    if ws_num is None:
        return ws.numel()
    if not 1 <= ws_num <= ws.numel():
        raise ValueError(f"ws_num = {ws_num} outside 1..{ws.numel()} (the scales in ws)")
    return ws_num


def _packed(packed, N, K):
    import torch
    _require(packed, torch.uint8, "packed", bl_packed_bytes(N, K))


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def bl_packed_bytes(N: int, K: int) -> int:
    return int(lib().bl_packed_bytes(N, K))


def pack_ternary_weights(w, n_invalid=None):
    """Pack an int8 N x K ternary matrix (device) into the 16x256-tile layout (uint8 tensor)."""
    import torch
    if w.dim() != 2:
        raise ValueError("w must be an N x K matrix")
    _require(w, torch.int8, "w")
    N, K = w.shape
    _optional(n_invalid, torch.int32, "n_invalid", 1)
    _on_device(w=w, n_invalid=n_invalid)
    packed = torch.empty(bl_packed_bytes(N, K), dtype=torch.uint8, device=w.device)
    _check(lib().pack_ternary_weights(_ptr(w), _ptr(packed), N, K, _ptr(n_invalid), _stream()),
           "pack_ternary_weights")
    return packed


def bl_pack_ternary_host(w: np.ndarray):
    """Host twin of pack_ternary_weights on a numpy int8 N x K array -> (packed uint8, n_invalid)."""
    w = np.ascontiguousarray(w, dtype=np.int8)
    N, K = w.shape
    out = np.zeros(bl_packed_bytes(N, K), dtype=np.uint8)
    r = lib().bl_pack_ternary_host(w.ctypes.data_as(_P), out.ctypes.data_as(_P), N, K)
    if r < 0:
        raise BitLinearError(int(r), "bl_pack_ternary_host")
    return out, int(r)


def ternarize_weights_absmean(w, workspace=None):
    """bf16 N x K weights (device) -> (packed uint8, scales bf16[3] = ws, s, mean).

    Ternarises by the mean absolute value and packs (include/bitlinear.h);
    ``workspace`` (uint8, TERNARIZE_WORKSPACE_BYTES) is allocated when not given.
    """
    import torch
    if w.dim() != 2:
        raise ValueError("w must be an N x K matrix")
    _require(w, torch.bfloat16, "w")
    N, K = w.shape
    _optional(workspace, torch.uint8, "workspace", TERNARIZE_WORKSPACE_BYTES)
    _on_device(w=w, workspace=workspace)
    packed = torch.empty(bl_packed_bytes(N, K), dtype=torch.uint8, device=w.device)
    scales = torch.empty(3, dtype=torch.bfloat16, device=w.device)
    if workspace is None:
        workspace = torch.empty(TERNARIZE_WORKSPACE_BYTES, dtype=torch.uint8, device=w.device)
    _check(lib().ternarize_weights_absmean(_ptr(w), _ptr(packed), _ptr(scales), _ptr(workspace),
                                           N, K, _stream()), "ternarize_weights_absmean")
    return packed, scales


def quantize_act_absmax_i8(x):
    """Per-row absmax int8 quantisation of fp32 or bf16 M x K (device) -> (q int8, s fp32)."""
    import torch
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("x must be float32 or bfloat16")
    _require(x, x.dtype, "x")
    _on_device(x=x)
    x2 = x.reshape(-1, x.shape[-1])
    M, K = x2.shape
    q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    s = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(lib().quantize_act_absmax_i8(_ptr(x2), 1 if x.dtype == torch.bfloat16 else 0, _ptr(q),
                                        _ptr(s), M, K, _stream()), "quantize_act_absmax_i8")
    return q, s


def bitlinear_i8xi2(xq, packed, s, ws, N, ws_num=None, y=None, acc=None):
    """int8 activations (M x K), packed weights, fp32 s (M), bf16 ws -> bf16 y (M x N).

    ``acc`` (int32 M x N) receives the int32 accumulators when given; ``y``
    may be passed to reuse an output buffer.
    """
    import torch
    _require(xq, torch.int8, "xq")
    xq2 = xq.reshape(-1, xq.shape[-1])
    M, K = xq2.shape
    _packed(packed, N, K)
    _require(s, torch.float32, "s", M)
    _require(ws, torch.bfloat16, "ws")
    ws_num = _ws_num(ws, ws_num)
    _optional(y, torch.bfloat16, "y", M * N)
    _optional(acc, torch.int32, "acc", M * N)
    _on_device(xq=xq, packed=packed, s=s, ws=ws, y=y, acc=acc)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    _check(lib().bitlinear_i8xi2(_ptr(xq2), _ptr(packed), _ptr(s), _ptr(ws), ws_num, _ptr(y),
                                 _ptr(acc), M, N, K, _stream()), "bitlinear_i8xi2")
    return y


def bitlinear_lut_i8xi2(xq, packed, s, ws, N, ws_num=None, y=None, acc=None):
    """The M = 1 layer by table lookup: int8 xq (K), packed weights, fp32 s (1), bf16 ws ->
    bf16 y (N); the same bits as bitlinear_i8xi2 (a second algorithm, K <= LUT_MAX_K)."""
    import torch
    K = xq.shape[-1]
    if xq.numel() != K:
        raise ValueError("bitlinear_lut_i8xi2 takes one activation row")
    _require(xq, torch.int8, "xq")
    _packed(packed, N, K)
    _require(s, torch.float32, "s", 1)
    _require(ws, torch.bfloat16, "ws")
    ws_num = _ws_num(ws, ws_num)
    _optional(y, torch.bfloat16, "y", N)
    _optional(acc, torch.int32, "acc", N)
    _on_device(xq=xq, packed=packed, s=s, ws=ws, y=y, acc=acc)
    if y is None:
        y = torch.empty((N,), dtype=torch.bfloat16, device=xq.device)
    _check(lib().bitlinear_lut_i8xi2(_ptr(xq), _ptr(packed), _ptr(s), _ptr(ws), ws_num, _ptr(y),
                                     _ptr(acc), N, K, _stream()), "bitlinear_lut_i8xi2")
    return y


def bitlinear_bf16_i8xi2(x, packed, ws, N, ws_num=None, y=None, q_out=None, s_out=None, acc=None):
    """bf16 activations (M x K) -> per-token int8 quantisation + the layer -> bf16 y (M x N).

    For M > 1 the quantised activations are staged in ``q_out``/``s_out``;
    they are allocated here when not given.
    """
    import torch
    _require(x, torch.bfloat16, "x")
    x2 = x.reshape(-1, x.shape[-1])
    M, K = x2.shape
    _packed(packed, N, K)
    _require(ws, torch.bfloat16, "ws")
    ws_num = _ws_num(ws, ws_num)
    _optional(y, torch.bfloat16, "y", M * N)
    _optional(q_out, torch.int8, "q_out", M * K)
    _optional(s_out, torch.float32, "s_out", M)
    _optional(acc, torch.int32, "acc", M * N)
    _on_device(x=x, packed=packed, ws=ws, y=y, q_out=q_out, s_out=s_out, acc=acc)
    if (M > 1 or K > GEMV_MAX_K) and q_out is None:
        q_out = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if (M > 1 or K > GEMV_MAX_K) and s_out is None:
        s_out = torch.empty((M,), dtype=torch.float32, device=x.device)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check(lib().bitlinear_bf16_i8xi2(_ptr(x2), _ptr(packed), _ptr(ws), ws_num, _ptr(y),
                                      _ptr(q_out), _ptr(s_out), _ptr(acc), M, N, K, _stream()),
           "bitlinear_bf16_i8xi2")
    return y


def bitlinear_rmsnorm_i8xi2(x, packed, gamma, ws, N, ws_num=None, x_up=None, residual=None,
                            eps=RMS_EPS, y=None, xn_out=None, q_out=None, s_out=None, acc=None):
    """One projection with its glue (M = 1): [relu(x)^2 * x_up] -> RMSNorm(gamma, eps) ->
    per-token int8 quantisation -> the layer -> [+ residual].  Returns y (bf16, N)."""
    import torch
    _require(x, torch.bfloat16, "x")
    K = x.numel()
    _optional(x_up, torch.bfloat16, "x_up", K)
    _require(gamma, torch.bfloat16, "gamma", K)
    _packed(packed, N, K)
    _require(ws, torch.bfloat16, "ws")
    ws_num = _ws_num(ws, ws_num)
    _optional(residual, torch.bfloat16, "residual", N)
    _optional(y, torch.bfloat16, "y", N)
    _optional(xn_out, torch.bfloat16, "xn_out", K)
    _optional(q_out, torch.int8, "q_out", K)
    _optional(s_out, torch.float32, "s_out", 1)
    _optional(acc, torch.int32, "acc", N)
    _on_device(x=x, x_up=x_up, gamma=gamma, packed=packed, ws=ws, residual=residual, y=y,
               xn_out=xn_out, q_out=q_out, s_out=s_out, acc=acc)
    if y is None:
        y = torch.empty((N,), dtype=torch.bfloat16, device=x.device)
    _check(lib().bitlinear_rmsnorm_i8xi2(_ptr(x), _ptr(x_up), _ptr(gamma), float(eps),
                                         _ptr(packed), _ptr(ws), ws_num, _ptr(residual),
                                         _ptr(y), _ptr(xn_out), _ptr(q_out), _ptr(s_out),
                                         _ptr(acc), N, K, _stream()),
           "bitlinear_rmsnorm_i8xi2")
    return y


class DecodeGraph:
    """A chain of M = 1 bf16 layer calls captured once (bl_graph_create) and replayed.

    ``calls`` is a list of dicts with keys x, packed, ws, ws_num, y, N, K and
    optionally acc (device tensors); they must stay alive as long as the graph.
    """

    def __init__(self, calls):
        import torch
        for i, c in enumerate(calls):
            N, K = c["N"], c["K"]
            _require(c["x"], torch.bfloat16, f"calls[{i}].x", K)
            _packed(c["packed"], N, K)
            _require(c["ws"], torch.bfloat16, f"calls[{i}].ws")
            _ws_num(c["ws"], c["ws_num"])
            _require(c["y"], torch.bfloat16, f"calls[{i}].y", N)
            _optional(c.get("acc"), torch.int32, f"calls[{i}].acc", N)
        for i, c in enumerate(calls):
            _on_device(**{f"calls[{i}].{k}": c.get(k) for k in ("x", "packed", "ws", "y", "acc")})
        self._keep = calls
        arr = (bl_gemv_desc * len(calls))()
        for i, c in enumerate(calls):
            arr[i] = bl_gemv_desc(c["x"].data_ptr(), c["packed"].data_ptr(), c["ws"].data_ptr(),
                                  c["ws_num"], c["y"].data_ptr(),
                                  c["acc"].data_ptr() if c.get("acc") is not None else None,
                                  c["N"], c["K"])
        h = ctypes.c_void_p()
        _check(lib().bl_graph_create(arr, len(calls), ctypes.byref(h)), "bl_graph_create")
        self._h = h

    def __len__(self):
        return lib().bl_graph_size(self._h)

    @property
    def kernels(self):
        """Kernel launches per replay (independent calls share a grouped launch)."""
        return lib().bl_graph_kernels(self._h)

    def launch(self):
        _check(lib().bl_graph_launch(self._h, _stream()), "bl_graph_launch")

    def close(self):
        if self._h:
            _check(lib().bl_graph_destroy(self._h), "bl_graph_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class ChainedDecodeGraph(DecodeGraph):
    """A decode step chained through its glue (bl_graph_create_norm): ``calls`` is a list of
    dicts with keys x, gamma, packed, ws, ws_num, y, N, K and optionally x_up, residual, eps;
    each call may read an earlier call's y.  The tensors must stay alive with the graph."""

    def __init__(self, calls):
        import torch
        for i, c in enumerate(calls):
            N, K = c["N"], c["K"]
            _require(c["x"], torch.bfloat16, f"calls[{i}].x", K)
            _optional(c.get("x_up"), torch.bfloat16, f"calls[{i}].x_up", K)
            _require(c["gamma"], torch.bfloat16, f"calls[{i}].gamma", K)
            _packed(c["packed"], N, K)
            _require(c["ws"], torch.bfloat16, f"calls[{i}].ws")
            _ws_num(c["ws"], c["ws_num"])
            _optional(c.get("residual"), torch.bfloat16, f"calls[{i}].residual", N)
            _require(c["y"], torch.bfloat16, f"calls[{i}].y", N)
        for i, c in enumerate(calls):
            _on_device(**{f"calls[{i}].{k}": c.get(k)
                          for k in ("x", "x_up", "gamma", "packed", "ws", "residual", "y")})
        self._keep = calls
        arr = (bl_norm_desc * len(calls))()

        def p(c, k):
            return c[k].data_ptr() if c.get(k) is not None else None
        for i, c in enumerate(calls):
            arr[i] = bl_norm_desc(p(c, "x"), p(c, "x_up"), p(c, "gamma"), float(c.get("eps", RMS_EPS)),
                                  p(c, "packed"), p(c, "ws"), c["ws_num"], p(c, "residual"),
                                  p(c, "y"), c["N"], c["K"])
        h = ctypes.c_void_p()
        _check(lib().bl_graph_create_norm(arr, len(calls), ctypes.byref(h)), "bl_graph_create_norm")
        self._h = h

    @property
    def linked(self):
        """Calls that take the activation and its norm statistics from the call before them."""
        return lib().bl_graph_linked(self._h)
