"""Host-side checks of the C ABI (no GPU needed): exported symbols, the packed
size, the host packer against the oracle's unpacker, and argument validation
(every error path returns its status before touching the device)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import bit_gemv_bitlinear_amd as bl
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "bitlinear.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*\(", text)
    skip = {"defined", "extern", "sizeof"}
    decl = set()
    for m in re.finditer(r"^(?:const\s+)?[A-Za-z_][A-Za-z0-9_ \*]*?\b([a-z_][a-z0-9_]*)\s*\(",
                         text, flags=re.M):
        if m.group(1) not in skip:
            decl.add(m.group(1))
    return decl & set(names)


def test_header_declares_the_bound_entry_points():
    decl = _declared_functions()
    assert decl == set(bl.SIGNATURES), (decl, set(bl.SIGNATURES))


def test_library_exports_every_declared_symbol():
    l = ctypes.CDLL(bl.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(l, name), name
    assert bl.lib().bl_abi_version() == 1


@pytest.mark.parametrize("N,K", [(1, 1), (64, 64), (65, 64), (64, 65), (13824, 2560),
                                 (2560, 6912), (70, 80), (0, 64), (64, 0)])
def test_packed_bytes_matches_oracle(N, K):
    assert bl.bl_packed_bytes(N, K) == (oracle.packed_bytes(N, K) if N > 0 and K > 0 else 0)


@pytest.mark.parametrize("N,K", [(16, 256), (128, 2560), (70, 80), (1, 16), (130, 6912), (3, 200),
                                 (17, 300)])
def test_host_packer_round_trips_through_oracle_unpack(N, K):
    g = np.random.Generator(np.random.PCG64(N * 100003 + K))
    w = g.integers(-1, 2, size=(N, K), dtype=np.int8)
    packed, bad = bl.bl_pack_ternary_host(w)
    assert bad == 0
    np.testing.assert_array_equal(oracle.unpack_tiles(packed, N, K), w)


def test_host_packer_counts_invalid_entries():
    w = np.zeros((16, 256), dtype=np.int8)
    w[3, 4] = 2
    w[5, 6] = -7
    packed, bad = bl.bl_pack_ternary_host(w)
    assert bad == 2
    with pytest.raises(oracle.OracleError, match="code 0"):
        oracle.unpack_tiles(packed, 16, 256)


# Argument validation.  Non-null dummy addresses are fine: every call below
# must fail on the host before any device access.
A = 4096            # 16-byte aligned dummy address
U = 4097            # misaligned dummy address


def _i8(xq=A, packed=A, s=A, ws=A, ws_num=1, y=A, acc=None, M=1, N=64, K=64):
    return bl.lib().bitlinear_i8xi2(xq, packed, s, ws, ws_num, y, acc, M, N, K, None)


def _bf(x=A, packed=A, ws=A, ws_num=1, y=A, q=None, s=None, acc=None, M=1, N=64, K=64):
    return bl.lib().bitlinear_bf16_i8xi2(x, packed, ws, ws_num, y, q, s, acc, M, N, K, None)


def test_bitlinear_i8xi2_errors():
    assert _i8(xq=None) == bl.BL_ERR_NULL
    assert _i8(packed=None) == bl.BL_ERR_NULL
    assert _i8(s=None) == bl.BL_ERR_NULL
    assert _i8(ws=None) == bl.BL_ERR_NULL
    assert _i8(y=None) == bl.BL_ERR_NULL
    assert _i8(M=0) == bl.BL_ERR_SHAPE
    assert _i8(N=0) == bl.BL_ERR_SHAPE
    assert _i8(K=8) == bl.BL_ERR_SHAPE
    assert _i8(K=72) == bl.BL_ERR_SHAPE                  # K % 16 != 0
    assert _i8(K=(1 << 20) + 16) == bl.BL_ERR_SHAPE
    assert _i8(N=(1 << 24) + 16) == bl.BL_ERR_SHAPE
    assert _i8(M=(1 << 20) + 1) == bl.BL_ERR_SHAPE
    assert _i8(M=1 << 20, N=(1 << 16) + 16) == bl.BL_ERR_SHAPE   # M * N > 2^36
    assert _bf(M=(1 << 20) + 1) == bl.BL_ERR_SHAPE
    assert _i8(ws_num=0) == bl.BL_ERR_ARG
    assert _i8(ws_num=3, N=64) == bl.BL_ERR_ARG          # N % ws_num != 0
    assert _i8(ws_num=65, N=65 * 64) == bl.BL_ERR_ARG
    assert _i8(xq=U) == bl.BL_ERR_ALIGN
    assert _i8(packed=A + 8) == bl.BL_ERR_ALIGN
    assert _i8(s=A + 2) == bl.BL_ERR_ALIGN
    assert _i8(acc=A + 2) == bl.BL_ERR_ALIGN
    assert _i8(y=U) == bl.BL_ERR_ALIGN


def _lut(xq=A, packed=A, s=A, ws=A, ws_num=1, y=A, acc=None, N=64, K=256):
    return bl.lib().bitlinear_lut_i8xi2(xq, packed, s, ws, ws_num, y, acc, N, K, None)


def test_bitlinear_lut_errors():
    assert _lut(xq=None) == bl.BL_ERR_NULL
    assert _lut(packed=None) == bl.BL_ERR_NULL
    assert _lut(s=None) == bl.BL_ERR_NULL
    assert _lut(y=None) == bl.BL_ERR_NULL
    assert _lut(N=0) == bl.BL_ERR_SHAPE
    assert _lut(K=72) == bl.BL_ERR_SHAPE
    assert _lut(K=bl.LUT_MAX_K + 16) == bl.BL_ERR_SHAPE     # the tables of the row in LDS
    assert _lut(ws_num=3, N=64) == bl.BL_ERR_ARG
    assert _lut(xq=U) == bl.BL_ERR_ALIGN
    assert _lut(acc=A + 2) == bl.BL_ERR_ALIGN


def test_bitlinear_bf16_errors():
    assert _bf(x=None) == bl.BL_ERR_NULL
    assert _bf(M=2) == bl.BL_ERR_NULL                    # M > 1 needs the staging buffers
    assert _bf(M=2, q=A) == bl.BL_ERR_NULL
    assert _bf(K=61440 + 16) == bl.BL_ERR_NULL           # beyond the fused K limit
    assert _bf(K=40) == bl.BL_ERR_SHAPE
    assert _bf(ws_num=2, N=65) == bl.BL_ERR_ARG
    assert _bf(x=A + 8) == bl.BL_ERR_ALIGN
    assert _bf(M=2, q=A + 4, s=A) == bl.BL_ERR_ALIGN


def test_quantize_and_pack_errors():
    q = bl.lib().quantize_act_absmax_i8
    assert q(None, 0, A, A, 1, 64, None) == bl.BL_ERR_NULL
    assert q(A, 2, A, A, 1, 64, None) == bl.BL_ERR_ARG
    assert q(A, 0, A, A, 0, 64, None) == bl.BL_ERR_SHAPE
    assert q(A, 0, A, A, 1, 24, None) == bl.BL_ERR_SHAPE
    assert q(A, 0, A, A, (1 << 20) + 1, 64, None) == bl.BL_ERR_SHAPE
    assert q(A + 4, 1, A, A, 1, 64, None) == bl.BL_ERR_ALIGN
    p = bl.lib().pack_ternary_weights
    assert p(None, A, 64, 64, None, None) == bl.BL_ERR_NULL
    assert p(A, A, 0, 64, None, None) == bl.BL_ERR_SHAPE
    assert p(A, A + 4, 64, 64, None, None) == bl.BL_ERR_ALIGN


def test_ternarize_errors():
    t = bl.lib().ternarize_weights_absmean
    assert t(None, A, A, A, 64, 64, None) == bl.BL_ERR_NULL
    assert t(A, A, A, None, 64, 64, None) == bl.BL_ERR_NULL
    assert t(A, A, A, A, 0, 64, None) == bl.BL_ERR_SHAPE
    assert t(A, A, A, A, 64, 40, None) == bl.BL_ERR_SHAPE         # K % 16 != 0
    assert t(A, A, A, A, 64, (1 << 20) + 16, None) == bl.BL_ERR_SHAPE
    assert t(A + 8, A, A, A, 64, 64, None) == bl.BL_ERR_ALIGN      # w must be 16-byte aligned
    assert t(A, A, U, A, 64, 64, None) == bl.BL_ERR_ALIGN
    assert t(A, A, A, A + 4, 64, 64, None) == bl.BL_ERR_ALIGN
    assert bl.TERNARIZE_WORKSPACE_BYTES == 2048


def test_graph_errors():
    g = ctypes.c_void_p()
    lib = bl.lib()
    assert lib.bl_graph_create(None, 1, ctypes.byref(g)) == bl.BL_ERR_NULL
    arr = (bl.bl_gemv_desc * 1)()
    arr[0] = bl.bl_gemv_desc(A, A, A, 1, A, None, 64, 64)
    assert lib.bl_graph_create(arr, 0, ctypes.byref(g)) == bl.BL_ERR_ARG
    arr[0] = bl.bl_gemv_desc(A, A, A, 1, A, None, 64, 40)
    assert lib.bl_graph_create(arr, 1, ctypes.byref(g)) == bl.BL_ERR_SHAPE
    assert g.value is None
    assert lib.bl_graph_launch(None, None) == bl.BL_ERR_NULL
    assert lib.bl_graph_size(None) == bl.BL_ERR_NULL
    assert lib.bl_graph_destroy(None) == bl.BL_OK
    assert bl.status_string(bl.BL_ERR_ALIGN).startswith("a pointer")


def _nrm(x=A, x_up=None, gamma=A, eps=1e-5, packed=A, ws=A, ws_num=1, res=None, y=A, xn=None,
         q=None, s=None, acc=None, N=64, K=64):
    return bl.lib().bitlinear_rmsnorm_i8xi2(x, x_up, gamma, eps, packed, ws, ws_num, res, y, xn,
                                            q, s, acc, N, K, None)


def test_rmsnorm_entry_errors():
    assert _nrm(x=None) == bl.BL_ERR_NULL
    assert _nrm(gamma=None) == bl.BL_ERR_NULL
    assert _nrm(packed=None) == bl.BL_ERR_NULL
    assert _nrm(ws=None) == bl.BL_ERR_NULL
    assert _nrm(y=None) == bl.BL_ERR_NULL
    assert _nrm(N=0) == bl.BL_ERR_SHAPE
    assert _nrm(K=40) == bl.BL_ERR_SHAPE                 # K % 16 != 0
    assert _nrm(K=32768 + 16) == bl.BL_ERR_SHAPE         # beyond the glue kernel's K
    assert _nrm(eps=-1.0) == bl.BL_ERR_ARG
    assert _nrm(eps=float("nan")) == bl.BL_ERR_ARG
    assert _nrm(eps=float("inf")) == bl.BL_ERR_ARG
    assert _nrm(ws_num=3, N=64) == bl.BL_ERR_ARG
    assert _nrm(x=A + 8) == bl.BL_ERR_ALIGN
    assert _nrm(x_up=A + 8) == bl.BL_ERR_ALIGN
    assert _nrm(gamma=A + 2) == bl.BL_ERR_ALIGN
    assert _nrm(res=U) == bl.BL_ERR_ALIGN
    assert _nrm(xn=A + 8) == bl.BL_ERR_ALIGN
    assert _nrm(q=A + 4) == bl.BL_ERR_ALIGN
    assert _nrm(s=A + 2) == bl.BL_ERR_ALIGN


def test_chained_graph_errors():
    g = ctypes.c_void_p()
    lib = bl.lib()
    assert lib.bl_graph_create_norm(None, 1, ctypes.byref(g)) == bl.BL_ERR_NULL
    arr = (bl.bl_norm_desc * 1)()
    arr[0] = bl.bl_norm_desc(A, None, A, 1e-5, A, A, 1, None, A, 64, 64)
    assert lib.bl_graph_create_norm(arr, 0, ctypes.byref(g)) == bl.BL_ERR_ARG
    arr[0] = bl.bl_norm_desc(A, None, A, 1e-5, A, A, 1, None, A, 64, 40)
    assert lib.bl_graph_create_norm(arr, 1, ctypes.byref(g)) == bl.BL_ERR_SHAPE
    arr[0] = bl.bl_norm_desc(A, None, None, 1e-5, A, A, 1, None, A, 64, 64)
    assert lib.bl_graph_create_norm(arr, 1, ctypes.byref(g)) == bl.BL_ERR_NULL
    assert g.value is None
