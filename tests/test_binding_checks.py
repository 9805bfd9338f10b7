"""Host checks of the Python binding's argument validation (no GPU needed).

Every tensor the caller passes is checked for dtype, contiguity and element
count before the library is called, so an undersized buffer can never reach a
kernel.  The checks run before the device check, so CPU tensors exercise
them here: a wrong size raises ValueError naming the element count; the right
sizes get past every size check and stop at the device check.
"""
import pytest

torch = pytest.importorskip("torch")

import bit_gemv_bitlinear_amd as bl  # noqa: E402

N, K, M = 64, 256, 2


def t(n, dtype):
    return torch.zeros(n, dtype=dtype)


def packed():
    return t(bl.bl_packed_bytes(N, K), torch.uint8)


def check(fn, bad_name, **kw):
    """fn(**kw), with bad_name given the wrong element count, must raise the size error."""
    with pytest.raises(ValueError, match=r"elements, the call needs"):
        fn(**kw)


def device_error(fn, **kw):
    with pytest.raises(ValueError, match="device tensor"):
        fn(**kw)


def i8_args(**over):
    a = dict(xq=torch.zeros((M, K), dtype=torch.int8), packed=packed(),
             s=t(M, torch.float32), ws=t(2, torch.bfloat16), N=N, ws_num=2,
             y=t(M * N, torch.bfloat16), acc=t(M * N, torch.int32))
    a.update(over)
    return a


@pytest.mark.parametrize("name,bad", [("y", t(M * N - 1, torch.bfloat16)),
                                      ("acc", t(M * N - 1, torch.int32)),
                                      ("s", t(M - 1, torch.float32)),
                                      ("packed", t(bl.bl_packed_bytes(N, K) - 16, torch.uint8))])
def test_bitlinear_i8xi2_sizes(name, bad):
    check(bl.bitlinear_i8xi2, name, **i8_args(**{name: bad}))
    device_error(bl.bitlinear_i8xi2, **i8_args())


def test_ws_num_within_ws():
    with pytest.raises(ValueError, match="ws_num"):
        bl.bitlinear_i8xi2(**i8_args(ws_num=3))
    with pytest.raises(ValueError, match="ws_num"):
        bl.bitlinear_i8xi2(**i8_args(ws_num=0))


def bf16_args(**over):
    a = dict(x=torch.zeros((M, K), dtype=torch.bfloat16), packed=packed(), ws=t(1, torch.bfloat16),
             N=N, y=t(M * N, torch.bfloat16), q_out=t(M * K, torch.int8), s_out=t(M, torch.float32),
             acc=t(M * N, torch.int32))
    a.update(over)
    return a


@pytest.mark.parametrize("name,bad", [("y", t(M * N - 2, torch.bfloat16)),
                                      ("q_out", t(M * K - 1, torch.int8)),
                                      ("s_out", t(M - 1, torch.float32)),
                                      ("acc", t(M * N + 1, torch.int32))])
def test_bitlinear_bf16_i8xi2_sizes(name, bad):
    check(bl.bitlinear_bf16_i8xi2, name, **bf16_args(**{name: bad}))
    device_error(bl.bitlinear_bf16_i8xi2, **bf16_args())


def lut_args(**over):
    a = dict(xq=t(K, torch.int8), packed=packed(), s=t(1, torch.float32), ws=t(1, torch.bfloat16),
             N=N, y=t(N, torch.bfloat16), acc=t(N, torch.int32))
    a.update(over)
    return a


@pytest.mark.parametrize("name,bad", [("y", t(N - 1, torch.bfloat16)), ("acc", t(N - 1, torch.int32)),
                                      ("s", t(2, torch.float32))])
def test_bitlinear_lut_sizes(name, bad):
    check(bl.bitlinear_lut_i8xi2, name, **lut_args(**{name: bad}))
    device_error(bl.bitlinear_lut_i8xi2, **lut_args())


def norm_args(**over):
    a = dict(x=t(K, torch.bfloat16), packed=packed(), gamma=t(K, torch.bfloat16),
             ws=t(1, torch.bfloat16), N=N, x_up=t(K, torch.bfloat16), residual=t(N, torch.bfloat16),
             y=t(N, torch.bfloat16), xn_out=t(K, torch.bfloat16), q_out=t(K, torch.int8),
             s_out=t(1, torch.float32), acc=t(N, torch.int32))
    a.update(over)
    return a


@pytest.mark.parametrize("name,bad", [("x_up", t(K - 1, torch.bfloat16)),
                                      ("gamma", t(K + 1, torch.bfloat16)),
                                      ("residual", t(N - 1, torch.bfloat16)),
                                      ("y", t(N - 1, torch.bfloat16)),
                                      ("xn_out", t(K - 8, torch.bfloat16)),
                                      ("q_out", t(K - 1, torch.int8)),
                                      ("s_out", t(0, torch.float32)),
                                      ("acc", t(N - 1, torch.int32))])
def test_bitlinear_rmsnorm_sizes(name, bad):
    check(bl.bitlinear_rmsnorm_i8xi2, name, **norm_args(**{name: bad}))
    device_error(bl.bitlinear_rmsnorm_i8xi2, **norm_args())


def test_pack_and_ternarize_sizes():
    with pytest.raises(ValueError, match="elements"):
        bl.pack_ternary_weights(torch.zeros((N, K), dtype=torch.int8), n_invalid=t(0, torch.int32))
    with pytest.raises(ValueError, match="elements"):
        bl.ternarize_weights_absmean(torch.zeros((N, K), dtype=torch.bfloat16),
                                     workspace=t(bl.TERNARIZE_WORKSPACE_BYTES - 8, torch.uint8))
    device_error(bl.pack_ternary_weights, w=torch.zeros((N, K), dtype=torch.int8))


def graph_call(**over):
    c = dict(x=t(K, torch.bfloat16), packed=packed(), ws=t(1, torch.bfloat16), ws_num=1,
             y=t(N, torch.bfloat16), N=N, K=K)
    c.update(over)
    return c


@pytest.mark.parametrize("name,bad", [("x", t(K - 1, torch.bfloat16)), ("y", t(N - 1, torch.bfloat16)),
                                      ("acc", t(N - 1, torch.int32))])
def test_decode_graph_sizes(name, bad):
    with pytest.raises(ValueError, match="elements"):
        bl.DecodeGraph([graph_call(), graph_call(**{name: bad})])
    with pytest.raises(ValueError, match="ws_num"):
        bl.DecodeGraph([graph_call(ws_num=2)])
    with pytest.raises(ValueError, match="device tensor"):
        bl.DecodeGraph([graph_call()])


@pytest.mark.parametrize("name,bad", [("x", t(K - 1, torch.bfloat16)), ("x_up", t(K + 1, torch.bfloat16)),
                                      ("gamma", t(K - 1, torch.bfloat16)),
                                      ("residual", t(N - 1, torch.bfloat16)),
                                      ("y", t(N + 1, torch.bfloat16))])
def test_chained_graph_sizes(name, bad):
    base = dict(gamma=t(K, torch.bfloat16))
    with pytest.raises(ValueError, match="elements"):
        bl.ChainedDecodeGraph([graph_call(**{**base, name: bad})])
    with pytest.raises(ValueError, match="device tensor"):
        bl.ChainedDecodeGraph([graph_call(**base)])
