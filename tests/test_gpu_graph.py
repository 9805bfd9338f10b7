"""The decode-step graph (W2A8 page §六 item 1: every decode step is a graph
replay): 30 layers x {qkv, o, gate+up, down} of the 2B-style model, fused
per-token quantisation of bf16 x ~ N(0,1) before each GEMV, captured once.

Every replay must equal the eager calls bit for bit, and both the oracle;
replays are interleaved with unrelated eager device work and host syncs.
Independent calls share one grouped launch: the 120-call step is one kernel.
Calls that read or overwrite an earlier call's output start a new launch,
and must see that output (or leave the earlier call its input); calls the
grouped kernel does not take (K > 10240) run on their own.
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


def _build(bl, nodes):
    import torch
    calls = []
    for c in nodes:
        calls.append(dict(x=bf16_dev(c.x), packed=bl.pack_ternary_weights(dev(c.w)),
                          ws=bf16_dev(c.ws), ws_num=c.ws_num,
                          y=torch.full((c.N,), float("nan"), dtype=torch.bfloat16, device="cuda"),
                          acc=torch.zeros((c.N,), dtype=torch.int32, device="cuda"),
                          N=c.N, K=c.K))
    return calls


def test_decode_step_graph(bl):
    import torch
    print("decode graph: build 120 nodes", flush=True)
    nodes = synth.decode_step_nodes()
    calls = _build(bl, nodes)
    torch.cuda.synchronize()
    expect = oracle.decode_step([(c.x, c.w, c.ws, c.ws_num) for c in nodes])

    print("decode graph: eager", flush=True)
    for c in calls:
        bl.bitlinear_bf16_i8xi2(c["x"], c["packed"], c["ws"], c["N"], c["ws_num"], y=c["y"],
                                acc=c["acc"])
    torch.cuda.synchronize()
    eager = [host_bits(c["y"]).copy() for c in calls]
    for i, (c, e) in enumerate(zip(calls, expect)):
        np.testing.assert_array_equal(c["acc"].cpu().numpy(), e[2][0], err_msg=f"node {i}")
        np.testing.assert_array_equal(eager[i], e[3][0], err_msg=f"node {i}")

    print("decode graph: capture", flush=True)
    g = bl.DecodeGraph(calls)
    assert len(g) == len(calls) == 120
    assert g.kernels == 1                    # 120 independent calls, one grouped launch
    scratch = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        for c in calls:
            c["y"].fill_(float("nan"))
            c["acc"].fill_(0)
        scratch.mul_(1.0001)                 # unrelated eager work between replays
        torch.cuda.synchronize()
        print(f"decode graph: replay {rep}", flush=True)
        g.launch()
        torch.cuda.synchronize()
        for i, c in enumerate(calls):
            np.testing.assert_array_equal(host_bits(c["y"]), eager[i], err_msg=f"rep {rep} node {i}")
            np.testing.assert_array_equal(c["acc"].cpu().numpy(), expect[i][2][0])
    g.close()


def _node(name, N, K, ws_num, seed):
    return synth.make_float_gemv(name, 1, N, K, ws_num, seed, bf16=True)


def _check_calls(bl, calls, nodes, xs=None, label=""):
    """Each call's acc and y against the oracle on its (possibly produced) input row."""
    for i, (c, nd) in enumerate(zip(calls, nodes)):
        x = nd.x if xs is None or xs[i] is None else xs[i]
        _, _, acc, y = oracle.bitlinear_bf16(x.reshape(1, -1), nd.w, nd.ws, nd.ws_num)
        np.testing.assert_array_equal(c["acc"].cpu().numpy(), acc[0], err_msg=f"{label} call {i}")
        np.testing.assert_array_equal(host_bits(c["y"]), y[0], err_msg=f"{label} call {i}")


def test_grouped_ragged_shapes(bl):
    import torch
    # rows that are not whole bands or workgroups, K from one 16-wide chunk to
    # four chunks of ten tiles, weight-scale segments that split bands
    shapes = [(1, 16, 1), (17, 272, 1), (2560, 2560, 1), (100, 2576, 4), (13824, 2560, 2),
              (2560, 6912, 1), (48, 10240, 3), (4000, 5120, 5), (3, 7936, 3), (1, 2560, 1)]
    nodes = [_node(f"ragged{i}", N, K, wn, synth.seed_for(7, 1, i))
             for i, (N, K, wn) in enumerate(shapes)]
    print(f"grouped graph: ragged shapes {shapes}", flush=True)
    calls = _build(bl, nodes)
    g = bl.DecodeGraph(calls)
    assert g.kernels == 1
    for rep in range(2):
        for c in calls:
            c["y"].fill_(float("nan"))
            c["acc"].fill_(0)
        torch.cuda.synchronize()
        g.launch()
        torch.cuda.synchronize()
        _check_calls(bl, calls, nodes, label=f"rep {rep}")
    g.close()


def test_dependent_call_sees_its_producer(bl):
    import torch
    # a, b independent; d reads a's output as its activation row; e independent
    # of all: runs [a, b] and [d, e], two launches
    a = _node("a", 2560, 2560, 1, synth.seed_for(7, 2, 0))
    b = _node("b", 3840, 2560, 1, synth.seed_for(7, 2, 1))
    d = _node("d", 6912, 2560, 2, synth.seed_for(7, 2, 2))
    e = _node("e", 2560, 6912, 1, synth.seed_for(7, 2, 3))
    nodes = [a, b, d, e]
    print("grouped graph: dependent call", flush=True)
    calls = _build(bl, nodes)
    calls[2]["x"] = calls[0]["y"]            # d's input is a's output
    g = bl.DecodeGraph(calls)
    assert g.kernels == 2
    for rep in range(2):
        for c in calls:
            c["acc"].fill_(0)
        for c in (calls[1], calls[3]):
            c["y"].fill_(float("nan"))
        calls[0]["y"].fill_(float("nan"))    # d must read what a writes, not this
        torch.cuda.synchronize()
        g.launch()
        torch.cuda.synchronize()
        produced = host_bits(calls[0]["y"]).copy()
        _check_calls(bl, calls, nodes, xs=[None, None, produced, None], label=f"rep {rep}")
        _, _, _, ya = oracle.bitlinear_bf16(a.x.reshape(1, -1), a.w, a.ws, a.ws_num)
        np.testing.assert_array_equal(produced, ya[0])
    g.close()


def test_overwritten_input_is_read_first(bl):
    import torch
    # p reads row r; q writes its output over r: q must run after p
    p = _node("p", 2560, 2560, 1, synth.seed_for(7, 3, 0))
    q = _node("q", 2560, 2560, 1, synth.seed_for(7, 3, 1))
    print("grouped graph: write after read", flush=True)
    calls = _build(bl, [p, q])
    calls[1]["y"] = calls[0]["x"]
    g = bl.DecodeGraph(calls)
    assert g.kernels == 2
    torch.cuda.synchronize()
    g.launch()
    torch.cuda.synchronize()
    _, _, accp, yp = oracle.bitlinear_bf16(p.x.reshape(1, -1), p.w, p.ws, p.ws_num)
    _, _, accq, yq = oracle.bitlinear_bf16(q.x.reshape(1, -1), q.w, q.ws, q.ws_num)
    np.testing.assert_array_equal(host_bits(calls[0]["y"]), yp[0])
    np.testing.assert_array_equal(calls[0]["acc"].cpu().numpy(), accp[0])
    np.testing.assert_array_equal(host_bits(calls[1]["y"]).reshape(-1), yq[0])
    g.close()


def test_long_rows_run_on_their_own(bl):
    import torch
    # K > 10240 is beyond the grouped kernel: [u, v] grouped, w alone, [x2] alone
    nodes = [_node("u", 640, 2560, 1, synth.seed_for(7, 4, 0)),
             _node("v", 1024, 6912, 1, synth.seed_for(7, 4, 1)),
             _node("w", 512, 13824, 1, synth.seed_for(7, 4, 2)),
             _node("x2", 256, 2560, 1, synth.seed_for(7, 4, 3))]
    print("grouped graph: long rows", flush=True)
    calls = _build(bl, nodes)
    g = bl.DecodeGraph(calls)
    assert g.kernels == 3
    torch.cuda.synchronize()
    g.launch()
    torch.cuda.synchronize()
    _check_calls(bl, calls, nodes, label="long rows")
    g.close()


def test_call_overwriting_its_own_input_is_refused(bl):
    import torch
    n = _node("self", 2560, 2560, 1, synth.seed_for(7, 5, 0))
    calls = _build(bl, [n])
    calls[0]["y"] = calls[0]["x"]
    with pytest.raises(bl.BitLinearError) as e:
        bl.DecodeGraph(calls)
    assert e.value.status == bl.BL_ERR_ARG
