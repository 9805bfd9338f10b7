"""The decode-step graph (W2A8 page §六 item 1: every decode step is a graph
replay): 30 layers x {qkv, o, gate+up, down} of the 2B-style model, fused
per-token quantisation of bf16 x ~ N(0,1) before each GEMV, captured once.

Every replay must equal the eager calls bit for bit, and both the oracle;
replays are interleaved with unrelated eager device work and host syncs.
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
