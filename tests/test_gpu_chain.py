"""GPU parity of the decode step chained through its glue (bitlinear_rmsnorm_i8xi2 and
bl_graph_create_norm) against the oracle.

Each projection of the pages' 2B layer with the glue it takes in the chain -- qkv
after attention_norm, o after attn_sub_norm plus the residual, gate+up after ffn_norm,
down after relu(gate)^2 * up and ffn_sub_norm plus the residual -- compared output by
output: the normalised row, its int8 quantisation and scale, the int32 accumulators and
the bf16 result.  Then rows that are not multiples of the kernel's tiles, the smallest K,
a zero row, a large-magnitude row, eps = 0, and chains of two layers and of the 30 the bench
times replayed as one graph.
The normalised row is defined in fp64; the kernel adds the squares in another order, which
could in principle move a value by 1 ulp, but no input here does: every output is asserted
exactly equal.
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


def run_proj(bl, x, gamma, w, ws, ws_num, x_up=None, residual=None, eps=oracle.RMS_EPS):
    import torch
    N, K = w.shape
    packed = bl.pack_ternary_weights(dev(w))
    xn = torch.empty((K,), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((K,), dtype=torch.int8, device="cuda")
    s = torch.empty((1,), dtype=torch.float32, device="cuda")
    acc = torch.empty((N,), dtype=torch.int32, device="cuda")
    y = bl.bitlinear_rmsnorm_i8xi2(bf16_dev(x), packed, bf16_dev(gamma), bf16_dev(ws), N, ws_num,
                                   x_up=None if x_up is None else bf16_dev(x_up),
                                   residual=None if residual is None else bf16_dev(residual),
                                   eps=eps, xn_out=xn, q_out=q, s_out=s, acc=acc)
    torch.cuda.synchronize()
    return host_bits(xn), q.cpu().numpy(), s.cpu().numpy(), acc.cpu().numpy(), host_bits(y)


def check_proj(bl, name, x, gamma, w, ws, ws_num, x_up=None, residual=None, eps=oracle.RMS_EPS):
    print(f"chain projection {name}: N={w.shape[0]} K={w.shape[1]} glu={x_up is not None} "
          f"residual={residual is not None}", flush=True)
    got = run_proj(bl, x, gamma, w, ws, ws_num, x_up, residual, eps)
    want = oracle.norm_bitlinear(x, gamma, w, ws, ws_num, up_bits=x_up, residual_bits=residual,
                                 eps=eps)
    for label, g_, w_ in zip(("xn", "q", "s", "acc", "y"), got, want):
        np.testing.assert_array_equal(np.asarray(g_).reshape(-1), np.asarray(w_).reshape(-1),
                                      err_msg=f"{name}: {label}")


@pytest.mark.parametrize("proj", ["qkv", "o", "gate_up", "down"])
def test_model_projection_with_glue(bl, proj):
    L = synth.chained_layer(0)
    h = synth.chained_h0()
    g = synth.rng(4242)
    if proj == "qkv":
        check_proj(bl, proj, h, L.gamma["attn"], L.w["qkv"], L.ws["qkv"], 1)
    elif proj == "o":
        check_proj(bl, proj, L.attn_out, L.gamma["attn_sub"], L.w["o"], L.ws["o"], 1, residual=h)
    elif proj == "gate_up":
        check_proj(bl, proj, h, L.gamma["ffn"], L.w["gate_up"], L.ws["gate_up"], 2)
    else:
        gate = synth.normal_bf16_bits(g, 1, synth.FFN).reshape(-1)
        up = synth.normal_bf16_bits(g, 1, synth.FFN).reshape(-1)
        check_proj(bl, proj, gate, L.gamma["ffn_sub"], L.w["down"], L.ws["down"], 1, x_up=up,
                   residual=h)


# (6400, 2320), (16, 28688) and (64, 32768): rows longer than the chunks a
# thread caches, so the kernel's loop over uncached chunks runs; K = 32768 is
# the largest, 16 steps per wavefront
@pytest.mark.parametrize("N,K,ws_num,glu", [(100, 272, 2, False), (16, 16, 1, True),
                                            (1000, 4096, 4, True), (8200, 512, 1, False),
                                            (6400, 2320, 2, True), (16, 28688, 1, False),
                                            (64, 32768, 2, True)])
def test_ragged_shapes(bl, N, K, ws_num, glu):
    g = synth.rng(N + K)
    x = synth.normal_bf16_bits(g, 1, K).reshape(-1)
    up = synth.normal_bf16_bits(g, 1, K).reshape(-1) if glu else None
    gamma = synth._top16((1.0 + 0.1 * g.standard_normal(K)).astype(np.float32))
    w = synth.ternary_uniform(g, N, K)
    res = synth.normal_bf16_bits(g, 1, N).reshape(-1)
    check_proj(bl, f"ragged{N}x{K}", x, gamma, w, synth.ws_bits(g, ws_num), ws_num, x_up=up,
               residual=res)


def test_zero_and_large_rows_and_no_eps(bl):
    g = synth.rng(31)
    K, N = 2560, 2560
    w = synth.ternary_uniform(g, N, K)
    ws = synth.ws_bits(g, 1)
    gamma = synth._top16((1.0 + 0.1 * g.standard_normal(K)).astype(np.float32))
    res = synth.normal_bf16_bits(g, 1, N).reshape(-1)
    zero = np.zeros(K, dtype=np.uint16)
    check_proj(bl, "zero row", zero, gamma, w, ws, 1, residual=res)            # y = residual
    big = synth._top16((1e30 * g.standard_normal(K)).astype(np.float32))
    check_proj(bl, "large row", big, gamma, w, ws, 1)
    x = synth.normal_bf16_bits(g, 1, K).reshape(-1)
    check_proj(bl, "eps 0", x, gamma, w, ws, 1, eps=0.0)
    neg = synth._top16(-np.abs(g.standard_normal(K)).astype(np.float32))       # GLU gate <= 0
    check_proj(bl, "negative gate", neg, gamma, w, ws, 1, x_up=x, residual=res)


def test_rounding_extremes(bl):
    # values whose roundings land among bf16's subnormals or far from 1
    g = synth.rng(47)
    K, N = 2560, 2560
    w = synth.ternary_uniform(g, N, K)
    ws = synth.ws_bits(g, 1)
    x = synth.normal_bf16_bits(g, 1, K).reshape(-1)
    gamma_sub = synth._top16((1e-39 * g.standard_normal(K)).astype(np.float32))   # subnormal gamma
    check_proj(bl, "subnormal gamma", x, gamma_sub, w, ws, 1)
    gamma = synth._top16(g.standard_normal(K).astype(np.float32))                  # signed gamma
    tiny_gate = synth._top16((1e-20 * g.standard_normal(K)).astype(np.float32))    # m subnormal
    check_proj(bl, "subnormal GLU", tiny_gate, gamma, w, ws, 1, x_up=x)
    big_gate = synth._top16((1e15 * g.standard_normal(K)).astype(np.float32))
    big_up = synth._top16((1e5 * g.standard_normal(K)).astype(np.float32))
    check_proj(bl, "large GLU", big_gate, gamma, w, ws, 1, x_up=big_up)


def test_bf16_midpoints(bl):
    # normalised values that are exactly a bf16 midpoint (eps = 0), and values
    # just below one whose nearest fp32 is the midpoint (eps = 2^-28): the
    # oracle's pin test derives both by hand; repeated over a row of 2560
    g = synth.rng(53)
    K, N = 2560, 1024
    w = synth.ternary_uniform(g, N, K)
    ws = synth.ws_bits(g, 1)
    x = np.tile(np.array([0x3FC0] * 4 + [0x3F80] * 7 + [0] * 5, dtype=np.uint16), K // 16)
    gamma = np.full(K, 0x3F81, dtype=np.uint16)
    check_proj(bl, "midpoint ties", x, gamma, w, ws, 1, eps=0.0)
    check_proj(bl, "below midpoints", x, gamma, w, ws, 1, eps=np.float32(2.0 ** -28))


@pytest.mark.parametrize("n_layers", [2, synth.N_LAYERS])
def test_chained_layers_as_graph(bl, n_layers):
    # two layers, and the whole step the bench times (its layers, inputs and
    # graph), every output of every layer checked on every replay
    import torch
    h0 = synth.chained_h0()
    print(f"chained graph: {n_layers} layers x 4 projections", flush=True)
    dim, ffn = synth.DIM, synth.FFN
    h = [bf16_dev(h0)] + [torch.empty(dim, dtype=torch.bfloat16, device="cuda") for _ in range(n_layers)]
    calls, keep, outs, want = [], [], [], []
    hb = h0
    for l in range(n_layers):
        # each layer's weights are made, packed and run through the oracle
        # in turn, so that the host holds one layer at a time
        L = synth.chained_layer(l)
        r = oracle.chained_layer(L.w, L.ws, L.ws_num, L.gamma, L.attn_out, hb)
        want.append(r)
        hb = r["h2"]
        p = {k: bl.pack_ternary_weights(dev(v)) for k, v in L.w.items()}
        wsd = {k: bf16_dev(v) for k, v in L.ws.items()}
        gm = {k: bf16_dev(v) for k, v in L.gamma.items()}
        a = bf16_dev(L.attn_out)
        qkv = torch.empty(3840, dtype=torch.bfloat16, device="cuda")
        h1 = torch.empty(dim, dtype=torch.bfloat16, device="cuda")
        gu = torch.empty(2 * ffn, dtype=torch.bfloat16, device="cuda")
        keep += [p, wsd, gm, a]
        outs.append({"qkv": qkv, "h1": h1, "gu": gu, "h2": h[l + 1]})
        calls += [
            dict(x=h[l], gamma=gm["attn"], packed=p["qkv"], ws=wsd["qkv"], ws_num=1, y=qkv, N=3840, K=dim),
            dict(x=a, gamma=gm["attn_sub"], packed=p["o"], ws=wsd["o"], ws_num=1, residual=h[l], y=h1,
                 N=dim, K=dim),
            dict(x=h1, gamma=gm["ffn"], packed=p["gate_up"], ws=wsd["gate_up"], ws_num=2, y=gu,
                 N=2 * ffn, K=dim),
            dict(x=gu[:ffn], x_up=gu[ffn:], gamma=gm["ffn_sub"], packed=p["down"], ws=wsd["down"],
                 ws_num=1, residual=h1, y=h[l + 1], N=dim, K=ffn),
        ]
    graph = bl.ChainedDecodeGraph(calls)
    assert len(graph) == 4 * n_layers
    # per layer: qkv and o (independent, one kernel instance) share a launch,
    # then gate+up, then down, which takes the activation and its statistics
    # from gate+up's epilogue
    assert graph.kernels == 3 * n_layers
    assert graph.linked == n_layers
    scratch = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        # every output poisoned, and unrelated eager work, between replays
        for o in outs:
            for k in ("qkv", "h1", "gu", "h2"):
                o[k].fill_(float("nan"))
        scratch.mul_(1.0001)
        torch.cuda.synchronize()
        graph.launch()
        torch.cuda.synchronize()
        for l in range(n_layers):
            for k in ("qkv", "h1", "gu", "h2"):
                np.testing.assert_array_equal(host_bits(outs[l][k]), want[l][k],
                                              err_msg=f"replay {rep} layer {l} {k}")
    graph.close()


def test_independent_projections_share_a_launch(bl):
    import torch
    # five independent calls: four of one kernel instance (rows of 2560;
    # narrow and ragged N; one adding its residual in place) in one grouped
    # launch, and the GLU projection of another instance on its own
    g = synth.rng(synth.seed_for(6, 50, 0))
    dim, ffn = synth.DIM, synth.FFN
    specs = [("qkv", 3840, dim, 1, False, None), ("o_inplace", dim, dim, 1, False, "inplace"),
             ("o", dim, dim, 1, False, "separate"), ("ragged", 2600, dim, 4, False, None),
             ("down", dim, ffn, 1, True, "separate")]
    calls, want = [], []
    for name, N, K, wn, glu, res in specs:
        w = synth.ternary_uniform(g, N, K)
        ws = synth.ws_bits(g, wn)
        x = synth.normal_bf16_bits(g, 1, K).reshape(-1)
        up = synth.normal_bf16_bits(g, 1, K).reshape(-1) if glu else None
        gam = oracle.bf16_rne(1.0 + 0.1 * g.normal(size=K))
        r = synth.normal_bf16_bits(g, 1, N).reshape(-1) if res else None
        want.append(oracle.norm_bitlinear(x, gam, w, ws, wn, up_bits=up, residual_bits=r)[4])
        y = bf16_dev(r) if res == "inplace" else torch.full((N,), float("nan"), dtype=torch.bfloat16,
                                                            device="cuda")
        c = dict(x=bf16_dev(x), gamma=bf16_dev(gam), packed=bl.pack_ternary_weights(dev(w)),
                 ws=bf16_dev(ws), ws_num=wn, y=y, N=N, K=K)
        if glu:
            c["x_up"] = bf16_dev(up)
        if res == "inplace":
            c["residual"] = y
        elif res == "separate":
            c["residual"] = bf16_dev(r)
        calls.append(c)
    print("chained graph: five independent projections", flush=True)
    graph = bl.ChainedDecodeGraph(calls)
    assert graph.kernels == 2
    torch.cuda.synchronize()
    graph.launch()
    torch.cuda.synchronize()
    for (name, *_), c, wv in zip(specs, calls, want):
        np.testing.assert_array_equal(host_bits(c["y"]), wv, err_msg=name)
    graph.close()


def _chain_case(bl, g, specs, ws0=None, x0=None):
    # specs: (N, K, ws_num, src, residual) per call; src "ext" reads a fresh row,
    # "halves" the two halves of the previous call's y as (x, x_up), "swapped"
    # them the other way round.  ws0 / x0 replace the first call's weight
    # scales / row.
    import torch
    calls, want, prev = [], [], None
    for i, (N, K, wn, src, res) in enumerate(specs):
        w = synth.ternary_uniform(g, N, K)
        ws = synth.ws_bits(g, wn) if i or ws0 is None else ws0
        gam = oracle.bf16_rne(1.0 + 0.1 * g.normal(size=K))
        r = synth.normal_bf16_bits(g, 1, N).reshape(-1) if res else None
        c = dict(gamma=bf16_dev(gam), packed=bl.pack_ternary_weights(dev(w)), ws=bf16_dev(ws),
                 ws_num=wn, y=torch.full((N,), float("nan"), dtype=torch.bfloat16, device="cuda"),
                 N=N, K=K)
        if src == "ext":
            x, up = synth.normal_bf16_bits(g, 1, K).reshape(-1), None
            if i == 0 and x0 is not None:
                x = x0
            c["x"] = bf16_dev(x)
        else:
            # "halves" / "swapped" of the previous call, or ("halves", i) of call i
            if isinstance(src, tuple):
                src, (pc, pw) = src[0], (calls[src[1]], want[src[1]])
            else:
                (pc, pw) = prev
            lo, hi = (slice(0, K), slice(K, 2 * K)) if src == "halves" else (slice(K, 2 * K), slice(0, K))
            c["x"], c["x_up"] = pc["y"][lo], pc["y"][hi]
            x, up = pw[lo], pw[hi]
        if res:
            c["residual"] = bf16_dev(r)
        yw = oracle.norm_bitlinear(x, gam, w, ws, wn, up_bits=up, residual_bits=r)[4]
        calls.append(c)
        want.append(yw)
        prev = (c, yw)
    return calls, want


def _replay_and_check(bl, label, calls, want, linked, reps=2, kernels=None):
    import torch
    print(f"chained graph: hand-off {label}", flush=True)
    graph = bl.ChainedDecodeGraph(calls)
    assert graph.kernels == (len(calls) if kernels is None else kernels)
    assert graph.linked == linked
    for rep in range(reps):
        for c in calls:
            c["y"].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.launch()
        torch.cuda.synchronize()
        for i, (c, wv) in enumerate(zip(calls, want)):
            np.testing.assert_array_equal(host_bits(c["y"]), wv, err_msg=f"{label} call {i} rep {rep}")
    graph.close()


@pytest.mark.parametrize("case", ["b4_256_parts", "producer_and_consumer", "swapped", "b1_small",
                                  "model_shape_ws2", "grouped"])
def test_glu_hand_off(bl, case):
    # The GLU projection takes m and its statistics from the call before it
    # when it reads that call's y as (gate, up): a producer of four bands per
    # workgroup (16384 rows: 256 workgroups, the most partials a consumer
    # reads) with residuals on both sides; a call that takes one hand-off and
    # gives the next (producers of four and of two bands per workgroup, the
    # second in 256 workgroups; consumer rows of 4096);
    # halves swapped, and a producer of one band per workgroup, which do not
    # link; the model's gate+up and down with split weight scales; and two
    # producers sharing a grouped launch, each read by one of two consumers
    # that share the next (no hand-off from or into a grouped launch).
    g = synth.rng(synth.seed_for(6, 60, len(case)))
    specs, linked = {
        "b4_256_parts": ([(16384, 512, 1, "ext", True), (100, 8192, 1, "halves", True)], 1),
        "producer_and_consumer": ([(8192, 512, 2, "ext", False), (8192, 4096, 1, "halves", False),
                                   (300, 4096, 3, "halves", True)], 2),
        "swapped": ([(13824, 2560, 2, "ext", False), (2560, 6912, 1, "swapped", True)], 0),
        "b1_small": ([(128, 256, 1, "ext", False), (48, 64, 1, "halves", False)], 0),
        "model_shape_ws2": ([(13824, 2560, 2, "ext", False), (2560, 6912, 2, "halves", True)], 1),
        "grouped": ([(13824, 2560, 1, "ext", False), (13824, 2560, 2, "ext", False),
                     (2560, 6912, 1, ("halves", 0), True), (2560, 6912, 1, ("halves", 1), False)], 0),
    }[case]
    calls, want = _chain_case(bl, g, specs)
    _replay_and_check(bl, case, calls, want, linked, kernels=2 if case == "grouped" else None)


@pytest.mark.parametrize("edge", ["zeros", "tiny", "huge"])
def test_glu_hand_off_edge_rows(bl, edge):
    # The hand-off over extreme activations, set through gate+up's input row
    # and weight scale: a zero row (m = 0, the consumer's row all zeros), a
    # weight scale of 2^-52 (m subnormal or zero), one of 2^30 (m up to about
    # 1e34, squares far beyond fp32)
    g = synth.rng(synth.seed_for(6, 61, len(edge)))
    specs = [(13824, 2560, 1, "ext", False), (2560, 6912, 1, "halves", True)]
    ws0 = {"zeros": None, "tiny": oracle.bf16_rne(np.array([2.0 ** -52])),
           "huge": oracle.bf16_rne(np.array([2.0 ** 30]))}[edge]
    x0 = np.zeros(2560, dtype=np.uint16) if edge == "zeros" else None
    calls, want = _chain_case(bl, g, specs, ws0=ws0, x0=x0)
    _replay_and_check(bl, f"edge rows {edge}", calls, want, 1, reps=1)


def test_output_over_another_input_is_refused(bl):
    import torch
    g = synth.rng(synth.seed_for(6, 51, 0))
    K = N = 256
    w = synth.ternary_uniform(g, N, K)
    x = bf16_dev(synth.normal_bf16_bits(g, 1, K).reshape(-1))
    gam = bf16_dev(oracle.bf16_rne(1.0 + 0.1 * g.normal(size=K)))
    c = dict(x=x, gamma=gam, packed=bl.pack_ternary_weights(dev(w)), ws=bf16_dev(synth.ws_bits(g, 1)),
             ws_num=1, y=gam, N=N, K=K)
    with pytest.raises(bl.BitLinearError) as e:
        bl.ChainedDecodeGraph([c])
    assert e.value.status == bl.BL_ERR_ARG
