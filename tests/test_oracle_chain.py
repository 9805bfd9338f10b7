"""Pin of the oracle's composition of a chained decode-step layer
(oracle.norm_bitlinear / oracle.chained_layer).

The page ("BitNet GPU 推理框架：从零构建 W2A8 的 2-bit 大模型 CUDA GEMV 内核",
§4.1) names the converted model's norms and fused projections: attention_norm
before wqkv, attn_sub_norm before wo, ffn_norm before w13 (gate_proj rows
first, then up_proj rows) and ffn_sub_norm before w2.  The reading the oracle
follows, with the residual stream h and a stand-in for the attention output:

    qkv = wqkv( RMSNorm_attn(h) )
    h1  = bf16( h  + wo( RMSNorm_attn_sub(attn_out) ) )
    gu  = w13( RMSNorm_ffn(h1) ),   gate = gu[:F], up = gu[F:]
    h2  = bf16( h1 + w2( RMSNorm_ffn_sub( bf16(relu(gate)^2 * up) ) ) )

where each projection quantises its input per token (s = 127/amax in fp32,
q = round-half-even of fl32(x * s)), takes the exact int32 dot products and
rounds acc * ws / s once to fp64 and once to bf16, and where the residual is
added to the projection's bf16 output and rounded once more.

Here that layer is recomputed with nothing from the oracle: Python integers
and Fractions, every rounding (bf16, fp32, fp64; nearest, ties to even)
written out from the formats' definitions, RMSNorm decided exactly.  Small
shapes (dim 32, F = 32) with distinct gate and up halves; several layers
chained so that each layer's h2 feeds the next.  Variants that read the page
differently (gate and up swapped, the residual added before the projection is
rounded, the attention norms' weights swapped) are computed the same way and
must differ from the oracle, so the pin tells these readings apart.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from exact_bf16 import bf16_bits, bits_to_fraction, r32, r64, rmsnorm_exact

DIM, FFN, QKV = 32, 32, 48


def bf16_vec(values):
    return np.array([bf16_bits(v) for v in values], dtype=np.uint16)


def frac_vec(bits):
    return [bits_to_fraction(b) for b in bits]


def quantise(xn_bits):
    """Per-token absmax int8: s = fl32(127 / max(amax, fl32(1e-5))), q = rne(fl32(x * s))."""
    x = frac_vec(xn_bits)
    amax = max(max(abs(v) for v in x), r32(Fraction(1, 100000)))
    s = r32(Fraction(127) / amax)
    q = [max(-128, min(127, round(r32(v * s)))) for v in x]
    return q, s


def project(w, ws_bits, ws_num, xn_bits):
    """The ternary layer at M = 1 on the quantised row: y_n = bf16(fl64(acc_n * ws / s))."""
    q, s = quantise(xn_bits)
    N = w.shape[0]
    seg = N // ws_num
    out = []
    for n in range(N):
        acc = sum(int(a) * int(b) for a, b in zip(q, w[n]))
        ws = bits_to_fraction(ws_bits[n // seg])
        out.append(r64(acc * ws / s))
    return bf16_vec(out)


def add(a_bits, b_bits):
    return bf16_vec([x + y for x, y in zip(frac_vec(a_bits), frac_vec(b_bits))])


def glu(gate_bits, up_bits):
    """bf16(relu(gate)^2 * up); a zero product takes IEEE's sign, that of up (relu gives +0)."""
    out = []
    for g, ub in zip(frac_vec(gate_bits), up_bits):
        v = (g if g > 0 else 0) ** 2 * bits_to_fraction(ub)
        out.append(bf16_bits(v) if v != 0 else (int(ub) & 0x8000))
    return np.array(out, dtype=np.uint16)


def layer_exact(L, h, swap_gate_up=False, residual_before_rounding=False, swap_attn_norms=False):
    ga, gas = (L["gamma"]["attn_sub"], L["gamma"]["attn"]) if swap_attn_norms else \
              (L["gamma"]["attn"], L["gamma"]["attn_sub"])
    w, ws, wn = L["w"], L["ws"], L["ws_num"]
    qkv = project(w["qkv"], ws["qkv"], wn["qkv"], rmsnorm_exact(h, ga))
    if residual_before_rounding:
        q, s = quantise(rmsnorm_exact(L["attn_out"], gas))
        seg = DIM // wn["o"]
        h1 = bf16_vec([hv + r64(sum(int(a) * int(b) for a, b in zip(q, w["o"][n])) *
                                bits_to_fraction(ws["o"][n // seg]) / s)
                       for n, hv in enumerate(frac_vec(h))])
    else:
        h1 = add(h, project(w["o"], ws["o"], wn["o"], rmsnorm_exact(L["attn_out"], gas)))
    gu = project(w["gate_up"], ws["gate_up"], wn["gate_up"], rmsnorm_exact(h1, L["gamma"]["ffn"]))
    gate, up = gu[:FFN], gu[FFN:]
    if swap_gate_up:
        gate, up = up, gate
    m = glu(gate, up)
    h2 = add(h1, project(w["down"], ws["down"], wn["down"], rmsnorm_exact(m, L["gamma"]["ffn_sub"])))
    return {"qkv": qkv, "h1": h1, "gu": gu, "h2": h2}


def make_layer(g):
    def bf16(a):
        return oracle.bf16_rne(np.asarray(a, dtype=np.float64))
    shapes = {"qkv": (QKV, DIM, 1), "o": (DIM, DIM, 1), "gate_up": (2 * FFN, DIM, 2),
              "down": (DIM, FFN, 1)}
    w = {k: g.integers(-1, 2, size=(N, K)).astype(np.int8) for k, (N, K, _) in shapes.items()}
    ws = {k: bf16(g.uniform(0.02, 0.08, size=n)) for k, (_, _, n) in shapes.items()}
    ws_num = {k: n for k, (_, _, n) in shapes.items()}
    gamma = {"attn": bf16(1 + 0.1 * g.normal(size=DIM)), "attn_sub": bf16(1 + 0.1 * g.normal(size=DIM)),
             "ffn": bf16(1 + 0.1 * g.normal(size=DIM)), "ffn_sub": bf16(1 + 0.1 * g.normal(size=FFN))}
    return {"w": w, "ws": ws, "ws_num": ws_num, "gamma": gamma,
            "attn_out": bf16(g.normal(size=DIM))}


def layer_oracle(L, h):
    return oracle.chained_layer(L["w"], L["ws"], L["ws_num"], L["gamma"], L["attn_out"], h)


N_CHAIN = 4


@pytest.fixture(scope="module")
def chain():
    g = np.random.default_rng(20261202)
    layers = [make_layer(g) for _ in range(N_CHAIN)]
    h0 = oracle.bf16_rne(g.normal(size=DIM))
    return layers, h0


def test_rounding_helpers_against_ieee_hardware():
    # the format roundings written out here agree with numpy's fp32 and torch's
    # fp32 -> bf16 conversion (round to nearest even) on random values
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(1)
    for v in g.normal(size=300) * np.exp2(g.integers(-30, 30, size=300)):
        f = Fraction(float(v))
        assert r64(f) == f
        v32 = np.float32(v)
        assert r32(f) == Fraction(float(v32))
        t = torch.tensor([float(v32)], dtype=torch.float32).to(torch.bfloat16)
        assert bf16_bits(Fraction(float(v32))) == int(t.view(torch.int16).item()) & 0xFFFF
    assert r32(Fraction(1, 3)) == Fraction(float(np.float32(1) / np.float32(3)))


def test_chained_layers_match_exact_composition(chain):
    layers, h = chain
    for i, L in enumerate(layers):
        got = layer_oracle(L, h)
        want = layer_exact(L, h)
        for k in ("qkv", "h1", "gu", "h2"):
            np.testing.assert_array_equal(got[k], want[k], err_msg=f"layer {i}: {k}")
        h = got["h2"]


def test_gate_first_half_projection_helper(chain):
    # norm_bitlinear's pieces: the GLU input order and the residual of one projection
    layers, h = chain
    L = layers[0]
    out = layer_oracle(L, h)
    gate, up = out["gu"][:FFN], out["gu"][FFN:]
    xn, q, s, acc, y = oracle.norm_bitlinear(gate, L["gamma"]["ffn_sub"], L["w"]["down"],
                                             L["ws"]["down"], 1, up_bits=up,
                                             residual_bits=out["h1"])
    np.testing.assert_array_equal(xn, rmsnorm_exact(glu(gate, up), L["gamma"]["ffn_sub"]))
    qe, se = quantise(xn)
    np.testing.assert_array_equal(q, np.array(qe, dtype=np.int8))
    assert Fraction(float(s[0])) == se
    np.testing.assert_array_equal(y, out["h2"])


@pytest.mark.parametrize("variant", ["swap_gate_up", "residual_before_rounding", "swap_attn_norms"])
def test_other_readings_are_told_apart(chain, variant):
    layers, h = chain
    differs = False
    for L in layers:
        got = layer_oracle(L, h)
        alt = layer_exact(L, h, **{variant: True})
        differs |= any(not np.array_equal(got[k], alt[k]) for k in ("qkv", "h1", "gu", "h2"))
        h = got["h2"]
    assert differs, f"the {variant} reading gives the same bits: the pin would not catch it"
