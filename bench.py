#!/usr/bin/env python3
"""Benchmark of the W2A8 ternary linear layer on one MI355X.

Headline: the M = 1 GEMV (int8 activations x packed ternary weights -> bf16)
at N = 13824, K = 2560 (the fused gate+up projection of the 2B-style model
in the W2A8 page, "BitNet GPU 推理框架：从零构建 W2A8 的 2-bit 大模型 CUDA GEMV
内核", §一 and §7.1), reported as microseconds per GEMV and achieved HBM
GB/s against MI355X's 8 TB/s.

Method:
  * inputs are seeded synthetic data of the page's shapes (module ``synth``),
    resident in HBM before timing starts;
  * the packed weights are replicated into enough copies (>= 512 MiB in
    total) that consecutive GEMVs never find their weights in the 256 MiB
    Infinity Cache or the 4 MiB L2s; launch i reads copy i % copies;
  * the K timed launches are captured in one HIP graph, bracketed by HIP
    events recorded on the stream the graph runs on, after W untimed
    warm-up launches and one untimed replay of the same graph (a graph's
    first replay runs every launch slower; a decode loop replays its graph
    once per token);
  * bytes per GEMV = N*K/4 (packed weights) + M*K (int8 x) + 2*M*N (bf16 y)
    + 4*M (s) + 2*ws_num (ws) -- the algorithmic bytes, each read once.

Prints one JSON line.  ``--gpus`` above 1 is refused: this build runs on one GPU.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, published peak
PEAK_INT8_TOPS = 5000.0          # MI355X dense int8 MFMA, published peak (TOP/s)
A100_W2A8_GBS_13824x2560 = 473.5  # the page's 18.75 us on A100 (§7.1), as GB/s by the same formula
CACHE_DEFEAT_BYTES = 512 << 20
PROFILE_PMC = os.path.join(ROOT, "profiles", "gemv_i8_13824x2560_pmc.txt")
# the headline kernel's sources and the build script that holds its compile flags
GEMV_SOURCES = [os.path.join(ROOT, "bit_gemv_bitlinear_amd", "csrc", f)
                for f in ("gemv.hip", "gemv_core.hpp", "common.hpp")] + \
               [os.path.join(ROOT, "bit_gemv_bitlinear_amd", "build.py")]
PROBE_LIB = os.path.join(ROOT, "bit_gemv_bitlinear_amd", "libstream_floor.so")


def gemv_bytes(M, N, K, ws_num, x_bytes=1):
    return N * K // 4 + x_bytes * M * K + 2 * M * N + 4 * M + 2 * ws_num


def _torch():
    import torch
    return torch


def bf16_dev(bits):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16).cuda()


def copies_for(nbytes):
    return max(2, -(-CACHE_DEFEAT_BYTES // nbytes))


def replicate(packed, n):
    torch = _torch()
    out = torch.empty((n, packed.numel()), dtype=torch.uint8, device=packed.device)
    out.copy_(packed.unsqueeze(0).expand(n, -1))
    return [out[i] for i in range(n)]


def time_graph(launch, steps, warmup):
    """Average ms per launch of `steps` launches captured in one graph (after `warmup` launches).

    The timed graph is replayed once, untimed, before the timed replay: on this runtime a
    graph's first replay runs every launch slower than later replays (measured same box:
    13824 x 2560 int8 3.43 against 3.32 us, bf16 input 4.14 against 3.63 us), and a decode
    loop replays its graph once per token.  Uploading the graph beforehand (hipGraphUpload)
    does not remove that cost."""
    torch = _torch()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(min(warmup, 8)):
            launch(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    if warmup > 8:
        gw = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gw):
            for i in range(warmup - 8):
                launch(i)
        gw.replay()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            launch(i)
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def headline(bl, steps, warmup):
    """M=1 GEMV, N=13824, K=2560, ws_num=2, int8 uniform activations."""
    torch = _torch()
    c = synth.layer("gate_up")
    packed = bl.pack_ternary_weights(torch.from_numpy(c.w).cuda())
    n_copies = copies_for(packed.numel())
    copies = replicate(packed, n_copies)
    xq = torch.from_numpy(c.xq).cuda()
    s = torch.from_numpy(c.s).cuda()
    ws = bf16_dev(c.ws)
    y = torch.empty((1, c.N), dtype=torch.bfloat16, device="cuda")
    lib = bl.lib()
    args = [xq.data_ptr(), None, s.data_ptr(), ws.data_ptr(), c.ws_num, y.data_ptr(), None, 1,
            c.N, c.K]
    ptrs = [p.data_ptr() for p in copies]

    def launch(i):
        args[1] = ptrs[i % n_copies]
        rc = lib.bitlinear_i8xi2(*args, torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"bitlinear_i8xi2 failed: {rc}")

    ms = time_graph(launch, steps, warmup)
    return c, ms, n_copies, copies


def fused(bl, steps, warmup):
    """Same shape, bf16 activations quantised per token inside the kernel."""
    torch = _torch()
    c = synth.make_float_gemv("gate_up_bf16", 1, 13824, 2560, 2, synth.seed_for(6), bf16=True)
    packed = bl.pack_ternary_weights(torch.from_numpy(c.w).cuda())
    n_copies = copies_for(packed.numel())
    copies = replicate(packed, n_copies)
    x = bf16_dev(c.x)
    ws = bf16_dev(c.ws)
    y = torch.empty((1, c.N), dtype=torch.bfloat16, device="cuda")
    lib = bl.lib()
    ptrs = [p.data_ptr() for p in copies]

    def launch(i):
        rc = lib.bitlinear_bf16_i8xi2(x.data_ptr(), ptrs[i % n_copies], ws.data_ptr(), c.ws_num,
                                      y.data_ptr(), None, None, None, 1, c.N, c.K,
                                      torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"bitlinear_bf16_i8xi2 failed: {rc}")

    ms = time_graph(launch, steps, warmup)
    return ms


def layer_shapes(bl, steps, warmup, lut=False):
    """The int8 layer set through bitlinear_i8xi2, or through the table-lookup GEMV
    (bitlinear_lut_i8xi2, the cross-check algorithm) when lut is set."""
    torch = _torch()
    out = {}
    lib = bl.lib()
    for c in synth.layer_set():
        packed = bl.pack_ternary_weights(torch.from_numpy(c.w).cuda())
        n_copies = copies_for(packed.numel())
        copies = replicate(packed, n_copies)
        ptrs = [p.data_ptr() for p in copies]
        xq = torch.from_numpy(c.xq).cuda()
        s = torch.from_numpy(c.s).cuda()
        ws = bf16_dev(c.ws)
        y = torch.empty((1, c.N), dtype=torch.bfloat16, device="cuda")

        def launch(i, c=c, xq=xq, s=s, ws=ws, y=y, ptrs=ptrs, n_copies=n_copies):
            st = torch.cuda.current_stream().cuda_stream
            if lut:
                rc = lib.bitlinear_lut_i8xi2(xq.data_ptr(), ptrs[i % n_copies], s.data_ptr(),
                                             ws.data_ptr(), c.ws_num, y.data_ptr(), None, c.N,
                                             c.K, st)
            else:
                rc = lib.bitlinear_i8xi2(xq.data_ptr(), ptrs[i % n_copies], s.data_ptr(),
                                         ws.data_ptr(), c.ws_num, y.data_ptr(), None, 1, c.N, c.K,
                                         st)
            if rc != 0:
                raise RuntimeError(f"layer launch failed: {rc}")

        ms = time_graph(launch, steps, warmup)
        b = gemv_bytes(1, c.N, c.K, c.ws_num)
        out[f"{c.name}_{c.N}x{c.K}"] = {"us": round(ms * 1e3, 3),
                                        "GBps": round(b / (ms * 1e-3) / 1e9, 1)}
        del copies
    return out


def batched(bl, steps, warmup, ms=synth.BATCHED_M):
    torch = _torch()
    out = {}
    lib = bl.lib()
    for M in ms:
        c = synth.batched(M)
        packed = bl.pack_ternary_weights(torch.from_numpy(c.w).cuda())
        n_copies = copies_for(packed.numel())
        copies = replicate(packed, n_copies)
        ptrs = [p.data_ptr() for p in copies]
        q, s = bl.quantize_act_absmax_i8(torch.from_numpy(c.x).cuda())
        ws = bf16_dev(c.ws)
        y = torch.empty((M, c.N), dtype=torch.bfloat16, device="cuda")

        def launch(i, c=c, q=q, s=s, ws=ws, y=y, ptrs=ptrs, n_copies=n_copies, M=M):
            rc = lib.bitlinear_i8xi2(q.data_ptr(), ptrs[i % n_copies], s.data_ptr(), ws.data_ptr(),
                                     c.ws_num, y.data_ptr(), None, M, c.N, c.K,
                                     torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(f"bitlinear_i8xi2 failed: {rc}")

        ms = time_graph(launch, steps, warmup)
        b = gemv_bytes(M, c.N, c.K, c.ws_num)
        ops = 2.0 * M * c.N * c.K
        out[f"M{M}"] = {"us": round(ms * 1e3, 3), "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                        "mfma_util": round(ops / (ms * 1e-3) / (PEAK_INT8_TOPS * 1e12), 4)}
        del copies
    return out


def ternarize(bl, steps, warmup):
    """Weight ternarisation + packing of a bf16 13824 x 2560 matrix ([W2A8] §4.2): one call
    = exponent histogram, finalise, ternarise-and-pack.  Four rotating weight copies (283 MB)."""
    torch = _torch()
    N, K = 13824, 2560
    g = synth.rng(synth.seed_for(9, 1, 0))
    w = bf16_dev(synth.weights_bf16(g, N, K))
    copies = [w] + [w.clone() for _ in range(3)]
    packed = torch.empty(bl.bl_packed_bytes(N, K), dtype=torch.uint8, device="cuda")
    scales = torch.empty(3, dtype=torch.bfloat16, device="cuda")
    work = torch.empty(bl.TERNARIZE_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    lib = bl.lib()

    def launch(i):
        rc = lib.ternarize_weights_absmean(copies[i % 4].data_ptr(), packed.data_ptr(),
                                           scales.data_ptr(), work.data_ptr(), N, K,
                                           torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"ternarize_weights_absmean failed: {rc}")

    ms = time_graph(launch, steps, warmup)
    b = 2 * (2 * N * K) + N * K // 4 + 2048 + 6   # bf16 read twice, packed written
    return {"us": round(ms * 1e3, 3), "GBps": round(b / (ms * 1e-3) / 1e9, 1), "bytes": b}


def decode_step(bl, reps):
    """30 layers x {qkv, o, gate+up, down}, fused quantisation, one bl_graph per step."""
    torch = _torch()
    calls = []
    for c in synth.decode_step_nodes():
        calls.append(dict(x=bf16_dev(c.x), packed=bl.pack_ternary_weights(torch.from_numpy(c.w).cuda()),
                          ws=bf16_dev(c.ws), ws_num=c.ws_num,
                          y=torch.empty((c.N,), dtype=torch.bfloat16, device="cuda"),
                          N=c.N, K=c.K))
    nbytes = sum(gemv_bytes(1, c["N"], c["K"], c["ws_num"], x_bytes=2) for c in calls)
    g = bl.DecodeGraph(calls)
    for _ in range(3):
        g.launch()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        g.launch()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    g.close()
    return {"us_per_step": round(ms * 1e3, 2), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "bytes_per_step": nbytes, "gemvs_per_step": len(calls)}


def chained_step(bl, reps):
    """The decode step chained through its glue (readings of the norms and MLP activation the
    pages name): 30 layers x {qkv after attention_norm, o after attn_sub_norm + residual,
    gate+up after ffn_norm, down after relu(gate)^2 * up and ffn_sub_norm + residual}; one
    kernel per projection, one bl_graph per step.  The attention is out of scope: each layer's
    o reads a seeded attention output."""
    torch = _torch()
    dim, ffn = synth.DIM, synth.FFN
    h = [bf16_dev(synth.chained_h0())] + [torch.empty(dim, dtype=torch.bfloat16, device="cuda")
                                          for _ in range(synth.N_LAYERS)]
    calls, nbytes = [], 0
    for l in range(synth.N_LAYERS):
        L = synth.chained_layer(l)
        p = {k: bl.pack_ternary_weights(torch.from_numpy(v).cuda()) for k, v in L.w.items()}
        wsd = {k: bf16_dev(v) for k, v in L.ws.items()}
        gm = {k: bf16_dev(v) for k, v in L.gamma.items()}
        qkv = torch.empty(3840, dtype=torch.bfloat16, device="cuda")
        h1 = torch.empty(dim, dtype=torch.bfloat16, device="cuda")
        gu = torch.empty(2 * ffn, dtype=torch.bfloat16, device="cuda")
        calls += [
            dict(x=h[l], gamma=gm["attn"], packed=p["qkv"], ws=wsd["qkv"], ws_num=1, y=qkv,
                 N=3840, K=dim),
            dict(x=bf16_dev(L.attn_out), gamma=gm["attn_sub"], packed=p["o"], ws=wsd["o"], ws_num=1,
                 residual=h[l], y=h1, N=dim, K=dim),
            dict(x=h1, gamma=gm["ffn"], packed=p["gate_up"], ws=wsd["gate_up"], ws_num=2, y=gu,
                 N=2 * ffn, K=dim),
            dict(x=gu[:ffn], x_up=gu[ffn:], gamma=gm["ffn_sub"], packed=p["down"], ws=wsd["down"],
                 ws_num=1, residual=h1, y=h[l + 1], N=dim, K=ffn),
        ]
    for c in calls:
        # weights + scales + bf16 row (twice for the GLU) + its weight + output (+ residual)
        nbytes += gemv_bytes(1, c["N"], c["K"], c["ws_num"], x_bytes=2)
        nbytes += 2 * c["K"] * (2 if c.get("x_up") is not None else 1) - 2 * c["K"]
        nbytes += 2 * c["K"] + (2 * c["N"] if c.get("residual") is not None else 0)
    g = bl.ChainedDecodeGraph(calls)
    for _ in range(3):
        g.launch()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        g.launch()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    g.close()
    return {"us_per_step": round(ms * 1e3, 2), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "bytes_per_step": nbytes, "projections_per_step": len(calls)}


def torch_bf16_context(steps):
    """The page's comparison column: torch bf16 matmul, 1 x 2560 by 2560 x 13824, weights rotated."""
    torch = _torch()
    g = torch.Generator(device="cuda").manual_seed(1)
    n_copies = copies_for(13824 * 2560 * 2)
    ws = [torch.randn((13824, 2560), device="cuda", dtype=torch.bfloat16, generator=g)
          for _ in range(n_copies)]
    x = torch.randn((1, 2560), device="cuda", dtype=torch.bfloat16, generator=g)
    outs = torch.empty((1, 13824), device="cuda", dtype=torch.bfloat16)

    def launch(i):
        torch.matmul(x, ws[i % n_copies].t(), out=outs)

    ms = time_graph(launch, steps, 16)
    return {"us": round(ms * 1e3, 3)}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands
# ---------------------------------------------------------------------------

def cpu_baseline(seconds):
    import oracle
    c = synth.layer("gate_up")
    oracle.bitlinear_i8(c.xq, c.w, c.s, c.ws, c.ws_num)     # load + warm
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.bitlinear_i8(c.xq, c.w, c.s, c.ws, c.ws_num)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per = el / n
    b = gemv_bytes(1, c.N, c.K, c.ws_num)
    return {"value": round(b / per / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "us_per_gemv": round(per * 1e6, 1),
            "sample": f"{n} full M=1 GEMVs at N=13824 K=2560 (int8 x, unpacked ternary w, int64 "
                      f"sums, fp64 epilogue), single-threaded C, {el:.1f} s"}


def gemv_source_sha256():
    h = hashlib.sha256()
    for f in GEMV_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def pmc_traffic():
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it is for this kernel source."""
    if not os.path.exists(PROFILE_PMC):
        return None
    vals = {}
    for line in open(PROFILE_PMC):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("gemv_source_sha256") != gemv_source_sha256() or "traffic_bytes_per_launch" not in vals:
        return None
    return float(vals["traffic_bytes_per_launch"])


def gemv_geometry(N, K):
    """(bands per workgroup, wavefronts per workgroup, K-steps per wavefront) of the library's
    M=1 GEMV for this shape (the same rule as gemv_shape in bit_gemv_bitlinear_amd/csrc/gemv.hip)."""
    S = -(-K // 256)
    nbands = -(-N // 16)
    target = 4 if nbands < 400 else 5 if nbands < 768 else 10
    Wb = 1
    while Wb < 16 and -(-S // Wb) > target:
        Wb *= 2
    while Wb > 8 and -(-S // (Wb // 2)) <= 15:
        Wb //= 2
    P = -(-S // Wb)
    B = 4
    while B > 1 and (nbands // B < 200 or B * Wb > 16):
        B //= 2
    return B, B * Wb, P


def stream_floor(copies, N, K, steps, warmup):
    """Same launch shape and bytes as the GEMV: an empty launch and a pure streaming read."""
    import ctypes
    torch = _torch()
    lib = ctypes.CDLL(PROBE_LIB)
    P_ = ctypes.c_void_p
    I_ = ctypes.c_int
    lib.stream_floor_empty.argtypes = [I_, I_, P_, P_]
    lib.stream_floor_read.argtypes = [P_, I_, I_, I_, I_, I_, P_, P_]
    nbands, S = -(-N // 16), -(-K // 256)
    B, W, P = gemv_geometry(N, K)
    groups = -(-nbands // B)
    out = torch.zeros(groups, dtype=torch.int32, device="cuda")
    ptrs = [c.data_ptr() for c in copies]

    def empty(i):
        if lib.stream_floor_empty(groups, W, out.data_ptr(), torch.cuda.current_stream().cuda_stream):
            raise RuntimeError("stream_floor_empty failed")

    def read(i):
        if lib.stream_floor_read(ptrs[i % len(ptrs)], nbands, S, B, W, P, out.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream):
            raise RuntimeError("stream_floor_read failed")

    e_ms = time_graph(empty, steps, warmup)
    r_ms = time_graph(read, steps, warmup)
    nbytes = nbands * S * 1024
    return {"launch_shape": f"{groups} workgroups x {W} wavefronts ({B} bands), {P} 16-byte loads per lane",
            "empty_launch_us": round(e_ms * 1e3, 3), "stream_read_us": round(r_ms * 1e3, 3),
            "stream_read_GBps": round(nbytes / (r_ms * 1e-3) / 1e9, 1)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--quick", action="store_true", help="headline only")
    ap.add_argument("--sections",
                    default="fused,layer_set,lut,batched,prefill,decode_step,chained_step,ternarize,torch",
                    help="detail sections to run after the headline (comma list; for profiling one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--pmc-calibrate", action="store_true",
                    help="also run a plain copy of 256 MiB (for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is not sharded across GPUs in this build)", file=sys.stderr)
        sys.exit(2)

    torch = _torch()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import bit_gemv_bitlinear_amd as bl

    c, ms, n_copies, copies = headline(bl, args.steps, args.warmup)
    nbytes = gemv_bytes(1, c.N, c.K, c.ws_num)
    gbs = nbytes / (ms * 1e-3) / 1e9
    detail = {}
    if os.path.exists(PROBE_LIB) and not args.pmc_calibrate:
        fl = stream_floor(copies, c.N, c.K, args.steps, args.warmup)
        fl["gemv_us_over_stream_read_us"] = round(ms * 1e3 / fl["stream_read_us"], 3)
        detail["single_launch_floor_13824x2560"] = fl
    del copies
    if args.pmc_calibrate:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        detail["calibration_copy_bytes"] = 256 << 20
    sections = set() if args.quick else set(args.sections.split(","))
    if "fused" in sections:
        fms = fused(bl, max(args.steps // 2, 100), min(args.warmup, 100))
        fb = gemv_bytes(1, 13824, 2560, 2, x_bytes=2)
        detail["fused_bf16_13824x2560"] = {"us": round(fms * 1e3, 3),
                                           "GBps": round(fb / (fms * 1e-3) / 1e9, 1)}
    if "layer_set" in sections:
        detail["layer_set_int8"] = layer_shapes(bl, max(args.steps // 4, 100), 50)
    if "lut" in sections:
        detail["layer_set_int8_lut"] = layer_shapes(bl, max(args.steps // 4, 100), 50, lut=True)
    if "batched" in sections:
        detail["batched_mfma"] = batched(bl, max(args.steps // 8, 50), 20)
    if "prefill" in sections:
        detail["prefill_13824x2560"] = batched(bl, 50, 10, synth.PREFILL_M)
    if "decode_step" in sections:
        detail["decode_step_graph"] = decode_step(bl, 20)
    if "chained_step" in sections:
        detail["chained_decode_step_graph"] = chained_step(bl, 20)
    if "ternarize" in sections:
        detail["ternarize_pack_bf16_13824x2560"] = ternarize(bl, 50, 10)
    if "torch" in sections:
        detail["torch_bf16_matmul_13824x2560"] = torch_bf16_context(200)

    traffic = pmc_traffic()
    line = {
        "metric": "M=1 W2A8 GEMV µs + achieved HBM GB/s (% of peak) at N=13824,K=2560",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "us_per_gemv": round(ms * 1e3, 3),
        "pct_of_peak_hbm": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(gbs / A100_W2A8_GBS_13824x2560, 3),
        "vs_baseline_note": "context only: the page's A100 kernel, host-timed 18.75 us = 473.5 GB/s",
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "M=1 W2A8 GEMV N=13824 K=2560 (gate+up of a 2B-style layer), "
                               "uniform ternary weights, uniform int8 activations, ws_num=2",
                   "M": 1, "N": c.N, "K": c.K, "ws_num": c.ws_num,
                   "bytes_per_gemv": nbytes, "weight_copies": n_copies,
                   "timing": "one HIP graph of `steps` launches after one untimed replay of it, HIP events on its stream"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic},
    }
    if detail:
        line["detail"] = detail
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
