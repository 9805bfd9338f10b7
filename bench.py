#!/usr/bin/env python3
"""Benchmark of the W2A8 ternary linear layer on one MI355X.

Headline: the M = 1 GEMV (int8 activations x packed ternary weights -> bf16)
at N = 13824, K = 2560 (the fused gate+up projection of the 2B-style model
in the W2A8 page, "BitNet GPU 推理框架：从零构建 W2A8 的 2-bit 大模型 CUDA GEMV
内核", §一 and §7.1), reported as microseconds per GEMV and achieved HBM
GB/s against MI355X's 8 TB/s.

Method (the same for every launch-per-step workload):
  * inputs are seeded synthetic data of the page's shapes (module ``synth``),
    resident in HBM before timing starts;
  * the packed weights are replicated into n >= 2 copies of >= 512 MiB in
    total, and every launch -- warm-up, untimed and timed alike -- reads the
    next copy of one continuing rotation: a timed launch's weights were last
    read n launches (>= 512 MiB of other weights) earlier, so neither the
    256 MiB Infinity Cache nor the 4 MiB L2s hold them;
  * K = --steps launches are captured in one HIP graph and 2K in another;
    each timed replay is preceded by an untimed prefix graph of 2n launches
    (the GPU is busy with it while the host submits the timed graph, so
    submission falls outside the timed region) and bracketed by HIP events
    recorded on the stream the graphs run on;
  * per launch = median over repetitions of (t(2K) - t(K)) / K: whatever a
    replay costs once (the events, the graph's first packet) cancels; the
    direct t(K) / K is reported beside it;
  * bytes per GEMV = N*K/4 (packed weights) + M*K (int8 x) + 2*M*N (bf16 y)
    + 4*M (s) + 2*ws_num (ws) -- the algorithmic bytes, each read once.

Prints one JSON line.  ``--gpus`` above 1 is refused: the layer runs on one GPU.
"""
import argparse
import hashlib
import json
import os
import statistics
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


def reps_for(steps):
    """Timed repetitions: enough that a short --steps still gives a steady median."""
    return max(5, min(41, -(-20000 // max(steps, 1))))


def _capture(launch, first, count):
    torch = _torch()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(first, first + count):
            launch(i)
    return g


def time_launches(launch, n_copies, steps, warmup):
    """Per-launch time in ms of launch(i) (launch i reads weight copy i % n_copies).

    Graphs of `steps` and 2 * `steps` launches, each replay after an untimed prefix graph of
    2 * n_copies launches; both start at copy 0, which the prefix last read n_copies launches
    before its end, so the rotation never breaks.  Returns (slope, direct, detail)."""
    torch = _torch()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(max(warmup, 1)):
            launch(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    L = steps
    pre = _capture(launch, 0, 2 * n_copies)
    g1 = _capture(launch, 0, L)
    g2 = _capture(launch, 0, 2 * L)
    for g in (pre, g1, pre, g2, pre):       # a graph's first replay runs slower
        g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    slopes, direct, pre_ms, host_ms = [], [], [], []
    for _ in range(reps_for(L)):
        torch.cuda.synchronize()
        ev[0].record()
        pre.replay()
        ev[1].record()
        h0 = time.perf_counter()
        g1.replay()
        h1 = time.perf_counter()
        ev[2].record()
        pre.replay()
        ev[3].record()
        g2.replay()
        ev[4].record()
        torch.cuda.synchronize()
        t1 = ev[1].elapsed_time(ev[2])
        t2 = ev[3].elapsed_time(ev[4])
        slopes.append((t2 - t1) / L)
        direct.append(t1 / L)
        pre_ms.append(ev[0].elapsed_time(ev[1]))
        host_ms.append((h1 - h0) * 1e3)
    slope = statistics.median(slopes)
    d = statistics.median(direct)
    detail = {"reps": len(slopes), "direct_us": round(d * 1e3, 3),
              "prefix_gpu_ms": round(statistics.median(pre_ms), 3),
              "host_submit_ms": round(statistics.median(host_ms), 3)}
    return slope, d, detail


def time_replays(replay, reps):
    """Per-replay ms of a whole-step graph: (t(2R) - t(R)) / R, each after untimed replays."""
    torch = _torch()
    for _ in range(3):
        replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    out = []
    for _ in range(5):
        torch.cuda.synchronize()
        replay()                            # untimed: busy while the timed replays are submitted
        ev[0].record()
        for _ in range(reps):
            replay()
        ev[1].record()
        replay()
        ev[2].record()
        for _ in range(2 * reps):
            replay()
        ev[3].record()
        torch.cuda.synchronize()
        out.append((ev[2].elapsed_time(ev[3]) - ev[0].elapsed_time(ev[1])) / reps)
    return statistics.median(out)


def rotating_layer(bl, c, steps, warmup, lut=False):
    """Time bitlinear_i8xi2 (or the table-lookup GEMV) on int8 instance c with rotating weights."""
    torch = _torch()
    packed = bl.pack_ternary_weights(torch.from_numpy(c.w).cuda())
    n_copies = copies_for(packed.numel())
    copies = replicate(packed, n_copies)
    ptrs = [p.data_ptr() for p in copies]
    xq = torch.from_numpy(np.ascontiguousarray(c.xq)).cuda()
    s = torch.from_numpy(c.s).cuda()
    ws = bf16_dev(c.ws)
    y = torch.empty((c.M, c.N), dtype=torch.bfloat16, device="cuda")
    lib = bl.lib()

    def launch(i):
        st = torch.cuda.current_stream().cuda_stream
        if lut:
            rc = lib.bitlinear_lut_i8xi2(xq.data_ptr(), ptrs[i % n_copies], s.data_ptr(),
                                         ws.data_ptr(), c.ws_num, y.data_ptr(), None, c.N, c.K, st)
        else:
            rc = lib.bitlinear_i8xi2(xq.data_ptr(), ptrs[i % n_copies], s.data_ptr(), ws.data_ptr(),
                                     c.ws_num, y.data_ptr(), None, c.M, c.N, c.K, st)
        if rc != 0:
            raise RuntimeError(f"layer launch failed: {rc}")

    slope, direct, detail = time_launches(launch, n_copies, steps, warmup)
    detail["weight_copies"] = n_copies
    del copies
    return slope, direct, detail


def gemv_entry(ms, nbytes, extra=None):
    e = {"us": round(ms * 1e3, 3), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
         "pct_of_peak_hbm": round(100.0 * nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 1)}
    if extra:
        e.update(extra)
    return e


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def headline(bl, steps, warmup):
    """M=1 GEMV, N=13824, K=2560, ws_num=2, int8 uniform activations."""
    c = synth.layer("gate_up")
    slope, direct, detail = rotating_layer(bl, c, steps, warmup)
    return c, slope, detail


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

    slope, _, _ = time_launches(launch, n_copies, steps, warmup)
    return gemv_entry(slope, gemv_bytes(1, 13824, 2560, 2, x_bytes=2))


def layer_shapes(bl, steps, warmup, lut=False):
    """The int8 layer set through bitlinear_i8xi2, or through the table-lookup GEMV
    (bitlinear_lut_i8xi2, the cross-check algorithm) when lut is set."""
    out = {}
    for c in synth.layer_set():
        slope, _, _ = rotating_layer(bl, c, steps, warmup, lut=lut)
        out[f"{c.name}_{c.N}x{c.K}"] = gemv_entry(slope, gemv_bytes(1, c.N, c.K, c.ws_num))
    return out


def large_shapes(bl, steps, warmup):
    """The large M=1 shapes (55296x5120, 13824x5120, 5120x13824): sparse ternary weights
    (P(0) = 1/2), activations quantised from x ~ N(0, 1) by the device quantiser."""
    torch = _torch()
    out = {}
    for cf in synth.large_set():
        q, s = bl.quantize_act_absmax_i8(torch.from_numpy(cf.x).cuda())
        torch.cuda.synchronize()
        c = synth.Gemv(cf.name, 1, cf.N, cf.K, cf.ws_num, cf.w, q.cpu().numpy(), s.cpu().numpy(),
                       cf.ws)
        slope, _, detail = rotating_layer(bl, c, steps, warmup)
        out[f"{cf.N}x{cf.K}"] = gemv_entry(slope, gemv_bytes(1, cf.N, cf.K, cf.ws_num),
                                           {"weight_copies": detail["weight_copies"]})
    return out


def batched(bl, steps, warmup, ms=synth.BATCHED_M):
    torch = _torch()
    out = {}
    for M in ms:
        cf = synth.batched(M)
        q, s = bl.quantize_act_absmax_i8(torch.from_numpy(cf.x).cuda())
        torch.cuda.synchronize()
        c = synth.Gemv(cf.name, M, cf.N, cf.K, cf.ws_num, cf.w, q.cpu().numpy(), s.cpu().numpy(),
                       cf.ws)
        slope, _, _ = rotating_layer(bl, c, steps, warmup)
        ops = 2.0 * M * c.N * c.K
        out[f"M{M}"] = gemv_entry(slope, gemv_bytes(M, c.N, c.K, c.ws_num),
                                  {"mfma_util": round(ops / (slope * 1e-3) / (PEAK_INT8_TOPS * 1e12), 4)})
    return out


def ternarize(bl, steps, warmup):
    """Weight ternarisation + packing of a bf16 13824 x 2560 matrix ([W2A8] §4.2): one call
    = exponent histogram, finalise, ternarise-and-pack.  Rotating bf16 weight copies."""
    torch = _torch()
    N, K = 13824, 2560
    g = synth.rng(synth.seed_for(9, 1, 0))
    w = bf16_dev(synth.weights_bf16(g, N, K))
    n_copies = copies_for(2 * N * K)
    copies = [w] + [w.clone() for _ in range(n_copies - 1)]
    packed = torch.empty(bl.bl_packed_bytes(N, K), dtype=torch.uint8, device="cuda")
    scales = torch.empty(3, dtype=torch.bfloat16, device="cuda")
    work = torch.empty(bl.TERNARIZE_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    lib = bl.lib()

    def launch(i):
        rc = lib.ternarize_weights_absmean(copies[i % n_copies].data_ptr(), packed.data_ptr(),
                                           scales.data_ptr(), work.data_ptr(), N, K,
                                           torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"ternarize_weights_absmean failed: {rc}")

    slope, _, _ = time_launches(launch, n_copies, steps, warmup)
    b = 2 * (2 * N * K) + N * K // 4 + 2048 + 6   # bf16 read twice, packed written
    del copies
    return {"us": round(slope * 1e3, 3), "GBps": round(b / (slope * 1e-3) / 1e9, 1), "bytes": b}


def decode_step(bl):
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
    ms = time_replays(g.launch, 10)
    kernels = g.kernels
    g.close()
    return {"us_per_step": round(ms * 1e3, 2), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "pct_of_peak_hbm": round(100.0 * nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 1),
            "bytes_per_step": nbytes, "gemvs_per_step": len(calls), "kernels_per_step": kernels}


def chained_step(bl):
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
    ms = time_replays(g.launch, 10)
    kernels, linked = g.kernels, g.linked
    g.close()
    return {"us_per_step": round(ms * 1e3, 2), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "bytes_per_step": nbytes, "projections_per_step": len(calls),
            "kernels_per_step": kernels, "hand_offs_per_step": linked}


def dispatch_probe(bl, n=400, sleep_cycles=400_000_000):
    """The headline GEMV launched n times straight onto the stream while the GPU is held by a
    sleep kernel (torch.cuda._sleep, a bounded spin): the launches queue up and then run back to
    back even where submitting each one is slow (under a kernel-tracing profiler).  HIP events
    bracket the n launches after the sleep.  Opt-in (``--sections dispatch_probe``): run under
    ``rocprofv3 --kernel-trace``, the same process then gives both the profiler's per-dispatch
    durations of these n back-to-back launches (the last n dispatches of the GEMV kernel) and
    the events' per-launch time, which can be compared; without the profiler it gives the
    per-launch time of direct (non-graph) launches."""
    torch = _torch()
    c = synth.layer("gate_up")
    packed = bl.pack_ternary_weights(torch.from_numpy(c.w).cuda())
    n_copies = copies_for(packed.numel())
    copies = replicate(packed, n_copies)
    ptrs = [p.data_ptr() for p in copies]
    xq = torch.from_numpy(np.ascontiguousarray(c.xq)).cuda()
    s = torch.from_numpy(c.s).cuda()
    ws = bf16_dev(c.ws)
    y = torch.empty((1, c.N), dtype=torch.bfloat16, device="cuda")
    lib = bl.lib()
    st = torch.cuda.current_stream()

    def launch(i):
        rc = lib.bitlinear_i8xi2(xq.data_ptr(), ptrs[i % n_copies], s.data_ptr(), ws.data_ptr(),
                                 c.ws_num, y.data_ptr(), None, 1, c.N, c.K, st.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"layer launch failed: {rc}")

    for i in range(2 * n_copies):
        launch(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    torch.cuda._sleep(sleep_cycles)
    ev[1].record()
    h0 = time.perf_counter()
    for i in range(n):
        launch(i)
    h1 = time.perf_counter()
    ev[2].record()
    torch.cuda.synchronize()
    sleep_ms = ev[0].elapsed_time(ev[1])
    run_ms = ev[1].elapsed_time(ev[2])
    submit_ms = (h1 - h0) * 1e3
    del copies
    return {"launches": n, "us_per_launch": round(run_ms / n * 1e3, 3),
            "sleep_ms": round(sleep_ms, 3), "host_submit_ms": round(submit_ms, 3),
            "queued_before_sleep_ended": submit_ms < sleep_ms}


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

    slope, _, _ = time_launches(launch, n_copies, steps, 16)
    return {"us": round(slope * 1e3, 3)}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands
# ---------------------------------------------------------------------------

def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads():
    """Threads for the all-cores leg: the cores this process may run on, within the
    OMP_NUM_THREADS share when one is set."""
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(n, 1)


def _oracle_gemv_threads(c, threads):
    """One full GEMV as `threads` slices of rows, each an unchanged oracle call (the oracle's C
    runs without the interpreter lock, so the slices run in parallel).  Slices stay inside
    one weight-scale segment."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    seg = c.N // c.ws_num
    per_seg = max(1, threads // c.ws_num)
    parts = []
    for sgi in range(c.ws_num):
        bounds = np.linspace(sgi * seg, (sgi + 1) * seg, per_seg + 1).astype(int)
        for a, b in zip(bounds[:-1], bounds[1:]):
            parts.append((a, b, c.ws[sgi:sgi + 1]))
    ex = ThreadPoolExecutor(max_workers=threads)

    def one(p):
        a, b, ws = p
        return oracle.bitlinear_i8(c.xq, c.w[a:b], c.s, ws, 1)

    def run():
        return list(ex.map(one, parts))
    return run, ex, parts


def cpu_baseline(seconds):
    import oracle
    c = synth.layer("gate_up")
    b = gemv_bytes(1, c.N, c.K, c.ws_num)
    oracle.bitlinear_i8(c.xq, c.w, c.s, c.ws, c.ws_num)     # load + warm

    def timed(fn):
        n, t0 = 0, time.perf_counter()
        while True:
            fn()
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return el / n, n, el

    per1, n1, el1 = timed(lambda: oracle.bitlinear_i8(c.xq, c.w, c.s, c.ws, c.ws_num))
    threads = host_threads()
    run, ex, parts = _oracle_gemv_threads(c, threads)
    # the slices together are the whole GEMV: same int32 sums and bf16 outputs
    whole = oracle.bitlinear_i8(c.xq, c.w, c.s, c.ws, c.ws_num)[1].reshape(-1)
    got = np.concatenate([r[1].reshape(-1) for r in run()])
    if not np.array_equal(got, whole):
        raise RuntimeError("threaded oracle slices disagree with the whole oracle GEMV")
    perT, nT, elT = timed(run)
    ex.shutdown()
    return {"value": round(b / perT / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "us_per_gemv": round(perT * 1e6, 1),
            "host_cpu": host_cpu_model(), "host_cpus_available": os.cpu_count(),
            "sample": f"{nT} full M=1 GEMVs at N=13824 K=2560 in {elT:.1f} s, each as {len(parts)} "
                      f"row slices on {threads} threads (the unchanged single-threaded C oracle per "
                      f"slice: int8 x, unpacked ternary w, int64 sums, fp64 epilogue)",
            "single_core": {"value": round(b / per1 / 1e9, 3), "unit": "GB/s",
                            "us_per_gemv": round(per1 * 1e6, 1),
                            "sample": f"{n1} full GEMVs, one thread, {el1:.1f} s"}}


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


def summarize_profile(path, tail=400):
    """Print, for every rocpd database under path: per kernel, the dispatches and their
    durations (ns: mean, median, p10, p90, min) and the median start-to-start period; the same
    for the last `tail` dispatches of each kernel with at least 2 * tail of them (the dispatch
    probe's back-to-back launches, when that section ran last); and per kernel and counter, the
    mean and median value per dispatch and the five largest (the calibration copies are the
    largest dispatches of the runtime's copy kernel)."""
    import glob
    import sqlite3
    dbs = sorted(glob.glob(os.path.join(path, "**", "*.db"), recursive=True))
    if not dbs:
        print(f"no rocpd database under {path}", file=sys.stderr)
        sys.exit(1)

    def stats(ev):
        d = sorted(e - b for b, e in ev)
        per = sorted(ev[i + 1][0] - ev[i][0] for i in range(len(ev) - 1)) or [0]
        k = len(d)
        return (f"{k} | {statistics.mean(d):.1f} | {d[k // 2]} | {d[k // 10]} | {d[9 * k // 10]} | "
                f"{d[0]} | {per[len(per) // 2]}")

    for dbp in dbs:
        db = sqlite3.connect(dbp)
        cur = db.cursor()
        print(f"# database {os.path.relpath(dbp, path)}")
        by = {}
        for name, b, e in cur.execute("select name, start, end from kernels order by start"):
            by.setdefault(name, []).append((b, e))
        print("## kernel | dispatches | mean ns | median | p10 | p90 | min | median period")
        for name, ev in sorted(by.items(), key=lambda kv: -sum(e - b for b, e in kv[1])):
            print(f"{name[:160]} | {stats(ev)}")
        for name, ev in by.items():
            if len(ev) >= 2 * tail:
                print(f"## last {tail} dispatches: {name[:160]} | {stats(ev[-tail:])}")
        try:
            rows = list(cur.execute(
                "select kernel_name, counter_name, value from counters_collection"))
        except sqlite3.Error:
            rows = []
        if rows:
            agg = {}
            for kn, cn, v in rows:
                agg.setdefault((kn, cn), []).append(v)
            print("## kernel | counter | dispatches | mean per dispatch | median | largest five")
            for (kn, cn), vs in sorted(agg.items()):
                vs.sort()
                top = ", ".join(f"{v:.1f}" for v in vs[-5:][::-1])
                print(f"{kn[:160]} | {cn} | {len(vs)} | {statistics.mean(vs):.3f} | "
                      f"{vs[len(vs) // 2]:.3f} | {top}")


ALL_SECTIONS = "fused,layer_set,large,lut,batched,prefill,decode_step,chained_step,ternarize,torch"


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--quick", action="store_true", help="headline only")
    ap.add_argument("--sections", default=ALL_SECTIONS,
                    help="detail sections to run after the headline (comma list; for profiling one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--pmc-calibrate", action="store_true",
                    help="also run a plain copy of 256 MiB (for counter calibration)")
    ap.add_argument("--summarize", metavar="DIR",
                    help="summarise the rocprofv3 databases (*.db) under DIR and exit")
    args = ap.parse_args()
    if args.summarize:
        summarize_profile(args.summarize)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the layer runs on one GPU and is not sharded across GPUs)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        print("--steps must be at least 1", file=sys.stderr)
        sys.exit(2)

    torch = _torch()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import bit_gemv_bitlinear_amd as bl

    c, ms, hdetail = headline(bl, args.steps, args.warmup)
    nbytes = gemv_bytes(1, c.N, c.K, c.ws_num)
    gbs = nbytes / (ms * 1e-3) / 1e9
    detail = {}
    if args.pmc_calibrate:
        # five plain device-to-device copies of 256 MiB through the HIP runtime (its blit
        # kernel): a copy of known size for scaling the memory-traffic counters
        import ctypes
        hip = ctypes.CDLL("libamdhip64.so")
        hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_int, ctypes.c_void_p]
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            rc = hip.hipMemcpyAsync(dst.data_ptr(), src.data_ptr(), 256 << 20, 3,   # device to device
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if rc != 0:
                raise RuntimeError(f"hipMemcpyAsync failed: {rc}")
        torch.cuda.synchronize()
        detail["calibration_copy_bytes"] = 256 << 20
    sections = set() if args.quick else set(args.sections.split(","))
    short = min(args.steps, 400)
    if "fused" in sections:
        detail["fused_bf16_13824x2560"] = fused(bl, short, 20)
    if "layer_set" in sections:
        detail["layer_set_int8"] = layer_shapes(bl, short, 20)
    if "large" in sections:
        detail["large_int8"] = large_shapes(bl, min(args.steps, 100), 10)
    if "lut" in sections:
        detail["layer_set_int8_lut"] = layer_shapes(bl, short, 20, lut=True)
    if "batched" in sections:
        detail["batched_mfma"] = batched(bl, short, 20)
    if "prefill" in sections:
        detail["prefill_13824x2560"] = batched(bl, min(args.steps, 100), 10, synth.PREFILL_M)
    if "decode_step" in sections:
        detail["decode_step_graph"] = decode_step(bl)
    if "chained_step" in sections:
        detail["chained_decode_step_graph"] = chained_step(bl)
    if "ternarize" in sections:
        detail["ternarize_pack_bf16_13824x2560"] = ternarize(bl, min(args.steps, 50), 5)
    if "torch" in sections:
        detail["torch_bf16_matmul_13824x2560"] = torch_bf16_context(min(args.steps, 200))
    if "dispatch_probe" in sections:       # last: its launches are the GEMV kernel's last n
        detail["dispatch_probe_13824x2560"] = dispatch_probe(bl)

    traffic = pmc_traffic()
    B, W, P = gemv_geometry(c.N, c.K)
    groups = -(-(-(-c.N // 16)) // B)        # ceil(ceil(N / 16) / B)
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
                   "bytes_per_gemv": nbytes, "weight_copies": hdetail["weight_copies"],
                   "launch": f"{groups} workgroups x {W} wavefronts, "
                             f"{P} K-steps per wavefront",
                   "timing": "per launch = median over reps of (t(2*steps) - t(steps)) / steps, "
                             "graphs of steps and 2*steps launches each after an untimed prefix of "
                             "2*copies launches, HIP events on the graphs' stream; every launch "
                             "reads the next weight copy of one rotation",
                   "timing_detail": hdetail},
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
