#!/usr/bin/env python3
"""Benchmark of the Hedgehog causal linear-attention forward (feature map included).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = one hh_linattn_fwd call over one batch of synthetic input (all
kernels of the path: feature maps, intra-chunk products, state carry,
read-out).  Inputs, outputs and workspace are resident in HBM before the
timed region; steps rotate over 4 input sets (about 670 MB for the default
workload, more than twice the 256 MB MALL) so repeated steps do not run out
of the last-level cache.  Before the warm-up steps the step is replayed,
untimed, for CLOCK_SETTLE_S seconds so that the device has raised its clocks
(the timed steps then see the steady state of a busy GPU).  Prints one JSON
line.

Default workload: Llama-2-7B head shapes, B=1, H=32, N=4096, d=128, bf16
(the configuration the throughput metric is quoted on).  Other workloads can
be selected for measurement with --workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from softmax_mimicking_feature_amd import workloads as wl  # noqa: E402

PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
PEAK_MFMA_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
N_SETS = 4
GRAPH_STEPS = 20                 # calls per captured graph (a multiple of N_SETS)
CLOCK_SETTLE_S = 0.3             # untimed replays before the warm-up steps (clock ramp)
METRIC = "causal linear-attn fwd tokens/s (\u03c6 incl.) at Llama-2-7B heads; % MFMA peak"


def algorithmic_counts(w: wl.Workload):
    """Algorithmic FLOPs and HBM bytes of one forward (what the method itself must do).

    Per token-head: feature maps of q and k 4d^2 (Hedgehog; Taylor 2(d^2+d)), state update
    and read-out 4 d' d, normaliser update / dot / divide 3d' + d.  Bytes: read q, k, v and
    write y once, plus W and b once per head."""
    d, dp = w.d, wl.feature_dim(w.map, w.d)
    th = w.B * w.H * w.N
    fm = 2 * (d * d + d) if w.map == wl.MAP_TAYLOR2 else 4 * d * d
    flops = th * (fm + 4 * dp * d + 3 * dp + d)
    eb = wl.bytes_per_elem(w.dtype)
    byts = eb * 4 * th * d
    if w.map != wl.MAP_TAYLOR2:
        byts += eb * w.H * (d * d + (d if wl.map_has_bias(w.map) else 0))
    return float(flops), float(byts)


def distill_counts(w: wl.Workload):
    """Algorithmic FLOPs and HBM bytes of one distillation loss (Eq. 4).

    Per (query, key) pair with j <= i: the logit q.k (2d) and the linear weight phi(q).phi(k)
    (2d'); per token-head the feature maps of q and k (4d^2).  Bytes: read q and k, write one fp32
    loss per query, plus W and b once per head."""
    d, dp = w.d, wl.feature_dim(w.map, w.d)
    th = w.B * w.H * w.N
    pairs = w.B * w.H * w.N * (w.N + 1) // 2
    flops = pairs * (2 * d + 2 * dp) + th * 4 * d * d
    eb = wl.bytes_per_elem(w.dtype)
    byts = eb * 2 * th * d + 4 * th + eb * w.H * (d * d + d)
    return float(flops), float(byts)


def backward_counts(w: wl.Workload):
    """Algorithmic FLOPs and HBM bytes of one backward.

    Per token-head: the feature maps of q and k again (4d^2), dL/dphi(q) = S g + c z (2 d' d),
    dL/dphi(k) = R v + r and dL/dv = R^T phi(k) (4 d' d), the map's backward dq, dk = W^T du
    (4d^2) and dW = sum du x^T (4d^2), plus O(d') for den, c and the normalisers.  Bytes: read
    q, k, v, y, dy and write dq, dk, dv once, plus W, b and the fp32 dW, db once per head."""
    d, dp = w.d, wl.feature_dim(w.map, w.d)
    th = w.B * w.H * w.N
    flops = th * (12 * d * d + 6 * dp * d + 4 * dp)
    eb = wl.bytes_per_elem(w.dtype)
    byts = eb * 8 * th * d + (eb + 4) * w.H * (d * d + d)
    return float(flops), float(byts)


def decode_counts(w: wl.Workload):
    d, dp = w.d, wl.feature_dim(w.map, w.d)
    bh = w.B * w.H
    eb = wl.bytes_per_elem(w.dtype)
    byts = 2 * 4 * bh * (dp * d + dp) + eb * 4 * bh * d + eb * w.H * (d * d + d)
    fm = 4 * d * d if w.map == wl.MAP_HEDGEHOG else 2 * (d * d + d)
    flops = bh * (fm + 4 * dp * d + 3 * dp + d)
    return float(flops), float(byts)


def source_digest() -> str:
    """sha256 over the kernel and C-ABI sources: ties recorded counter figures to the code they
    were taken on."""
    csrc = os.path.join(ROOT, "softmax_mimicking_feature_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".cpp", ".h")):
            h.update(f.encode())
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, entry: str):
    """L2-miss bytes per call (read + written, from the TCC request-size counters) in the committed
    counter summary of this workload, or None when there is none or the kernels changed since it
    was taken."""
    path = os.path.join(ROOT, "profiles", f"{entry}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_call: (\d+) sources: ([0-9a-f]+)", text)
    if not m or m.group(2) != source_digest():
        return None
    return int(m.group(1))


def host_cpu_model() -> str:
    """Model name of the host CPU (from /proc/cpuinfo), for the CPU-baseline record."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_calibration(nbytes: int = 1 << 30, reps: int = 5):
    """A plain device-to-device copy of known size, profiled to scale the HBM byte counters."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": nbytes, "bytes_written": nbytes, "reps": reps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c3_llama2_causal", choices=sorted(wl.CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle", type=float, default=CLOCK_SETTLE_S,
                    help="seconds of untimed replays before the warm-up steps (0 for profiling runs)")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step from Python instead of replaying captured HIP graphs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (the path shards over "
              "(batch, head) pairs with no communication)", file=sys.stderr)
        sys.exit(2)

    import torch
    import softmax_mimicking_feature_amd as hh

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    w = wl.CONFIGS[args.workload]
    tdt = torch.bfloat16 if w.dtype == wl.DT_BF16 else torch.float32
    decode = args.workload.endswith("decode")
    distill = args.workload.endswith("distill")
    backward = args.workload.endswith("backward")

    # ---- input sets (set 0 from the seeded host generator, the others drawn on the GPU
    #      with the same distributions)
    host0 = wl.make_inputs(w) if not decode else None
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)

    def draw(shape, scale):
        return (torch.randn(shape, generator=g, device=dev) * scale).to(tdt)

    sets = []
    for si in range(N_SETS):
        if decode:
            shp = (w.B, w.H, w.d)
            s = {"q": draw(shp, w.qk_scale), "k": draw(shp, w.qk_scale), "v": draw(shp, w.v_scale)}
        elif si == 0:
            s = {k: torch.from_numpy(host0[k]).to(dev).to(tdt) for k in ("q", "k", "v")}
        else:
            shp = (w.B, w.H, w.N, w.d)
            s = {"q": draw(shp, w.qk_scale), "k": draw(shp, w.qk_scale), "v": draw(shp, w.v_scale)}
        sets.append(s)
    if w.map != wl.MAP_TAYLOR2:
        if host0 is not None:
            W = torch.from_numpy(host0["W"]).to(dev).to(tdt)
            b = torch.from_numpy(host0["b"]).to(dev).to(tdt)
        else:
            W = draw((w.H, w.d, w.d), w.w_std)
            b = draw((w.H, w.d), w.b_std)
        if not wl.map_has_bias(w.map):
            b = None
    else:
        W = b = None

    stream = torch.cuda.current_stream()
    if decode:
        dp = wl.feature_dim(w.map, w.d)
        # a 4096-token prefix state built by the forward itself (values only matter for realism)
        states = []
        for si in range(N_SETS):
            kq = draw((w.B, w.H, w.N, w.d), w.qk_scale)
            vv = draw((w.B, w.H, w.N, w.d), w.v_scale)
            _, S, z = hh.hh_linattn_fwd(kq, kq, vv, W, b, map=w.map, want_state=True)
            states.append((S, z))
            del kq, vv
        outs = [torch.empty((w.B, w.H, w.d), dtype=tdt, device=dev) for _ in range(N_SETS)]

        def step(i, st):
            s = sets[i % N_SETS]
            S, z = states[i % N_SETS]
            hh.hh_linattn_decode_step(s["q"], s["k"], s["v"], W, b, S, z, map=w.map, out=outs[i % N_SETS],
                                      stream=st)
        flops, byts = decode_counts(w)
    elif backward:
        need = hh.hh_linattn_bwd_workspace(w.map, w.dtype, w.causal, w.B, w.H, w.N, w.d)
        wss = [torch.empty((max(need, 16),), dtype=torch.uint8, device=dev) for _ in range(N_SETS)]
        shp = (w.B, w.H, w.N, w.d)
        for s in sets:  # the forward's output and a random dL/dy per input set
            s["y"] = hh.hh_linattn_fwd(s["q"], s["k"], s["v"], W, b, causal=w.causal, map=w.map)
            s["dy"] = draw(shp, 1.0)
        grads = [(torch.empty_like(sets[0]["q"]), torch.empty_like(sets[0]["q"]), torch.empty_like(sets[0]["q"]),
                  torch.empty((w.H, w.d, w.d), dtype=torch.float32, device=dev),
                  torch.empty((w.H, w.d), dtype=torch.float32, device=dev) if b is not None else None)
                 for _ in range(N_SETS)]

        def step(i, st):
            s = sets[i % N_SETS]
            dq, dk, dv, dW, db = grads[i % N_SETS]
            hh.hh_linattn_bwd(s["q"], s["k"], s["v"], W, b, s["y"], s["dy"], causal=w.causal, map=w.map, dq=dq,
                              dk=dk, dv=dv, dW=dW, db=db, workspace=wss[i % N_SETS], stream=st)
        flops, byts = backward_counts(w)
    elif distill:
        need = hh.hh_distill_loss_workspace(w.map, w.dtype, w.B, w.H, w.N, w.d)
        wss = [torch.empty((max(need, 16),), dtype=torch.uint8, device=dev) for _ in range(N_SETS)]
        outs = [torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev) for _ in range(N_SETS)]

        def step(i, st):
            s = sets[i % N_SETS]
            hh.hh_distill_loss(s["q"], s["k"], W, b, map=w.map, out=outs[i % N_SETS], workspace=wss[i % N_SETS],
                               stream=st)
        flops, byts = distill_counts(w)
    else:
        need = hh.hh_linattn_fwd_workspace(w.map, w.dtype, w.causal, w.B, w.H, w.N, w.d)
        wss = [torch.empty((max(need, 16),), dtype=torch.uint8, device=dev) for _ in range(N_SETS)]
        outs = [torch.empty_like(sets[0]["q"]) for _ in range(N_SETS)]

        def step(i, st):
            s = sets[i % N_SETS]
            hh.hh_linattn_fwd(s["q"], s["k"], s["v"], W, b, causal=w.causal, map=w.map, out=outs[i % N_SETS],
                              workspace=wss[i % N_SETS], stream=st)
        flops, byts = algorithmic_counts(w)

    # GRAPH_STEPS consecutive calls (cycling over the input sets) captured as one HIP graph, so
    # that host launch cost stays out of the timed region (a decode step is shorter than a
    # Python call); a "launch" below is then one replay of GRAPH_STEPS calls.  --eager launches
    # every call from Python.
    gsteps = 1 if args.eager else GRAPH_STEPS
    if args.steps % gsteps:
        args.steps += gsteps - args.steps % gsteps
    if args.eager:
        def run(i):
            step(i, stream)
    else:
        for j in range(N_SETS):
            step(j, stream)  # each input set once before capture
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for j in range(gsteps):
                step(j, torch.cuda.current_stream())

        def run(i):
            graph.replay()

    # Clock settling: the GPU raises its clocks only after tens of milliseconds of load, so the
    # step is replayed (untimed) for CLOCK_SETTLE_S seconds before the W warm-up steps; without
    # it a short warm-up times the ramp rather than the steady state a busy device runs at.
    t_settle = time.perf_counter()
    i = 0
    while time.perf_counter() - t_settle < args.settle:
        for _ in range(8):
            run(i)
            i += 1
        torch.cuda.synchronize()
    for i in range(max(1, args.warmup // gsteps)):
        run(i)
    torch.cuda.synchronize()

    # ---- timed region: K steps, per-launch events on the launch stream
    nlaunch = args.steps // gsteps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nlaunch)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(nlaunch):
        ev[i][0].record(stream)
        run(i)
        ev[i][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    per = np.array([a.elapsed_time(bq) for a, bq in ev]) / gsteps  # per call
    ms_per_step = total_ms / args.steps
    launch_ms = float(per.mean())

    tokens = w.B * (1 if decode else w.N)
    value = tokens / (ms_per_step * 1e-3)
    # achieved rates over the whole timed region (the same clock as `value`); the mean of the
    # per-launch events is reported beside them
    ach_gbs = byts / (ms_per_step * 1e-3) / 1e9
    ach_tflops = flops / (ms_per_step * 1e-3) / 1e12
    ai = flops / byts
    ridge = PEAK_MFMA_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    bound = "hbm" if ai < ridge else "mfma"
    entry = ("hh_linattn_decode_step" if decode else "hh_distill_loss" if distill else
             "hh_linattn_bwd" if backward else "hh_linattn_fwd")
    traffic = recorded_traffic(args.workload, entry)
    traffic_gbs = None if traffic is None else round(traffic / (ms_per_step * 1e-3) / 1e9, 1)
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(ach_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach_gbs / PEAK_HBM_GBS, 4), "traffic": traffic_gbs}
    else:
        roof = {"bound": "mfma", "achieved": round(ach_tflops, 1), "peak": PEAK_MFMA_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach_tflops / PEAK_MFMA_BF16_TFLOPS, 4), "traffic": traffic_gbs}
    if traffic is not None:
        roof["traffic_bytes_per_call"] = traffic
    if decode:
        roof["kernel"] = "hh_linattn_decode_step (decode_kernel)"
    elif backward:
        roof["kernel"] = ("hh_linattn_bwd: every kernel of one call (feature maps, forward segment sums and scan, "
                          "q-side pass, reverse-sum scan, k-side pass, feature-map backward, dW/db reduction)")
    elif distill:
        roof["kernel"] = "hh_distill_loss: every kernel of one call (feature map of k, then distill_kernel, which maps its queries itself)"
    elif w.map == wl.MAP_TAYLOR2:
        roof["kernel"] = ("hh_linattn_fwd: every kernel of one call (segment aggregates, exclusive prefix "
                          "over segments, chunked causal pass)")
    elif w.map == wl.MAP_HEDGEHOG_SOFTMAX and w.causal and w.d in (64, 128):
        roof["kernel"] = ("hh_linattn_fwd: every kernel of one call (segment-state pass and chunked pass, each "
                          "forming and normalising the softmax features itself)")
    elif w.map != wl.MAP_HEDGEHOG:
        roof["kernel"] = ("hh_linattn_fwd: every kernel of one call (feature maps of q and k into the workspace, "
                          "segment aggregates, chunked causal pass over the features)")
    elif not w.causal:
        roof["kernel"] = ("hh_linattn_fwd: every kernel of one call (total state and read-out; one fused "
                          "kernel when a sequence is one segment)")
    else:
        roof["kernel"] = ("hh_linattn_fwd: every kernel of one call (segment-state pass, then the chunked pass, "
                          "which adds the earlier segments' aggregates itself)")
    roof["launch_ms_mean"] = round(launch_ms, 5)
    roof["calls_per_timed_launch"] = gsteps  # a timed launch: one graph replay of this many calls
    roof["launch_ms_p10_p90"] = [round(float(np.percentile(per, 10)), 5), round(float(np.percentile(per, 90)), 5)]
    roof["alg_flops"] = flops
    roof["alg_bytes"] = byts
    roof["mfma_frac_of_bf16_peak"] = round(ach_tflops / PEAK_MFMA_BF16_TFLOPS, 4)

    cpu = None
    cpu_model = host_cpu_model()
    if not args.no_cpu_baseline and distill:
        import oracle
        nthr = oracle.default_threads()
        xw = host0
        # query rows spread evenly over the sequence (their mean cost is the full loss's), in rounds
        # of 16 rows per head until about 10 s of wall time
        rows_done, tc, rnd = 0, 0.0, 0
        while rnd < 30 and (tc < 10.0 or rnd == 0):
            rows = [int((w.N - 1) * (j + 0.5 * (rnd % 2)) / 16) for j in range(16)]
            t0 = time.perf_counter()
            oracle.distill_loss(w.map, xw["q"], xw["k"], xw["W"], xw["b"], rows=rows, nthreads=nthr)
            tc += time.perf_counter() - t0
            rows_done += len(rows) * w.B
            rnd += 1
        # the same rows once more on one thread
        rows = [int((w.N - 1) * (j + 0.5) / 16) for j in range(16)]
        t0 = time.perf_counter()
        oracle.distill_loss(w.map, xw["q"], xw["k"], xw["W"], xw["b"], rows=rows, nthreads=1)
        t1 = time.perf_counter() - t0
        cpu = {"value": round(rows_done / tc, 1), "unit": "tokens/s", "cores": nthr, "kind": "oracle",
               "sample": f"{rnd} rounds of 16 query rows per head (all {w.H} heads, rows spread over the sequence) "
                         f"of {w.name} (B{w.B} H{w.H} N{w.N} d{w.d}) by the fp64 oracle, {tc:.2f} s wall on "
                         f"{nthr} threads",
               "cpu_model": cpu_model,
               "value_1_thread": round(len(rows) * w.B / t1, 2),
               "sample_1_thread": f"one round of 16 query rows per head on 1 thread, {t1:.2f} s wall"}
    elif not args.no_cpu_baseline and backward:
        import oracle
        nthr = oracle.default_threads()
        xw = host0
        rng = np.random.default_rng(w.seed + 1)
        hs = min(w.H, nthr)  # a bounded sample: the oracle's explicit form costs N^2 per head
        dy = rng.standard_normal((w.B, hs, w.N, w.d))
        sub = {k_: xw[k_][:, :hs] for k_ in ("q", "k", "v")}
        t0 = time.perf_counter()
        oracle.backward(w.map, sub["q"], sub["k"], sub["v"], xw["W"][:hs], xw["b"][:hs], dy, causal=w.causal,
                        nthreads=nthr)
        tc = time.perf_counter() - t0
        cpu = {"value": round(w.B * w.N * hs / w.H / tc, 1), "unit": "tokens/s", "cores": nthr, "kind": "oracle",
               "sample": f"the backward of {hs} of the {w.H} heads of {w.name} (B{w.B} N{w.N} d{w.d}) by the fp64 "
                         f"oracle's explicit form, {tc:.2f} s wall on {nthr} threads; scaled to the full workload",
               "cpu_model": cpu_model}
    elif not args.no_cpu_baseline and not decode:
        import oracle
        nthr = oracle.default_threads()
        xw = host0
        # whole forwards of the same workload, repeated until about 10 s of wall time (at most 30)
        reps, tc = 0, 0.0
        while reps < 30 and (tc < 10.0 or reps == 0):
            t0 = time.perf_counter()
            if w.causal:
                oracle.causal(w.map, xw["q"], xw["k"], xw["v"], xw["W"], xw["b"], nthreads=nthr)
            else:
                oracle.bidir(w.map, xw["q"], xw["k"], xw["v"], xw["W"], xw["b"], nthreads=nthr)
            tc += time.perf_counter() - t0
            reps += 1
        # one whole forward on a single thread
        t0 = time.perf_counter()
        if w.causal:
            oracle.causal(w.map, xw["q"], xw["k"], xw["v"], xw["W"], xw["b"], nthreads=1)
        else:
            oracle.bidir(w.map, xw["q"], xw["k"], xw["v"], xw["W"], xw["b"], nthreads=1)
        t1 = time.perf_counter() - t0
        cpu = {"value": round(reps * tokens / tc, 1), "unit": "tokens/s", "cores": nthr, "kind": "oracle",
               "sample": f"{reps} full forwards of {w.name} (B{w.B} H{w.H} N{w.N} d{w.d}) by the fp64 oracle, "
                         f"{tc:.2f} s wall on {nthr} threads",
               "cpu_model": cpu_model,
               "value_1_thread": round(tokens / t1, 1),
               "sample_1_thread": f"one full forward on 1 thread, {t1:.2f} s wall"}

    out = {
        "metric": (METRIC if w.name == "c3_llama2_causal" else
                   "decode step tokens/s (one token per sequence)" if decode else
                   "backward tokens/s (dq, dk, dv, dW, db) at Llama-2-7B heads" if backward else
                   "distillation loss (Eq. 4) query tokens/s at Llama-2-7B heads" if distill else
                   f"{'causal' if w.causal else 'bidirectional'} linear-attn fwd tokens/s (\u03c6 incl.), {w.name}"),
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle_s": args.settle,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == wl.DT_BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "map": {wl.MAP_HEDGEHOG: "hedgehog", wl.MAP_TAYLOR2: "taylor2",
                           wl.MAP_HEDGEHOG_SOFTMAX: "hedgehog_softmax", wl.MAP_EXP: "exp",
                           wl.MAP_SOFTMAX: "softmax"}[w.map], "causal": w.causal,
                   "input_sets_rotated": N_SETS, "launch": "eager" if args.eager else "hip_graph_replay"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 4),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
