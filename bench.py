#!/usr/bin/env python3
"""Benchmark of the quantized GEMV hot path on one MI355X.

Step = one batch-1 decode pass of a 7B-shaped model's projections: 28 layers x
{Wq 3584x3584, Wk 512x3584, Wv 512x3584, Wo 3584x3584, gate 18944x3584,
up 18944x3584, down 3584x18944}, all Q4_K (3,670,474,752 weight bytes), each with
its own fp32 activation vector. Launches follow the layer's dependency stages
{q,k,v} -> {o} -> {gate,up} -> {down}: one grouped launch per stage, 112 per step,
replayed from a captured HIP graph. Inputs are resident in HBM before timing; the
3.67 GB sweep is far larger than the 256 MB Infinity Cache, so it streams from HBM.

Printed (one JSON line): whole-step throughput in GB/s of algorithmic bytes
(weights + x + y), equivalent tokens/s (bytes per token as the pages' bandwidth
wall divides them), the roofline entry of the dominant kernel (Q4_K GEMV: bytes
per launch / average launch duration from HIP events on the launch stream), the
fp64 CPU oracle timed on a bounded sample, and the other hot-path rows (single
4096x4096 Q4_K GEMV, Q8_0 11008x4096 / 4096x11008, Q6_K 3584x18944 / 152064x3584,
fused 152064x3584 LM head + argmax, the same head verifying 5 columns (fp32 and int8
activations), top-20 with
log-probabilities and one sampled token, small-N verify N=5, N=32 and N=2 over the
same 196 matrices, the N=5 verify step and the decode step with int8 activations), each timed with rotation over
enough weight copies to defeat the Infinity Cache.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Q4_K GEMV achieved HBM GB/s (% of peak) and equiv. tokens/s at 7B shapes"
PEAK_HBM_GBS = 8000.0
MALL_BYTES = 256 << 20


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def graph_ms(torch, fn, reps: int, warm: int = 2) -> float:
    """Capture fn() into a HIP graph, replay it `reps` times, return ms per replay."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def graph_stats(torch, fn, reps: int, warm: int = 2):
    """As graph_ms, with an event before every replay: (mean, median, best, cv) of the
    per-replay times in ms; the mean is the timed region over its replays."""
    import numpy as np
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    for k in range(reps):
        evs[k].record()
        g.replay()
    evs[-1].record()
    torch.cuda.synchronize()
    per = np.array([evs[k].elapsed_time(evs[k + 1]) for k in range(reps)])
    mean = evs[0].elapsed_time(evs[-1]) / reps
    return mean, float(np.median(per)), float(per.min()), float(per.std() / per.mean())


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "q4k_gemv_7b_decode_step_traffic.md")
TRAFFIC_SOURCES = ("quantized_gemv_argmax_amd/csrc/q4k_gemv.hip", "quantized_gemv_argmax_amd/csrc/qg_device.h")


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per Q4_K GEMV launch from the committed counter summary (FETCH_SIZE and
    WRITE_SIZE, scaled by a plain copy's counts), or None when the kernel sources have
    changed since the counters were taken."""
    try:
        with open(TRAFFIC_PROFILE) as fh:
            kv = dict(line.split(": ", 1) for line in fh.read().splitlines() if ": " in line and not line.startswith(" "))
    except OSError:
        return None
    if kv.get("kernel-source-hash", "").strip() != kernel_source_hash():
        return None
    return float(kv["traffic-per-launch-bytes"])


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=28, help=argparse.SUPPRESS)
    ap.add_argument("--no-rows", action="store_true", help="skip the other hot-path rows")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-ref", action="store_true",
                    help="end with one plain 256 MiB device copy (a reference dispatch for traffic counters)")
    ap.add_argument("--counters", action="store_true",
                    help="instead of the timed rows, run each other hot-path kernel a few times on distinct "
                         "weight copies (a short program for rocprofv3 --pmc passes)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the projections would shard by rows across GPUs). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import quantized_gemv_argmax_amd as qg
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    qg.lib()
    ws = qg.Workspace(dev, 64 << 20)

    # ------------------------------------------------------------ 7B decode step
    n_layers = args.layers
    t0 = time.time()
    layers = []
    cpu_sample = []
    w_bytes = 0
    xy_bytes = 0
    for L in range(n_layers):
        mats = []
        for i, (name, M, K) in enumerate(wl.LAYER_MATRICES):
            W = wl.q4k_blocks(M, K, key=(3, L, i))
            canon = torch.from_numpy(W.reshape(-1)).to(dev)
            wp = qg.pack_q4k(canon, M, K)
            del canon
            x = wl.x_vector(K, key=(3, L, i))
            mats.append((wp, torch.from_numpy(x).to(dev), torch.empty(M, dtype=torch.float32, device=dev), M, K))
            w_bytes += W.size
            xy_bytes += 4 * (K + M)
            if L == 0:
                cpu_sample.append((W, x, M, K))
        layers.append(mats)
        if L % 7 == 6:
            log(f"generated and packed {L + 1}/{n_layers} layers ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()
    step_bytes = w_bytes + xy_bytes
    stages = [[layers[L][i] for i in st] for L in range(n_layers) for st in wl.LAYER_STAGES]

    def step():
        for st in stages:
            qg.qgemv_q4k_batch(st)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    log("warm-up done; capturing the step graph")

    # timed region: K steps replayed from one captured graph; an event before every
    # replay and one after the last, all on the stream the graph is launched on
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        evs[k].record()
        g.replay()
    evs[-1].record()
    torch.cuda.synchronize()
    per_step = np.array([evs[k].elapsed_time(evs[k + 1]) for k in range(args.steps)])  # ms
    ms_step = evs[0].elapsed_time(evs[-1]) / args.steps
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    log(f"step {ms_step:.4f} ms -> {gbs:.1f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% of 8 TB/s); "
        f"median {np.median(per_step):.4f} ms, best {per_step.min():.4f} ms, cv {per_step.std() / per_step.mean():.4f}")

    # roofline of the dominant kernel (every launch of the step is a Q4_K GEMV): the
    # average launch duration is the timed region's length over its launch count
    # (launches run back to back inside the graph); per stage, the same for a graph
    # of one stage's 28 launches (different layers, so the weights stay cold)
    n_launch = len(stages)
    avg_launch_ms = ms_step / n_launch
    avg_launch_bytes = step_bytes / n_launch
    achieved = avg_launch_bytes / (avg_launch_ms * 1e-3) / 1e9
    per_stage = {}
    for k, name in enumerate(["qkv", "o", "gate_up", "down"]):
        sts = stages[k::4]
        nb = sum(p[0].numel() + 4 * (p[3] + p[4]) for p in sts[0])
        # rotate over enough weight copies that one replay streams >= 1 GB, more than
        # the 256 MB Infinity Cache holds (the 28 o projections are only 203 MB)
        copies = max(1, -(-(1 << 30) // (nb * len(sts))))
        extra = [[(p[0].clone(),) + tuple(p[1:]) for p in st] for _ in range(copies - 1) for st in sts]

        def stage_fn(sts=sts + extra):
            for st in sts:
                qg.qgemv_q4k_batch(st)
        us = graph_ms(torch, stage_fn, reps=max(10, args.steps // 2)) * 1e3 / (len(sts) + len(extra))
        per_stage[name] = {"avg_us": round(us, 3), "bytes": int(nb), "GBps": round(nb / (us * 1e-6) / 1e9, 1),
                           "weight_copies": copies}
        del extra
    log(f"dominant kernel: {achieved:.1f} GB/s, {avg_launch_ms * 1e3:.3f} us per launch; per stage {per_stage}")
    traffic = measured_traffic()
    roofline = {"kernel": "q4k_gemv_kernel", "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": None if traffic is None else int(traffic),
                "launches_per_step": n_launch, "avg_launch_us": round(avg_launch_ms * 1e3, 3),
                "avg_bytes_per_launch": int(avg_launch_bytes), "per_stage": per_stage}

    rows = {}
    if args.counters:
        counter_rows(torch, np, qg, wl, dev, ws, layers, n_layers)
    elif not args.no_rows:
        rows = other_rows(torch, np, qg, wl, dev, ws, layers, n_layers)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cpu_sample, args.cpu_seconds, step_bytes, wl)

    out = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16(x) * int4(q) -> fp32 accumulate (fp32 in/out)",
        "data": "synthetic",
        "config": {
            "workload": "7B-shaped decode step, batch 1: %d layers x {Wq 3584x3584, Wk 512x3584, Wv 512x3584, "
                        "Wo 3584x3584, gate 18944x3584, up 18944x3584, down 3584x18944}, Q4_K weights, "
                        "fp32 x per matrix" % n_layers,
            "bytes_per_step": int(step_bytes),
            "weight_bytes_per_step": int(w_bytes),
            "pct_of_peak_hbm": round(100 * gbs / PEAK_HBM_GBS, 2),
            "equiv_tokens_per_s": round(1e3 / ms_step, 1),
            "ms_per_step_median": round(float(np.median(per_step)), 4),
            "ms_per_step_best": round(float(per_step.min()), 4),
            "ms_per_step_cv": round(float(per_step.std() / per_step.mean()), 4),
            "launches_per_step": len(stages),
            "timing": "HIP graph of one step, replayed; events on the launch stream",
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(out), flush=True)
    if args.copy_ref:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()


def counter_rows(torch, np, qg, wl, dev, ws, layers, n_layers):
    """Each of the other hot-path kernels a few times, every call on its own weight
    copy, in this order: 4096x4096 Q4_K GEMV (3 calls), Q8_0 11008x4096 and
    4096x11008 (3 each), LM head + argmax 152064x3584 (2), the same head verifying 5
    columns (2, vector-ALU form) and 5 int8 columns (2), top-20 + sampling on that head (2), small-N N=5 then N=32 over
    the layers' stages (one grouped launch per stage), Q6_K 3584x18944 (3) and
    152064x3584 (2), int8-activation Q4_K 4096x4096 (3, after one quantization)."""
    M, K = 4096, 4096
    W = wl.q4k_blocks(M, K, key=(1, 0))
    wp = qg.pack_q4k(torch.from_numpy(W.reshape(-1)).to(dev), M, K)
    x = torch.from_numpy(wl.x_vector(K, key=(1, 0))).to(dev)
    y = torch.empty(M, device=dev)
    for c in [wp] + [wp.clone() for _ in range(2)]:
        qg.qgemv_q4k(c, x, M, K, y=y)
    for (M, K) in [(11008, 4096), (4096, 11008)]:
        W = wl.q8_0_blocks(M, K, key=(2, M))
        wp = qg.pack_q8_0(torch.from_numpy(W.reshape(-1)).to(dev), M, K)
        x = torch.from_numpy(wl.x_vector(K, key=(2, M))).to(dev)
        y = torch.empty(M, device=dev)
        for c in [wp] + [wp.clone() for _ in range(2)]:
            qg.qgemv_q8_0(c, x, M, K, y=y)
    M, K = wl.VOCAB, wl.HIDDEN
    W = wl.q8_0_blocks(M, K, key=(4, 0))
    wp = qg.pack_q8_0(torch.from_numpy(W.reshape(-1)).to(dev), M, K)
    del W
    x = torch.from_numpy(wl.x_vector(K, key=(4, 0))).to(dev)
    copies = (wp, wp.clone())
    for c in copies:
        qg.lmhead_argmax(c, x, M, K, ws=ws)
    X5 = torch.from_numpy(wl.x_columns(K, 5, key=(4, 3))).to(dev)
    for c in copies:
        qg.lmhead_argmax_verify(c, X5, M, K, ws=ws)
    X5q = qg.quantize_q8_1_columns(X5)
    for c in copies:
        qg.lmhead_argmax_verify_q8_1(c, X5q, M, K, 5, ws=ws)
    u_dev = torch.full((1,), 0.5, device=dev)
    for c in copies:
        qg.lmhead_topk(c, x, M, K, 20, sampler=(0.8, 0.95, 0.05, u_dev), ws=ws)
    del wp, copies
    for N in (5, 32, 2):
        for L in range(n_layers):
            for st in wl.LAYER_STAGES:
                grp = []
                for i in st:
                    wp_, _, _, M_, K_ = layers[L][i]
                    X_ = torch.from_numpy(wl.x_columns(K_, N, key=(5, L, i, N))).to(dev)
                    grp.append((wp_, X_, torch.empty((N, (M_ + 3) // 4 * 4), device=dev), M_, K_))
                qg.qgemm_q4k_smalln_batch_ws(grp)
    for L in range(n_layers):  # N = 5 on int8 activations
        for st in wl.LAYER_STAGES:
            grp = []
            for i in st:
                wp_, _, _, M_, K_ = layers[L][i]
                X_ = torch.from_numpy(wl.x_columns(K_, 5, key=(5, L, i, 5))).to(dev)
                grp.append((wp_, qg.quantize_q8_1_columns(X_), torch.empty((5, (M_ + 3) // 4 * 4), device=dev), M_, K_))
            qg.qgemm_q4k_q8_1_smalln_batch(grp)
    for (M, K), reps in [((wl.HIDDEN, wl.FFN), 3), ((wl.VOCAB, wl.HIDDEN), 2)]:
        W = wl.q6k_blocks(M, K, key=(6, M))
        wp = qg.pack_q6k(torch.from_numpy(W.reshape(-1)).to(dev), M, K)
        del W
        x = torch.from_numpy(wl.x_vector(K, key=(6, M))).to(dev)
        y = torch.empty(M, device=dev)
        for c in [wp] + [wp.clone() for _ in range(reps - 1)]:
            qg.qgemv_q6k(c, x, M, K, y=y)
        del wp
    M, K = 4096, 4096
    W = wl.q4k_blocks(M, K, key=(1, 0))
    wp = qg.pack_q4k(torch.from_numpy(W.reshape(-1)).to(dev), M, K)
    x = torch.from_numpy(wl.x_vector(K, key=(1, 0))).to(dev)
    xq = qg.quantize_q8_1(x)
    y = torch.empty(M, device=dev)
    for c in [wp] + [wp.clone() for _ in range(2)]:
        qg.qgemv_q4k_q8_1(c, xq, M, K, y=y)
    torch.cuda.synchronize()
    log("counter rows done")


def other_rows(torch, np, qg, wl, dev, ws, layers, n_layers):
    rows = {}

    # context: a plain device-to-device copy of 1 GiB (read + write bytes)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    ms = graph_ms(torch, lambda: dst.copy_(src), 10)
    rows["context_copy_1GiB"] = {"us": round(ms * 1e3, 1), "GBps": round(2 * src.numel() / (ms * 1e-3) / 1e9, 1)}
    log(f"row copy: {rows['context_copy_1GiB']}")
    del src, dst

    def rotated(wp, count):
        return [wp.clone() for _ in range(count)]

    # single Q4_K GEMV 4096x4096, 128 copies (1.2 GB) rotated
    M, K = 4096, 4096
    W = wl.q4k_blocks(M, K, key=(1, 0))
    wp = qg.pack_q4k(torch.from_numpy(W.reshape(-1)).to(dev), M, K)
    R = max(2, -(-(1 << 30) // wp.numel()))
    copies = rotated(wp, R)
    x = torch.from_numpy(wl.x_vector(K, key=(1, 0))).to(dev)
    y = torch.empty(M, device=dev)
    ms = graph_ms(torch, lambda: [qg.qgemv_q4k(c, x, M, K, y=y) for c in copies], 20) / R
    b = W.size + 4 * (M + K)
    rows["q4k_gemv_4096x4096"] = {"us": round(ms * 1e3, 3), "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                                  "bytes": b, "copies_rotated": R}
    log(f"row q4k 4096^2: {rows['q4k_gemv_4096x4096']}")
    del copies

    # Q8_0 GEMVs 11008x4096 and 4096x11008, rotated
    for (M, K) in [(11008, 4096), (4096, 11008)]:
        W = wl.q8_0_blocks(M, K, key=(2, M))
        wp = qg.pack_q8_0(torch.from_numpy(W.reshape(-1)).to(dev), M, K)
        R = max(2, -(-(1 << 30) // wp.numel()))
        copies = rotated(wp, R)
        x = torch.from_numpy(wl.x_vector(K, key=(2, M))).to(dev)
        y = torch.empty(M, device=dev)
        ms = graph_ms(torch, lambda: [qg.qgemv_q8_0(c, x, M, K, y=y) for c in copies], 20) / R
        b = W.size + 4 * (M + K)
        rows[f"q8_0_gemv_{M}x{K}"] = {"us": round(ms * 1e3, 3), "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                                      "bytes": b, "copies_rotated": R}
        log(f"row q8_0 {M}x{K}: {rows[f'q8_0_gemv_{M}x{K}']}")
        del copies

    # Q6_K GEMVs: the FFN down projection 3584x18944 (rotated copies) and the
    # 152064x3584 output head (2 copies), the two Q6_K matrices of a Q4_K_M 7B file
    for (M, K) in [(wl.HIDDEN, wl.FFN), (wl.VOCAB, wl.HIDDEN)]:
        W = wl.q6k_blocks(M, K, key=(6, M))
        wp = qg.pack_q6k(torch.from_numpy(W.reshape(-1)).to(dev), M, K)
        del W
        R = max(2, -(-(1 << 30) // wp.numel()))
        copies = rotated(wp, R)
        x = torch.from_numpy(wl.x_vector(K, key=(6, M))).to(dev)
        y = torch.empty(M, device=dev)
        ms = graph_ms(torch, lambda: [qg.qgemv_q6k(c, x, M, K, y=y) for c in copies], 20) / R
        b = wp.numel() + 4 * (M + K)
        rows[f"q6k_gemv_{M}x{K}"] = {"us": round(ms * 1e3, 3), "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                                     "bytes": b, "copies_rotated": R}
        log(f"row q6k {M}x{K}: {rows[f'q6k_gemv_{M}x{K}']}")
        del copies, wp

    # fused LM head + argmax 152064x3584 Q8_0, 2 copies
    M, K = wl.VOCAB, wl.HIDDEN
    W = wl.q8_0_blocks(M, K, key=(4, 0))
    wp = qg.pack_q8_0(torch.from_numpy(W.reshape(-1)).to(dev), M, K)
    del W
    copies = [wp, wp.clone()]
    x = torch.from_numpy(wl.x_vector(K, key=(4, 1, 0, 0))).to(dev)
    oi = torch.empty(1, dtype=torch.int32, device=dev)
    ov = torch.empty(1, dtype=torch.float32, device=dev)
    ms = graph_ms(torch, lambda: [qg.lmhead_argmax(c, x, M, K, out_index=oi, out_value=ov, ws=ws) for c in copies],
                  20) / 2
    b = wp.numel() + 4 * K + 8 * (-(-M // 16)) * 2 + 8  # weights, x, partials written and read, result
    # unfused comparison: Q8_0 GEMV writing the 608,256-byte logit vector + torch argmax
    logits = torch.empty(M, device=dev)
    ms_unfused = graph_ms(torch, lambda: [(qg.qgemv_q8_0(c, x, M, K, y=logits), torch.argmax(logits))
                                          for c in copies], 20) / 2
    h = torch.empty(M, dtype=torch.float32, pin_memory=True)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(20):
        h.copy_(logits, non_blocking=False)
    d2h_us = (time.perf_counter() - t) / 20 * 1e6
    hi = torch.empty(1, dtype=torch.int32, pin_memory=True)
    t = time.perf_counter()
    for _ in range(20):
        hi.copy_(oi, non_blocking=False)
    d2h4_us = (time.perf_counter() - t) / 20 * 1e6
    # stage 1 alone is not an entry point; the Q8_0 GEMV over the same head is the same
    # tile computation with the logits stored instead of reduced, so the difference
    # is what the second (argmax) launch adds inside a graph
    ms_gemv = graph_ms(torch, lambda: [qg.qgemv_q8_0(c, x, M, K, y=logits) for c in copies], 20) / 2
    rows["lmhead_argmax_152064x3584"] = {
        "us": round(ms * 1e3, 3), "GBps": round(b / (ms * 1e-3) / 1e9, 1), "bytes": int(b),
        "q8_0_gemv_same_head_us": round(ms_gemv * 1e3, 3),
        "stage2_argmax_us": round((ms - ms_gemv) * 1e3, 3),
        "unfused_gemv_plus_torch_argmax_us": round(ms_unfused * 1e3, 3),
        "d2h_logits_608256B_us": round(d2h_us, 2), "d2h_index_4B_us": round(d2h4_us, 2)}
    log(f"row lmhead: {rows['lmhead_argmax_152064x3584']}")

    # batched greedy verification on the same head: N = 5 columns in one pass
    N = 5
    X5 = torch.from_numpy(wl.x_columns(K, N, key=(4, 3))).to(dev)
    oi5 = torch.empty(N, dtype=torch.int32, device=dev)
    ov5 = torch.empty(N, dtype=torch.float32, device=dev)
    ms = graph_ms(torch, lambda: [qg.lmhead_argmax_verify(c, X5, M, K, out_index=oi5, out_value=ov5, ws=ws)
                                  for c in copies], 20) / 2
    b = wp.numel() + 4 * K * N + 8 * (-(-M // 16)) * N * 2 + 8 * N
    rows["lmhead_verify_N5_152064x3584"] = {"us": round(ms * 1e3, 3), "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                                            "bytes": int(b), "us_per_single_column_argmax": round(
                                                rows["lmhead_argmax_152064x3584"]["us"], 3)}
    log(f"row lmhead verify N=5: {rows['lmhead_verify_N5_152064x3584']}")
    # sixteen columns (15 drafts + 1), still one pass over the head
    N16 = 16
    X16 = torch.from_numpy(wl.x_columns(K, N16, key=(4, 4))).to(dev)
    oi16 = torch.empty(N16, dtype=torch.int32, device=dev)
    ov16 = torch.empty(N16, dtype=torch.float32, device=dev)
    ms = graph_ms(torch, lambda: [qg.lmhead_argmax_verify(c, X16, M, K, out_index=oi16, out_value=ov16, ws=ws)
                                  for c in copies], 20) / 2
    b = wp.numel() + 4 * K * N16 + 8 * (-(-M // 16)) * N16 * 2 + 8 * N16
    rows["lmhead_verify_N16_152064x3584"] = {"us": round(ms * 1e3, 3), "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                                             "bytes": int(b)}
    log(f"row lmhead verify N=16: {rows['lmhead_verify_N16_152064x3584']}")

    # the same verification on int8 activations: the five fp32 columns are quantized
    # (one launch) and verified, both inside the timed region
    X5q = qg.quantize_q8_1_columns(X5)
    ms = graph_ms(torch, lambda: [(qg.quantize_q8_1_columns(X5, out=X5q),
                                   qg.lmhead_argmax_verify_q8_1(c, X5q, M, K, N, out_index=oi5, out_value=ov5, ws=ws))
                                  for c in copies], 20) / 2
    ms_noq = graph_ms(torch, lambda: [qg.lmhead_argmax_verify_q8_1(c, X5q, M, K, N, out_index=oi5, out_value=ov5,
                                                                   ws=ws) for c in copies], 20) / 2
    b = wp.numel() + 4 * K * N + 2 * X5q.numel() + 8 * (-(-M // 16)) * N * 2 + 8 * N
    rows["lmhead_verify_N5_int8_activations"] = {
        "us": round(ms * 1e3, 3), "GBps": round(b / (ms * 1e-3) / 1e9, 1), "bytes": int(b),
        "quantization": "timed (one launch for the five columns)",
        "us_without_quantization": round(ms_noq * 1e3, 3),
        "us_fp32_activations": rows["lmhead_verify_N5_152064x3584"]["us"]}
    log(f"row lmhead verify N=5, int8 activations: {rows['lmhead_verify_N5_int8_activations']}")

    # top-20 log-probabilities and one sampled token on the same head (T 0.8,
    # top-p 0.95, min-p 0.05); the logits stay in a device buffer
    kk = 20
    u_dev = torch.full((1,), 0.5, device=dev)
    logits_buf = torch.empty(M, device=dev)
    tk = qg.TopK(kk, dev, True)
    smp = (0.8, 0.95, 0.05, u_dev)
    ms = graph_ms(torch, lambda: [qg.lmhead_topk(c, x, M, K, kk, logits=logits_buf, sampler=smp, ws=ws, out=tk)
                                  for c in copies], 20) / 2
    tiles = -(-M // 16)
    b = wp.numel() + 4 * K + 4 * M + 16 * tiles * 2 + 16 * kk * 4 + 4 * (3 * kk + 2)
    ms_sel = graph_ms(torch, lambda: qg.logits_topk(logits_buf, kk, sampler=smp, ws=ws, out=tk), 50)
    rows[f"lmhead_top{kk}_sample_152064x3584"] = {
        "us": round(ms * 1e3, 3), "GBps": round(b / (ms * 1e-3) / 1e9, 1), "bytes": int(b),
        "us_argmax_same_head": rows["lmhead_argmax_152064x3584"]["us"],
        "us_logits_topk_on_resident_logits": round(ms_sel * 1e3, 3)}
    log(f"row lmhead top-{kk} + sample: {rows[f'lmhead_top{kk}_sample_152064x3584']}")
    del copies, wp

    # small-N verify over the 196 decode matrices (weights read once per call), one
    # grouped launch per dependency stage as in the decode step
    for N in (5, 32, 2):
        sstages = []
        for L in range(n_layers):
            for st in wl.LAYER_STAGES:
                grp = []
                for i in st:
                    wp_, _, _, M_, K_ = layers[L][i]
                    X_ = torch.from_numpy(wl.x_columns(K_, N, key=(5, L, i, N))).to(dev)
                    grp.append((wp_, X_, torch.empty((N, (M_ + 3) // 4 * 4), device=dev), M_, K_))
                sstages.append(grp)

        # the workspace entry point, which may split few-tile stages over K slices
        # (the slices' sums are added by the last workgroup of each tile group); one
        # workspace serves every stage, allocated and zeroed before the timed region
        needs = [qg.qgemm_q4k_smalln_batch_workspace_bytes(grp) for grp in sstages]
        sws = qg.Workspace(dev, max(max(needs), 1))

        def vstep(sts=sstages):
            for grp in sts:
                qg.qgemm_q4k_smalln_batch_ws(grp, sws)

        ms, ms_med, ms_best, ms_cv = graph_stats(torch, vstep, 20)
        flat = [m for grp in sstages for m in grp]
        wb = sum(m[0].numel() for m in flat)
        b = wb + sum(4 * N * (m[3] + m[4]) for m in flat)
        per_stage = {}
        for k, name in enumerate(["qkv", "o", "gate_up", "down"]):
            sts = sstages[k::4]
            nb_ = sum(m[0].numel() + 4 * N * (m[3] + m[4]) for m in sts[0])
            us = graph_ms(torch, lambda sts=sts: vstep(sts), 5) * 1e3 / len(sts)
            per_stage[name] = {"avg_us": round(us, 3), "GBps": round(nb_ / (us * 1e-6) / 1e9, 1)}
        rows[f"smalln_verify_N{N}"] = {"ms_per_step": round(ms, 4), "ms_per_step_median": round(ms_med, 4),
                                       "ms_per_step_best": round(ms_best, 4), "ms_per_step_cv": round(ms_cv, 4),
                                       "replays": 20, "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                                       "bytes": int(b), "verified_tokens_per_s": round(N * 1e3 / ms, 1),
                                       "launches_per_step": len(sstages),
                                       "entry_point": "qgemm_q4k_smalln_batch_ws",
                                       "workspace_bytes": int(max(needs)), "per_stage": per_stage}
        log(f"row smalln N={N}: {rows[f'smalln_verify_N{N}']}")
        del sstages, flat

    # the verify step on int8 activations, N = 5: per dependency stage, one launch
    # quantizes the fp32 columns of all the stage's matrices (stacked, 5 per matrix)
    # and one grouped launch multiplies; both inside the timed region (224 launches
    # per step)
    N = 5
    qv = []
    for L in range(n_layers):
        for st in wl.LAYER_STAGES:
            K_ = layers[L][st[0]][4]
            Xs = torch.from_numpy(np.concatenate([wl.x_columns(K_, N, key=(5, L, i, N)) for i in st])).to(dev)
            nb8 = qg.q8_1_bytes(K_)
            xq = torch.empty(Xs.shape[0] * nb8, dtype=torch.uint8, device=dev)
            grp = []
            for j, i in enumerate(st):
                wp_, _, _, M_, _ = layers[L][i]
                grp.append((wp_, xq[j * N * nb8:(j + 1) * N * nb8], torch.empty((N, (M_ + 3) // 4 * 4), device=dev),
                            M_, K_))
            qv.append((Xs, xq, grp))

    def ivstep(sts=qv, quantize=True):
        for Xs, xq, grp in sts:
            if quantize:
                qg.quantize_q8_1_columns(Xs, out=xq)
            qg.qgemm_q4k_q8_1_smalln_batch(grp)

    ms, ms_med, ms_best, ms_cv = graph_stats(torch, ivstep, 20)
    ms_noq = graph_ms(torch, lambda: ivstep(quantize=False), 20)
    b = sum(Xs.numel() * 4 + 2 * xq.numel() + sum(m[0].numel() + 4 * N * m[3] for m in grp) for Xs, xq, grp in qv)
    per_stage = {}
    for k, name in enumerate(["qkv", "o", "gate_up", "down"]):
        sts = qv[k::4]
        Xs, xq, grp = sts[0]
        nb_ = Xs.numel() * 4 + 2 * xq.numel() + sum(m[0].numel() + 4 * N * m[3] for m in grp)
        us = graph_ms(torch, lambda sts=sts: ivstep(sts), 5) * 1e3 / len(sts)
        per_stage[name] = {"avg_us": round(us, 3), "GBps": round(nb_ / (us * 1e-6) / 1e9, 1)}
    rows["smalln_verify_N5_int8_activations"] = {
        "ms_per_step": round(ms, 4), "ms_per_step_median": round(ms_med, 4), "ms_per_step_best": round(ms_best, 4),
        "ms_per_step_cv": round(ms_cv, 4), "replays": 20, "GBps": round(b / (ms * 1e-3) / 1e9, 1), "bytes": int(b),
        "verified_tokens_per_s": round(N * 1e3 / ms, 1), "launches_per_step": 2 * len(qv), "per_stage": per_stage,
        "quantization": "timed (one launch per stage for all its columns)",
        "ms_per_step_without_quantization": round(ms_noq, 4)}
    log(f"row smalln N=5, int8 activations: {rows['smalln_verify_N5_int8_activations']}")
    del qv

    # the decode step with int8 activations (Q8_1-style, scale and sum per 32): per
    # dependency stage one launch quantizes the stage's fp32 x (stacked) and one
    # grouped launch multiplies on the integer path; both inside the timed region
    qstages = []
    for L in range(n_layers):
        for st in wl.LAYER_STAGES:
            K_ = layers[L][st[0]][4]
            Xs = torch.stack([layers[L][i][1] for i in st])
            nb8 = qg.q8_1_bytes(K_)
            xq = torch.empty(len(st) * nb8, dtype=torch.uint8, device=dev)
            grp = [(layers[L][i][0], xq[j * nb8:(j + 1) * nb8], layers[L][i][2], layers[L][i][3], K_)
                   for j, i in enumerate(st)]
            qstages.append((Xs, xq, grp))

    def qstep(sts=qstages, quantize=True):
        for Xs, xq, grp in sts:
            if quantize:
                qg.quantize_q8_1_columns(Xs, out=xq)
            qg.qgemv_q4k_q8_1_batch(grp)

    ms = graph_ms(torch, qstep, 20)
    ms_noq = graph_ms(torch, lambda: qstep(quantize=False), 20)
    b = sum(Xs.numel() * 4 + 2 * xq.numel() + sum(m[0].numel() + 4 * m[3] for m in grp) for Xs, xq, grp in qstages)
    per_stage = {}
    for k, name in enumerate(["qkv", "o", "gate_up", "down"]):
        sts = qstages[k::4]
        Xs, xq, grp = sts[0]
        nb_ = Xs.numel() * 4 + 2 * xq.numel() + sum(m[0].numel() + 4 * m[3] for m in grp)
        us = graph_ms(torch, lambda sts=sts: qstep(sts), 10) * 1e3 / len(sts)
        per_stage[name] = {"avg_us": round(us, 3), "GBps": round(nb_ / (us * 1e-6) / 1e9, 1)}
    rows["decode_step_int8_activations"] = {
        "ms_per_step": round(ms, 4), "GBps": round(b / (ms * 1e-3) / 1e9, 1), "bytes": int(b),
        "launches_per_step": 2 * len(qstages), "per_stage": per_stage,
        "quantization": "timed (one launch per stage for its x vectors)",
        "ms_per_step_without_quantization": round(ms_noq, 4)}
    log(f"row decode step, int8 activations: {rows['decode_step_int8_activations']}")
    del qstages
    return rows


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(sample, seconds, step_bytes, wl):
    """The fp64 C oracle (OpenMP over rows, otherwise untuned) on two bounded
    samples of the benchmark's workloads, once on one thread and once on every
    host core: layer 0 of the decode step (its seven Q4_K matrices) and the
    152064 x 3584 Q8_0 LM head (one x). Each leg runs whole passes for about a
    quarter of `seconds`; reported as GB/s of algorithmic bytes, ms per pass and,
    for the layer, equivalent decode tokens/s (28 layers)."""
    import oracle

    oracle.lib()
    all_cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    M, K = wl.VOCAB, wl.HIDDEN
    Wh = wl.q8_0_blocks(M, K, key=(4, 0))
    xh = wl.x_vector(K, key=(4, 1, 0, 0))
    head_bytes = Wh.size + 4 * (K + M)
    layer_bytes = sum(W.size + 4 * (Mm + Kk) for W, _, Mm, Kk in sample)

    def timed(fn, nbytes, budget):
        passes, t = 0, time.perf_counter()
        while True:
            fn()
            passes += 1
            el = time.perf_counter() - t
            if el >= budget:
                return passes, el, nbytes * passes / el / 1e9

    legs = {}
    for threads in (1, all_cores):
        oracle.set_num_threads(threads)
        got = oracle.num_threads()
        p, el, gbs = timed(lambda: [oracle.gemv_q4k(W, Mm, Kk, x) for W, x, Mm, Kk in sample], layer_bytes,
                           seconds / 4)
        legs[f"decode_layer_{got}t"] = {"GBps": round(gbs, 4), "ms_per_layer": round(1e3 * el / p, 2),
                                        "equiv_tokens_per_s": round(gbs * 1e9 / step_bytes, 4), "threads": got,
                                        "passes": p}
        p, el, gbs = timed(lambda: oracle.gemv_q8_0(Wh, M, K, xh), head_bytes, seconds / 4)
        legs[f"lm_head_{got}t"] = {"GBps": round(gbs, 4), "ms_per_head": round(1e3 * el / p, 2), "threads": got,
                                   "passes": p}
        log(f"cpu oracle, {got} thread(s): layer {legs[f'decode_layer_{got}t']}, head {legs[f'lm_head_{got}t']}")
    oracle.set_num_threads(all_cores)
    best = legs[f"decode_layer_{oracle.num_threads()}t"]
    return {"value": best["GBps"], "unit": "GB/s", "cores": best["threads"], "kind": "oracle",
            "sample": f"layer 0 of the 28-layer decode step (7 Q4_K matrices, {layer_bytes} algorithmic bytes), whole "
                      f"passes for ~{seconds / 4:.0f} s per leg; also the 152064x3584 Q8_0 head and one-thread runs "
                      f"(legs)",
            "cpu_model": cpu_model(), "host_threads": all_cores, "equiv_tokens_per_s": best["equiv_tokens_per_s"],
            "legs": legs}


if __name__ == "__main__":
    main()
