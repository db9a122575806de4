"""Benchmark of the MI355X routed-expert hot path; prints ONE JSON line.

Headline (value): batch-1 decode step, H=2048, I=768, a 64-slot expert pool,
top-k 8 with 8/8 routes active: x quant -> gate/up -> SiLU*up requant -> down
-> top-k reduce, replayed from captured hipGraphs with a fresh input set each
step (a ring of 16 graphs over 16 input sets already resident in HBM).  The
Infinity Cache is flushed before every step (outside the timed events), so
the expert weights come from HBM, and each step is bracketed by HIP events on
the stream the kernels run on.

Also reported: the same at 4/2/0 active routes and for H=4096, I=1024 (time
vs active routes), warm-cache times, the fused gather (k=7168, 8192 rows),
the grouped prefill GEMMs at 24576 routes (E=256, top-6, H=4096, I=1024) in
TFLOP/s against the fp8 dense peak and against the HBM roofline, the
roofline of the dominant decode kernel, and the CPU oracle timed on a bounded
sample of the headline workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-prefill]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, TFLOP/s
FLUSH_BYTES = 1 << 30          # > 256 MB Infinity Cache + 8 x 4 MB L2


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Timer:
    """Per-launch HIP event pairs on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append([e, None])

    def stop(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs[-1][1] = e

    def us(self):
        self.torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1000.0 for a, b in self.pairs]


def make_flush(torch):
    buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    buf.zero_()

    def flush():
        buf.add_(1.0)
    return flush


def decode_bench(torch, m, wl, H, I, S, topk, active, steps, warmup, flush, ring=16, seed=1):
    """Returns dict with cold/warm us per step for one (H, I, active)."""
    dev = torch.device("cuda")
    w13_q, w13_s = wl.block_fp8_weights(S, 2 * I, H, seed * 7 + 11, device=dev)
    w2_q, w2_s = wl.block_fp8_weights(S, H, I, seed * 7 + 13, device=dev)
    sets = []
    for i in range(ring):
        x = wl.bf16_normal((1, H), seed=1000 + i, device=dev)
        slots, w = wl.decode_slots(1, topk, S, active, seed=2000 + i)
        sets.append((x, torch.from_numpy(slots).to(dev), torch.from_numpy(w).to(dev),
                     torch.empty((1, H), dtype=torch.bfloat16, device=dev)))
    ws = m.fused_decode_workspace(1, H, I, topk, device=dev)
    torch.cuda.synchronize()
    graphs = []
    cap = torch.cuda.Stream()
    for x, sl, w, out in sets:
        m.fused_decode(x, sl, w, w13_q, w13_s, w2_q, w2_s, ws, out)      # eager warm-up
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            m.fused_decode(x, sl, w, w13_q, w13_s, w2_q, w2_s, ws, out)
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(warmup):
        graphs[i % ring].replay()
    torch.cuda.synchronize()
    # cold: flush before each step, events around the step only
    t = Timer(torch)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(steps):
        flush()
        t.start()
        graphs[i % ring].replay()
        t.stop()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    cold = t.us()
    # warm: back-to-back replays, no flush
    t2 = Timer(torch)
    for i in range(steps):
        t2.start()
        graphs[i % ring].replay()
        t2.stop()
    warm = t2.us()
    per_route = wl.nbytes_expert(H, I)
    nbytes = active * per_route
    res = dict(H=H, I=I, slots=S, topk=topk, active=active,
               us_cold_mean=statistics.fmean(cold), us_cold_median=statistics.median(cold),
               us_warm_median=statistics.median(warm), bytes_streamed=nbytes,
               wall_ms_per_iter_incl_flush=wall * 1000.0 / steps)
    res["hbm_gbs_cold"] = nbytes / (res["us_cold_mean"] * 1e-6) / 1e9 if nbytes else 0.0
    res["hbm_frac_cold"] = res["hbm_gbs_cold"] / HBM_PEAK_GBS
    del graphs, w13_q, w2_q
    return res


def gateup_kernel_roofline(torch, m, wl, H, I, S, topk, steps, flush):
    """Dominant decode kernel: the slot-mode block-FP8 gate/up GEMM over 8 active routes,
    one launch per event pair, cold cache."""
    dev = torch.device("cuda")
    w13_q, w13_s = wl.block_fp8_weights(S, 2 * I, H, 77, device=dev)
    a_q, a_s = wl.fp8_rows(1, H, seed=78, device=dev)
    slot_sets = [torch.from_numpy(wl.decode_slots(1, topk, S, topk, seed=3000 + i)[0].reshape(-1)).to(dev)
                 for i in range(16)]
    out = torch.empty((topk, 2 * I), dtype=torch.float32, device=dev)
    for i in range(5):
        m.bf8_grouped_gemm(a_q, a_s, w13_q, w13_s, out, mode=m.MOE_MODE_SLOT, slot_ids=slot_sets[i % 16],
                           a_row_div=topk)
    t = Timer(torch)
    for i in range(steps):
        flush()
        t.start()
        m.bf8_grouped_gemm(a_q, a_s, w13_q, w13_s, out, mode=m.MOE_MODE_SLOT, slot_ids=slot_sets[i % 16],
                           a_row_div=topk)
        t.stop()
    us = statistics.fmean(t.us())
    per_route = 2 * I * H + 4 * math.ceil(2 * I / 128) * math.ceil(H / 128)
    nbytes = topk * per_route
    achieved = nbytes / (us * 1e-6) / 1e9
    return dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s", frac=achieved / HBM_PEAK_GBS,
                traffic=None, kernel="slot_gemv_kernel<f32, fp8 A> (gate/up, 8 routes, H=%d, 2I=%d)" % (H, 2 * I),
                bytes_per_launch=nbytes, us_per_launch=us)


def gather_bench(torch, m, wl, k, tokens, topk, steps, flush):
    dev = torch.device("cuda")
    src_q, src_s, mp = wl.gather_case(k, tokens, topk, seed=5)
    src_q = torch.from_numpy(src_q).to(dev)
    src_s = torch.from_numpy(src_s).to(dev).view(torch.float32)
    mp_d = torch.from_numpy(mp).to(dev)
    g = src_s.shape[1]
    dq = torch.empty((len(mp), k), dtype=torch.uint8, device=dev)
    ds = torch.empty((len(mp), g), dtype=torch.float32, device=dev)
    for _ in range(5):
        m.gather_rows_scales(src_q, src_s, mp_d, dq, ds)
    t = Timer(torch)
    for _ in range(steps):
        flush()
        t.start()
        m.gather_rows_scales(src_q, src_s, mp_d, dq, ds)
        t.stop()
    us = statistics.median(t.us())
    row = k + 4 * g
    nbytes = len(mp) * row + len(set(mp.tolist())) * row
    return dict(k=k, tokens=tokens, rows=len(mp), us_median=us, bytes=nbytes,
                gbs=nbytes / (us * 1e-6) / 1e9, hbm_frac=nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS)


def prefill_bench(torch, m, wl, T, E, topk, H, I, steps, flush):
    dev = torch.device("cuda")
    rt = wl.prefill_routes(T, E, topk, seed=9)
    R = T * topk
    offs = torch.from_numpy(rt.expert_offsets).to(dev)
    w13_q, w13_s = wl.block_fp8_weights(E, 2 * I, H, 21, device=dev, chunk_experts=32)
    w2_q, w2_s = wl.block_fp8_weights(E, H, I, 22, device=dev, chunk_experts=32)
    a1_q, a1_s = wl.fp8_rows(R, H, seed=23, device=dev)
    a2_q, a2_s = wl.fp8_rows(R, I, seed=24, device=dev)
    c1 = torch.empty((R, 2 * I), dtype=torch.bfloat16, device=dev)
    c2 = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    touched = int((rt.expert_offsets[1:] > rt.expert_offsets[:-1]).sum())
    bm = m.pick_block_m(R, E)
    out = {}
    for name, (a_q, a_s, w_q, w_s, c, N, K) in {
            "gate_up": (a1_q, a1_s, w13_q, w13_s, c1, 2 * I, H),
            "down": (a2_q, a2_s, w2_q, w2_s, c2, H, I)}.items():
        for _ in range(3):
            m.bf8_grouped_gemm(a_q, a_s, w_q, w_s, c, mode=m.MOE_MODE_GROUPED, expert_offsets=offs)
        t = Timer(torch)
        for _ in range(steps):
            flush()
            t.start()
            m.bf8_grouped_gemm(a_q, a_s, w_q, w_s, c, mode=m.MOE_MODE_GROUPED, expert_offsets=offs)
            t.stop()
        us = statistics.median(t.us())
        flops = 2.0 * R * N * K
        nbytes = touched * (N * K + 4 * (N // 128) * (K // 128)) + R * (K + 4 * K // 128) + R * N * 2
        tflops = flops / (us * 1e-6) / 1e12
        ai = flops / nbytes
        attainable = min(FP8_PEAK_TFLOPS, ai * HBM_PEAK_GBS / 1000.0)
        out[name] = dict(us_median=us, tflops=tflops, fp8_peak_frac=tflops / FP8_PEAK_TFLOPS,
                         roofline_frac=tflops / attainable, arithmetic_intensity=ai, bytes=nbytes,
                         hbm_gbs=nbytes / (us * 1e-6) / 1e9)
    del w13_q, w2_q
    return dict(routes=R, experts=E, topk=topk, H=H, I=I, block_m=bm, **out)


def cpu_baseline(wl, budget_s=12.0):
    """The CPU oracle on the headline workload, one thread, repeated for about budget_s seconds."""
    import numpy as np
    import torch
    import oracle
    c = wl.decode_case(H=2048, I=768, topk=8, n_slots=64, active=8, seed=1)
    xb = c.x.view(torch.int16).numpy().view(np.uint16)
    args = [t.numpy() for t in (c.w13_q, c.w13_s, c.w2_q, c.w2_s)]
    oracle.fused_decode(xb, c.slot_ids, c.weights, *args)
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        oracle.fused_decode(xb, c.slot_ids, c.weights, *args)
        n += 1
    dt = time.perf_counter() - t0
    return dict(value=dt / n * 1e6, unit="us/step", cores=1, kind="oracle",
                sample="%d decode steps (bs=1, H=2048, I=768, 64 slots, 8/8 active), single-threaded C oracle" % n)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--skip-prefill", action="store_true")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--only-headline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only; --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import moe_routed_expert_amd as m
    import workloads as wl
    m.lib()
    torch.cuda.init()
    flush = make_flush(torch)

    log("decode H=2048 I=768 8/8 (headline)")
    head = decode_bench(torch, m, wl, 2048, 768, 64, 8, 8, args.steps, args.warmup, flush)
    extra = {"decode": [head]}
    roof = None
    if not args.only_headline:
        for (H, I) in ((2048, 768), (4096, 1024)):
            for active in ((4, 2, 0) if H == 2048 else (8, 4, 2, 0)):
                log("decode H=%d I=%d %d/8" % (H, I, active))
                extra["decode"].append(decode_bench(torch, m, wl, H, I, 64, 8, active, max(50, args.steps // 2),
                                                    10, flush))
        log("gate/up kernel roofline")
        roof = gateup_kernel_roofline(torch, m, wl, 2048, 768, 64, 8, args.steps, flush)
        log("gather")
        extra["gather"] = [gather_bench(torch, m, wl, 7168, t, 8, 100, flush) for t in (1, 64, 1024)]
        if not args.skip_prefill:
            log("prefill 24576 routes")
            extra["prefill"] = prefill_bench(torch, m, wl, 4096, 256, 6, 4096, 1024, 20, flush)
    cpu = None
    if not args.skip_cpu:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(wl)
    line = {
        "metric": "bs1 decode us/step & HBM GB/s (top-k 8); prefill fp8 TFLOP/s vs peak",
        "value": round(head["us_cold_mean"], 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["us_cold_mean"] / 1000.0,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic (seeded N(0,0.02) block-FP8 expert banks, N(0,1) bf16 activations)",
        "config": {"workload": "decode bs=1, H=2048, I=768, 64-slot pool, top-k 8, 8/8 active, cold cache",
                   "hbm_gbs": round(head["hbm_gbs_cold"], 1), "hbm_frac": round(head["hbm_frac_cold"], 4)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
