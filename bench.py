"""Benchmark of the MI355X routed-expert hot path; prints ONE JSON line.

Headline (value): one batch-1 decode step of the routed experts, H=2048,
I=768, a 64-slot expert pool, top-k 8 with 8/8 routes active: x quant ->
gate/up -> SiLU*up requant -> down -> top-k reduce.  Steps are timed the way
they run inside a model: a captured hipGraph of L=16 chained decode layers
(layer l+1 takes layer l's output as its token row), each layer with its own
64-slot expert pool, so the 16 pools (4.8 GB) cannot sit in the 256 MB
Infinity Cache and every step streams its experts from HBM.  HIP events on
the stream bracket five windows of back-to-back graph replays (the timed
max(5, ceil(steps/16)) replays, at least 4 per window, split five ways); a
step is window time / (replays x 16), and the headline is the median window,
the pages' method (their five ~100 ms windows are reported beside it).
Inputs are resident in HBM before the timed region; after timing, the
workspace's error word must be clear and the first layer's output must match
the oracle.

Also reported: 4/2/0 active routes and H=4096, I=1024 (time vs active
routes), the fused gather (k=7168 with 8, 64, 512 and 8192 rows; k=896 with
512 rows) timed the same way, the grouped prefill GEMMs at 1536, 6144 and
24576 routes (E=256, top-6, H=4096, I=1024) in TFLOP/s against the fp8 dense
peak and against the HBM roofline, from row-major banks and from the same banks
in the GEMMs' packed order (moe_pack_weights, a one-time copy), the
roofline of the dominant kernel (the single fused decode kernel), and the
CPU oracle timed on a bounded sample of the headline workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-prefill] [--skip-cpu]
       python bench.py --only-headline [--active A] | --only-prefill | --only-gather | --only-stream
                                                                         (for counter passes)
       python bench.py --sweep-bm     (every M tile at the three prefill densities, checked, then timed)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, TFLOP/s


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


def settle(torch, fn, min_ms=60.0, min_calls=3):
    """Untimed calls of fn back to back (a sync every 4) until min_ms of wall time and min_calls have passed.
    In a fresh process the first tens of calls of a memory-bound kernel run up to a third slower than the
    same calls later (the 24576-route gate/up: 583 -> 441 us over about 60 calls, one box), so each timed
    section starts from that steady state rather than from 3 calls."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while n < min_calls or (time.perf_counter() - t0) * 1e3 < min_ms:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


LAYERS = 16

DECODE_SOURCES = ("moe_routed_expert_amd/csrc/fused_decode.hip", "moe_routed_expert_amd/csrc/device.h",
                  "moe_routed_expert_amd/csrc/decode_args.h")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "decode_h2048_i768_top8_pmc.md")


def sources_sha256(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode step from the committed FETCH_SIZE/WRITE_SIZE summary, or None when the
    summary is absent or was taken from other kernel sources."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    m = re.search(r"^TRAFFIC (\{.*\})$", text, flags=re.M)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("sources_sha256") != sources_sha256(DECODE_SOURCES):
        return None
    return rec


def copy_calibration(torch, m):
    """One plain copy of known size: the gather entry point with an identity map moves 16384 rows of
    4096 bytes plus 32 scale words each (64 MiB + 2 MiB read, the same written)."""
    dev = torch.device("cuda")
    n, k, g = 16384, 4096, 32
    src_q = torch.randint(0, 256, (n, k), dtype=torch.uint8, device=dev)
    src_s = torch.rand((n, g), dtype=torch.float32, device=dev)
    dst_q, dst_s = torch.empty_like(src_q), torch.empty_like(src_s)
    ident = torch.arange(n, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    m.gather_rows_scales(src_q, src_s, ident, dst_q, dst_s)
    torch.cuda.synchronize()
    assert torch.equal(dst_q, src_q)
    return dict(rows=n, k=k, g=g, bytes_read=n * (k + 4 * g), bytes_written=n * (k + 4 * g))


def decode_pools(torch, wl, H, I, S, seed):
    dev = torch.device("cuda")
    pools = []
    for l in range(LAYERS):
        w13_q, w13_s = wl.block_fp8_weights(S, 2 * I, H, seed * 1000 + 2 * l, device=dev, chunk_experts=16)
        w2_q, w2_s = wl.block_fp8_weights(S, H, I, seed * 1000 + 2 * l + 1, device=dev, chunk_experts=16)
        pools.append((w13_q, w13_s, w2_q, w2_s))
    return pools


def decode_check(torch, m, wl, x0, route, pool, out, H, I, topk):
    """The first layer's output of the timed graph against the oracle: the active slots' weights are copied to
    the host (the rest of the pool is never read) and the oracle runs on that compacted bank.  Returns the
    (rel L2, max abs / max|oracle|) pair; raises when the output breaks the pages' tolerance."""
    import numpy as np
    import oracle
    slots = route[0].cpu().numpy().astype(np.int32)
    w = route[1].cpu().numpy().astype(np.float32)
    act = sorted(set(int(v) for v in slots.reshape(-1) if v >= 0))
    remap = {v: i for i, v in enumerate(act)}
    small = np.array([[remap[int(v)] if v >= 0 else -1 for v in row] for row in slots], np.int32)
    idx = torch.tensor(act if act else [0], dtype=torch.long, device=pool[0].device)
    bank = [t.index_select(0, idx).cpu().numpy() for t in pool]
    xb = x0.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.bf16_decode(oracle.fused_decode(xb, small, w, *bank)).astype(np.float64)
    got = oracle.bf16_decode(out.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    peak = np.abs(ref).max()
    if peak == 0.0:
        if not np.all(got == 0.0):
            raise RuntimeError("decode output is not zero where the oracle's is")
        return 0.0, 0.0
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    mad = float(np.abs(got - ref).max() / peak)
    if not (rel <= 5e-3 and mad <= 2e-2):
        raise RuntimeError("decode output differs from the oracle: rel L2 %.3e, max abs %.3e of peak" % (rel, mad))
    return rel, mad


def decode_error_word(torch, m, ws, T, H, I, topk):
    """The workspace's error word (0 = every hand-off of every call so far completed)."""
    off = m.fused_decode_workspace_layout(T, H, I, topk)["ctl"]
    return int(ws[off:off + 4].view(torch.int32).item())


def decode_bench(torch, m, wl, pools, H, I, S, topk, active, reps, warmup, pages_windows=True):
    """A graph of LAYERS chained decode steps, timed as on the pages: the median of five windows of
    back-to-back graph replays, one event pair per window.  The timed steps are split into the five
    windows (max(4, ceil(reps/5)) replays each; value = the median window's time per step); the pages' exact form,
    five windows of about 100 ms each, is reported beside it.  After timing, the workspace's error word must
    be clear and the first layer's output must match the oracle."""
    dev = torch.device("cuda")
    x0 = wl.bf16_normal((1, H), seed=7, device=dev)
    outs = [torch.empty((1, H), dtype=torch.bfloat16, device=dev) for _ in range(LAYERS)]
    routes = []
    for l in range(LAYERS):
        sl, w = wl.decode_slots(1, topk, S, active, seed=5000 + 97 * l + active)
        routes.append((torch.from_numpy(sl).to(dev), torch.from_numpy(w).to(dev)))
    ws = m.fused_decode_workspace(1, H, I, topk, device=dev)

    def step_all():
        x = x0
        for l in range(LAYERS):
            m.fused_decode(x, routes[l][0], routes[l][1], *pools[l], ws, outs[l])
            x = outs[l]

    step_all()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        step_all()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()

    def windows(n_win, per_window):
        out = []
        for _ in range(n_win):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(per_window):
                g.replay()
            b.record()
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b) * 1000.0 / (per_window * LAYERS))
        return out

    per_win = max(4, -(-reps // 5))      # at least 4 back-to-back replays (64 steps) per window
    wall0 = time.perf_counter()
    timed = windows(5, per_win)
    wall = time.perf_counter() - wall0
    med = statistics.median(timed)
    # the pages' method as printed: five windows of about 100 ms (left out of counter passes)
    per_100ms = max(1, int(100e3 / (med * LAYERS))) if pages_windows else 0
    pages = windows(5, per_100ms) if pages_windows else [float("nan")]
    err = decode_error_word(torch, m, ws, 1, H, I, topk)
    if err != 0:
        raise RuntimeError("decode H=%d I=%d %d/8: the workspace error word is %d after timing" % (H, I, active, err))
    rel, mad = decode_check(torch, m, wl, x0, routes[0], pools[0], outs[0], H, I, topk)
    nbytes = active * wl.nbytes_expert(H, I)
    res = dict(H=H, I=I, slots=S, topk=topk, active=active, layers_per_graph=LAYERS, windows=5,
               replays_per_window=per_win, steps_timed=5 * per_win * LAYERS,
               us_per_step_median=med, us_per_step_windows=timed, us_per_step_min=min(timed),
               us_per_step_max=max(timed), us_per_step_100ms_windows_median=statistics.median(pages),
               steps_per_100ms_window=per_100ms * LAYERS,
               bytes_streamed=nbytes, hbm_gbs=nbytes / (med * 1e-6) / 1e9 if nbytes else 0.0,
               wall_us_per_step=wall * 1e6 / (5 * per_win * LAYERS), error_word=err,
               check_layer0=dict(rel_l2=rel, max_abs_frac=mad))
    res["hbm_frac"] = res["hbm_gbs"] / HBM_PEAK_GBS
    del g
    return res


def active_fit(rows):
    """Least-squares fit t(a) = t0 + a * tau over the decode rows of one shape (a = active routes)."""
    a = [r["active"] for r in rows]
    t = [r["us_per_step_median"] for r in rows]
    n = len(a)
    ma, mt = sum(a) / n, sum(t) / n
    saa = sum((x - ma) ** 2 for x in a)
    tau = sum((x - ma) * (y - mt) for x, y in zip(a, t)) / saa
    t0 = mt - tau * ma
    ss_res = sum((y - (t0 + tau * x)) ** 2 for x, y in zip(a, t))
    ss_tot = sum((y - mt) ** 2 for y in t)
    return dict(H=rows[0]["H"], I=rows[0]["I"], actives=a, t0_us=t0, tau_us_per_route=tau,
                r2=1.0 - ss_res / ss_tot if ss_tot else 1.0,
                tau_gbs=(rows[0]["bytes_streamed"] / rows[0]["active"]) / (tau * 1e-6) / 1e9
                if rows[0]["active"] and tau > 0 else None)


def launch_floor(torch, reps=20):
    """The empty-kernel floor beside the small gathers: 16 launches of a one-element fill (torch's own
    kernel) in one graph, timed like the gathers (graph replay / 16)."""
    dev = torch.device("cuda")
    bufs = [torch.empty(1, dtype=torch.int32, device=dev) for _ in range(LAYERS)]
    for b in bufs:
        b.fill_(1)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=torch.cuda.Stream()):
        for b in bufs:
            b.fill_(1)
    settle(torch, gr.replay)
    t = Timer(torch)
    for _ in range(reps):
        t.start()
        gr.replay()
        t.stop()
    return dict(kernel="one-element fill, 16 per graph", us_per_launch=statistics.median(t.us()) / LAYERS)


def gather_all(torch, m, wl):
    """The gather at k=7168 for 1, 8, 64 and 1024 tokens (top-8) and at k=896 for 64 tokens."""
    rows = [gather_bench(torch, m, wl, 7168, t, 8, 20) for t in (1, 8, 64, 1024)]
    rows.append(gather_bench(torch, m, wl, 896, 64, 8, 20))
    return rows


def gather_bench(torch, m, wl, k, tokens, topk, reps):
    """16 gathers over 16 disjoint source/destination sets in one graph (cold by construction)."""
    dev = torch.device("cuda")
    sets = []
    for i in range(LAYERS):
        src_q, src_s, mp = wl.gather_case(k, tokens, topk, seed=50 + i)
        g = src_s.shape[1]
        sets.append((torch.from_numpy(src_q).to(dev), torch.from_numpy(src_s).to(dev).view(torch.float32),
                     torch.from_numpy(mp).to(dev), torch.empty((len(mp), k), dtype=torch.uint8, device=dev),
                     torch.empty((len(mp), g), dtype=torch.float32, device=dev), mp))

    def run_all():
        for sq, ss, mp_d, dq, ds, _ in sets:
            m.gather_rows_scales(sq, ss, mp_d, dq, ds)

    run_all()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=torch.cuda.Stream()):
        run_all()
    n_settle = settle(torch, gr.replay)
    t = Timer(torch)
    for _ in range(reps):
        t.start()
        gr.replay()
        t.stop()
    us = statistics.median(t.us()) / LAYERS
    row = k + 4 * sets[0][1].shape[1]
    mp = sets[0][5]
    nbytes = len(mp) * row + len(set(mp.tolist())) * row
    return dict(k=k, tokens=tokens, rows=len(mp), us_per_call=us, bytes=nbytes, settle_replays=n_settle, timed_replays=reps,
                gbs=nbytes / (us * 1e-6) / 1e9, hbm_frac=nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS)


def prefill_weights(torch, wl, E, H, I):
    dev = torch.device("cuda")
    w13 = wl.block_fp8_weights(E, 2 * I, H, 21, device=dev, chunk_experts=32)
    w2 = wl.block_fp8_weights(E, H, I, 22, device=dev, chunk_experts=32)
    return w13, w2


def packed_banks(m, weights, step):
    """The same banks in the GEMMs' packed order (moe_pack_weights), scales shared."""
    (w13, w13_s), (w2, w2_s) = weights
    return (m.pack_weights(w13, step), w13_s), (m.pack_weights(w2, step), w2_s)


def prefill_bench(torch, m, wl, T, E, topk, H, I, steps, weights, packed=False):
    """The block-FP8 gate/up and down GEMMs and the fused gate/up requant; `packed`: banks in the packed
    order (moe_pack_weights)."""
    dev = torch.device("cuda")
    rt = wl.prefill_routes(T, E, topk, seed=9)
    R = T * topk
    offs = torch.from_numpy(rt.expert_offsets).to(dev)
    (w13_q, w13_s), (w2_q, w2_s) = weights
    a1_q, a1_s = wl.fp8_rows(R, H, seed=23, device=dev)
    a2_q, a2_s = wl.fp8_rows(R, I, seed=24, device=dev)
    c1 = torch.empty((R, 2 * I), dtype=torch.bfloat16, device=dev)
    c2 = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    touched = int((rt.expert_offsets[1:] > rt.expert_offsets[:-1]).sum())
    bm = m.grouped_block_m(R, E, H, packed=packed)
    out = {}
    for name, (a_q, a_s, w_q, w_s, c, N, K) in {
            "gate_up": (a1_q, a1_s, w13_q, w13_s, c1, 2 * I, H),
            "down": (a2_q, a2_s, w2_q, w2_s, c2, H, I)}.items():
        n_settle = settle(torch, lambda: m.bf8_grouped_gemm(a_q, a_s, w_q, w_s, c, mode=m.MOE_MODE_GROUPED,
                                                            expert_offsets=offs, w_packed=packed))
        t = Timer(torch)
        for _ in range(steps):          # 2-3 GB of weights per call: cold by construction
            t.start()
            m.bf8_grouped_gemm(a_q, a_s, w_q, w_s, c, mode=m.MOE_MODE_GROUPED, expert_offsets=offs, w_packed=packed)
            t.stop()
        us = statistics.median(t.us())
        flops = 2.0 * R * N * K
        nbytes = touched * (N * K + 4 * (N // 128) * (K // 128)) + R * (K + 4 * K // 128) + R * N * 2
        tflops = flops / (us * 1e-6) / 1e12
        ai = flops / nbytes
        attainable = min(FP8_PEAK_TFLOPS, ai * HBM_PEAK_GBS / 1000.0)
        out[name] = dict(us_median=us, tflops=tflops, fp8_peak_frac=tflops / FP8_PEAK_TFLOPS,
                         roofline_frac=tflops / attainable, arithmetic_intensity=ai, bytes=nbytes,
                         hbm_gbs=nbytes / (us * 1e-6) / 1e9, settle_calls=n_settle, timed_calls=steps)
    # gate/up with the SiLU-mul requant fused into its epilogue, against the unfused pair (gate/up above
    # writing bf16 c1, then act_quant reading it)
    aq = torch.empty((R, I), dtype=torch.uint8, device=dev)
    as_ = torch.empty((R, I // 128), dtype=torch.float32, device=dev)
    n_settle_f = settle(torch, lambda: m.bf8_grouped_gemm_act_quant(a1_q, a1_s, w13_q, w13_s, offs, aq, as_,
                                                                   w_packed=packed))
    t = Timer(torch)
    for _ in range(steps):
        t.start()
        m.bf8_grouped_gemm_act_quant(a1_q, a1_s, w13_q, w13_s, offs, aq, as_, w_packed=packed)
        t.stop()
    us_f = statistics.median(t.us())
    settle(torch, lambda: m.act_quant(c1, aq, as_, act=m.MOE_ACT_SILU_MUL))
    t = Timer(torch)
    for _ in range(steps):
        t.start()
        m.act_quant(c1, aq, as_, act=m.MOE_ACT_SILU_MUL)
        t.stop()
    us_a = statistics.median(t.us())
    flops = 2.0 * R * 2 * I * H
    out["gate_up_act_quant"] = dict(us_median=us_f, tflops=flops / (us_f * 1e-6) / 1e12,
                                     unfused_us=out["gate_up"]["us_median"] + us_a, act_quant_us=us_a,
                                     settle_calls=n_settle_f, timed_calls=steps)
    return dict(routes=R, experts=E, topk=topk, H=H, I=I, block_m=bm,
                block_m_fused=m.grouped_block_m(R, E, H, packed=packed, fused=True),
                block_m_down=m.grouped_block_m(R, E, I, packed=packed), **out)


def prefill_mxfp4_bench(torch, m, wl, T, E, topk, H, I, steps, weights, packed=False):
    """The grouped GEMMs with MXFP4 expert weights (E2M1 codes, an E8M0 scale per 32 K) on the same routes:
    gate/up with the SiLU-mul requant fused, gate/up to bf16, and down to bf16."""
    dev = torch.device("cuda")
    rt = wl.prefill_routes(T, E, topk, seed=9)
    R = T * topk
    offs = torch.from_numpy(rt.expert_offsets).to(dev)
    (w13, w13_s), (w2, w2_s) = weights
    a1_q, a1_s = wl.fp8_rows(R, H, seed=23, device=dev)
    a2_q, a2_s = wl.fp8_rows(R, I, seed=24, device=dev)
    c1 = torch.empty((R, 2 * I), dtype=torch.bfloat16, device=dev)
    c2 = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    aq = torch.empty((R, I), dtype=torch.uint8, device=dev)
    as_ = torch.empty((R, I // 128), dtype=torch.float32, device=dev)
    touched = int((rt.expert_offsets[1:] > rt.expert_offsets[:-1]).sum())
    calls = {
        "gate_up_act_quant": (lambda: m.mxfp4_grouped_gemm_act_quant(a1_q, a1_s, w13, w13_s, offs, aq, as_,
                                                                     w_packed=packed),
                              2 * I, H, R * (I + 4 * I // 128)),
        "gate_up": (lambda: m.mxfp4_grouped_gemm(a1_q, a1_s, w13, w13_s, offs, c1, w_packed=packed), 2 * I, H,
                    R * 2 * I * 2),
        "down": (lambda: m.mxfp4_grouped_gemm(a2_q, a2_s, w2, w2_s, offs, c2, w_packed=packed), H, I, R * H * 2),
    }
    out = {}
    for name, (fn, N, K, out_bytes) in calls.items():
        n_settle = settle(torch, fn)
        t = Timer(torch)
        for _ in range(steps):
            t.start()
            fn()
            t.stop()
        us = statistics.median(t.us())
        flops = 2.0 * R * N * K
        nbytes = touched * (N * K // 2 + N * K // 32) + R * (K + 4 * K // 128) + out_bytes
        tflops = flops / (us * 1e-6) / 1e12
        ai = flops / nbytes
        attainable = min(FP8_PEAK_TFLOPS, ai * HBM_PEAK_GBS / 1000.0)
        out[name] = dict(us_median=us, tflops=tflops, fp8_peak_frac=tflops / FP8_PEAK_TFLOPS,
                         roofline_frac=tflops / attainable, arithmetic_intensity=ai, bytes=nbytes,
                         hbm_gbs=nbytes / (us * 1e-6) / 1e9, settle_calls=n_settle, timed_calls=steps)
    return dict(routes=R, experts=E, topk=topk, H=H, I=I,
                block_m=m.grouped_block_m(R, E, H, mxfp4=True, packed=packed),
                block_m_fused=m.grouped_block_m(R, E, H, mxfp4=True, packed=packed, fused=True),
                block_m_down=m.grouped_block_m(R, E, I, mxfp4=True, packed=packed),
                weights="MXFP4 (E2M1 + E8M0 per 32 K)", **out)


def prefill_layer_bench(torch, m, wl, T, E, topk, H, I, steps, weights, packed=False):
    """One whole prefill layer on the device from router logits: routing prep, input quant, gather,
    fused gate/up + SiLU-mul requant, down GEMM, top-k reduce (timed per layer with events)."""
    dev = torch.device("cuda")
    (w13_q, w13_s), (w2_q, w2_s) = weights
    R = T * topk
    # iid N(0,1) logits: each token's top-k is a uniform draw of distinct experts, as in the GEMM lines
    lg = torch.from_numpy(wl.router_logits(T, E, seed=41, skew=0.0)).to(dev)
    x = wl.bf16_normal((T, H), seed=42, device=dev)
    ids = torch.empty((T, topk), dtype=torch.int32, device=dev)
    w = torch.empty((T, topk), dtype=torch.float32, device=dev)
    d2s = torch.empty(R, dtype=torch.int32, device=dev)
    rr = torch.empty(R, dtype=torch.int32, device=dev)
    offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
    ws_size = m.lib().moe_route_prep_workspace_size(T, E)
    ws = torch.empty(ws_size, dtype=torch.uint8, device=dev)
    xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
    xs = torch.empty((T, H // 128), dtype=torch.float32, device=dev)
    gq = torch.empty((R, H), dtype=torch.uint8, device=dev)
    gs = torch.empty((R, H // 128), dtype=torch.float32, device=dev)
    aq = torch.empty((R, I), dtype=torch.uint8, device=dev)
    as_ = torch.empty((R, I // 128), dtype=torch.float32, device=dev)
    c2 = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    def layer():
        st = torch.cuda.current_stream().cuda_stream
        rc = m.lib().moe_route_prep(lg.data_ptr(), E, T, E, topk, ids.data_ptr(), w.data_ptr(), d2s.data_ptr(),
                                    rr.data_ptr(), offs.data_ptr(), ws.data_ptr(), ws_size, st)
        assert rc == 0, rc
        m.act_quant(x, xq, xs)
        m.gather_rows_scales(xq, xs, d2s, gq, gs)
        m.bf8_grouped_gemm_act_quant(gq, gs, w13_q, w13_s, offs, aq, as_, w_packed=packed)
        m.bf8_grouped_gemm(aq, as_, w2_q, w2_s, c2, mode=m.MOE_MODE_GROUPED, expert_offsets=offs, w_packed=packed)
        m.topk_reduce(c2, ids, w, out, route_rows=rr)

    n_settle = settle(torch, layer)
    t = Timer(torch)
    for _ in range(steps):
        t.start()
        layer()
        t.stop()
    us = statistics.median(t.us())
    flops = 2.0 * R * (2 * I * H + H * I)
    return dict(tokens=T, routes=R, experts=E, topk=topk, H=H, I=I, us_per_layer=us,
                gemm_tflops=flops / (us * 1e-6) / 1e12, routing="uniform (iid N(0,1) logits)",
                settle_calls=n_settle, timed_calls=steps)


def prefill_all(torch, m, wl):
    """The grouped GEMMs at 1536, 6144 and 24576 routes (E=256, top-6, H=4096, I=1024), with block-FP8 and
    with MXFP4 expert weights."""
    weights = prefill_weights(torch, wl, 256, 4096, 1024)
    packed = packed_banks(m, weights, 128)
    res = []
    for T in (256, 1024, 4096):
        log("prefill %d routes" % (T * 6))
        res.append(prefill_bench(torch, m, wl, T, 256, 6, 4096, 1024, 10, weights))
        res[-1]["layer"] = prefill_layer_bench(torch, m, wl, T, 256, 6, 4096, 1024, 10, weights)
        res[-1]["packed"] = prefill_bench(torch, m, wl, T, 256, 6, 4096, 1024, 10, packed, packed=True)
        res[-1]["packed"]["layer"] = prefill_layer_bench(torch, m, wl, T, 256, 6, 4096, 1024, 10, packed,
                                                         packed=True)
    del weights, packed
    torch.cuda.empty_cache()
    dev = torch.device("cuda")
    weights = (wl.mxfp4_weights(256, 2048, 4096, seed=31, device=dev), wl.mxfp4_weights(256, 4096, 1024, seed=32,
                                                                                        device=dev))
    packed = packed_banks(m, weights, 64)
    for i, T in enumerate((256, 1024, 4096)):
        log("prefill mxfp4 %d routes" % (T * 6))
        res[i]["mxfp4"] = prefill_mxfp4_bench(torch, m, wl, T, 256, 6, 4096, 1024, 10, weights)
        res[i]["mxfp4"]["packed"] = prefill_mxfp4_bench(torch, m, wl, T, 256, 6, 4096, 1024, 10, packed,
                                                        packed=True)
    del weights, packed
    torch.cuda.empty_cache()
    return res


def stream_ops_bench(torch, m, wl, reps=10):
    """The bandwidth-bound steps at the prefill sizes (T=4096 tokens, top-6, H=4096, I=1024): input quant
    of x [4096, 4096], the SiLU-mul requant of C1 [24576, 2048] (the unfused path) and the top-k reduce of
    C2 [24576, 4096]. Each runs in a graph over enough disjoint buffer sets (more than 256 MB in all) that
    no call finds its inputs in the GPU's caches; bytes = inputs read + outputs written."""
    dev = torch.device("cuda")
    T, topk, H, I = 4096, 6, 4096, 1024
    R = T * topk

    def timed(calls, nbytes):
        for c in calls:
            c()
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=torch.cuda.Stream()):
            for c in calls:
                c()
        settle(torch, gr.replay)
        t = Timer(torch)
        for _ in range(reps):
            t.start()
            gr.replay()
            t.stop()
        us = statistics.median(t.us()) / len(calls)
        del gr
        return dict(us_per_call=us, bytes=nbytes, gbs=nbytes / (us * 1e-6) / 1e9,
                    hbm_frac=nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS)

    res = {}
    sets = [(wl.bf16_normal((T, H), seed=60 + i, device=dev), torch.empty((T, H), dtype=torch.uint8, device=dev),
             torch.empty((T, H // 128), dtype=torch.float32, device=dev)) for i in range(6)]
    res["act_quant_identity"] = dict(rows=T, cols=H, **timed(
        [lambda s=s: m.act_quant(s[0], s[1], s[2]) for s in sets], T * H * 2 + T * H + T * (H // 128) * 4))
    del sets
    sets = [(wl.bf16_normal((R, 2 * I), seed=70 + i, device=dev), torch.empty((R, I), dtype=torch.uint8, device=dev),
             torch.empty((R, I // 128), dtype=torch.float32, device=dev)) for i in range(3)]
    res["act_quant_silu_mul"] = dict(rows=R, cols=I, **timed(
        [lambda s=s: m.act_quant(s[0], s[1], s[2], act=m.MOE_ACT_SILU_MUL) for s in sets],
        R * 2 * I * 2 + R * I + R * (I // 128) * 4))
    del sets
    sets = []
    for i in range(2):
        g = torch.Generator(device="cpu").manual_seed(80 + i)
        rows = torch.randperm(R, generator=g).to(torch.int32).view(T, topk).to(dev)
        ids = torch.zeros((T, topk), dtype=torch.int32, device=dev)          # every route active
        w = torch.rand((T, topk), generator=g).to(dev)
        sets.append((wl.bf16_normal((R, H), seed=90 + i, device=dev), ids, w,
                     torch.empty((T, H), dtype=torch.bfloat16, device=dev), rows))
    res["topk_reduce"] = dict(tokens=T, topk=topk, H=H, **timed(
        [lambda s=s: m.topk_reduce(s[0], s[1], s[2], s[3], route_rows=s[4]) for s in sets],
        R * H * 2 + T * H * 2 + T * topk * 12))
    del sets
    torch.cuda.empty_cache()
    return res


def route_prep_bench(torch, m, wl, T, E, topk, reps):
    """Device routing prep (top-k, weights, route maps) on skewed router logits: 16 calls over 16
    logit sets in one graph, so the time is the device's, not the host's launch latency."""
    dev = torch.device("cuda")
    size = m.lib().moe_route_prep_workspace_size(T, E)
    sets = []
    for i in range(LAYERS):
        sets.append(dict(lg=torch.from_numpy(wl.router_logits(T, E, seed=41 + i, skew=1.0)).to(dev),
                         ids=torch.empty((T, topk), dtype=torch.int32, device=dev),
                         w=torch.empty((T, topk), dtype=torch.float32, device=dev),
                         d2s=torch.empty(T * topk, dtype=torch.int32, device=dev),
                         rr=torch.empty(T * topk, dtype=torch.int32, device=dev),
                         offs=torch.empty(E + 1, dtype=torch.int32, device=dev),
                         ws=torch.empty(size, dtype=torch.uint8, device=dev)))

    def run_all():
        st = torch.cuda.current_stream().cuda_stream
        for b in sets:
            rc = m.lib().moe_route_prep(b["lg"].data_ptr(), E, T, E, topk, b["ids"].data_ptr(), b["w"].data_ptr(),
                                        b["d2s"].data_ptr(), b["rr"].data_ptr(), b["offs"].data_ptr(),
                                        b["ws"].data_ptr(), size, st)
            assert rc == 0, rc

    run_all()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=torch.cuda.Stream()):
        run_all()
    n_settle = settle(torch, gr.replay)
    t = Timer(torch)
    for _ in range(reps):
        t.start()
        gr.replay()
        t.stop()
    us = statistics.median(t.us()) / LAYERS
    nbytes = T * E * 4 + T * topk * (4 + 4 + 4 + 4) + T * topk * 4
    return dict(tokens=T, experts=E, topk=topk, us_per_call=us, bytes=nbytes, gbs=nbytes / (us * 1e-6) / 1e9,
                settle_replays=n_settle, timed_replays=reps)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def run_threads(fn, n):
    import threading
    th = [threading.Thread(target=fn, args=(i,)) for i in range(n)]
    for t in th:
        t.start()
    for t in th:
        t.join()


def cpu_baseline(wl, decode_s=8.0, single_s=2.0):
    """The CPU oracle, unchanged, on bounded samples of the workloads (its C calls release the GIL, so Python
    threads run it on several cores at once):
      * headline (value): decode steps of the headline workload on all of the host's cores (at most 16, one
        GPU's share of the host), one thread per core running whole steps back to back for decode_s seconds;
        value = wall time / steps completed;
      * the same step on one thread (median over single_s seconds of steps);
      * the 8192-row gather (k = 7168) on one thread and split over all cores;
      * the prefill GEMMs (gate/up and down) of the 6144-route workload for the rows of experts 0..31, on all
        cores, the work cut into (expert, 256-column N block) jobs."""
    import numpy as np
    import torch
    import oracle
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    c = wl.decode_case(H=2048, I=768, topk=8, n_slots=64, active=8, seed=1)
    xb = c.x.view(torch.int16).numpy().view(np.uint16)
    args = [t.numpy() for t in (c.w13_q, c.w13_s, c.w2_q, c.w2_s)]
    oracle.fused_decode(xb, c.slot_ids, c.weights, *args)
    # one thread
    single = []
    t_end = time.perf_counter() + single_s
    while time.perf_counter() < t_end or len(single) < 3:
        t0 = time.perf_counter()
        oracle.fused_decode(xb, c.slot_ids, c.weights, *args)
        single.append(time.perf_counter() - t0)
    # all cores
    counts = [0] * cores
    t0 = time.perf_counter()
    deadline = t0 + decode_s

    def worker(i):
        while time.perf_counter() < deadline:
            oracle.fused_decode(xb, c.slot_ids, c.weights, *args)
            counts[i] += 1

    run_threads(worker, cores)
    dt = time.perf_counter() - t0
    n = sum(counts)
    # gather: 8192 rows of 7168 bytes + 56 scale words
    src_q, src_s, mp = wl.gather_case(7168, 1024, 8, seed=50)
    src_s = src_s.view(np.float32)
    g1 = []
    for _ in range(3):
        t1 = time.perf_counter()
        oracle.gather_rows_scales(src_q, src_s, mp)
        g1.append(time.perf_counter() - t1)
    parts = np.array_split(mp, cores)
    t1 = time.perf_counter()
    run_threads(lambda i: oracle.gather_rows_scales(src_q, src_s, parts[i]), cores)
    g_all = time.perf_counter() - t1
    gbytes = len(mp) * (7168 + 4 * 56) + len(set(mp.tolist())) * (7168 + 4 * 56)
    # prefill sample: 6144 routes (T = 1024, E = 256, top-6), experts 0..31, gate/up then down
    E_s, H, I, T = 32, 4096, 1024, 1024
    rt = wl.prefill_routes(T, 256, 6, seed=9)
    r_end = int(rt.expert_offsets[E_s])
    w13_q, w13_s = (t.numpy() for t in wl.block_fp8_weights(E_s, 2 * I, H, 21, chunk_experts=32))
    w2_q, w2_s = (t.numpy() for t in wl.block_fp8_weights(E_s, H, I, 22, chunk_experts=32))
    a1_q, a1_s = (t.numpy()[:r_end] for t in wl.fp8_rows(T * 6, H, seed=23))
    a2_q, a2_s = (t.numpy()[:r_end] for t in wl.fp8_rows(T * 6, I, seed=24))
    jobs = []
    for e in range(E_s):
        r0, r1 = int(rt.expert_offsets[e]), int(rt.expert_offsets[e + 1])
        if r1 == r0:
            continue
        one = np.array([0, r1 - r0], np.int32)
        for n0 in range(0, 2 * I, 256):
            jobs.append((a1_q[r0:r1], a1_s[r0:r1], w13_q[e:e + 1, n0:n0 + 256], w13_s[e:e + 1, n0 // 128:n0 // 128 + 2],
                         one))
        for n0 in range(0, H, 256):
            jobs.append((a2_q[r0:r1], a2_s[r0:r1], w2_q[e:e + 1, n0:n0 + 256], w2_s[e:e + 1, n0 // 128:n0 // 128 + 2],
                         one))
    nxt = [0]
    import threading
    lock = threading.Lock()

    def gemm_worker(i):
        while True:
            with lock:
                j = nxt[0]
                nxt[0] += 1
            if j >= len(jobs):
                return
            a, sa, w, sw, o = jobs[j]
            oracle.block_gemm(a, sa, w, sw, mode=oracle.MODE_GROUPED, expert_offsets=o, out_dtype=np.uint16)

    t1 = time.perf_counter()
    run_threads(gemm_worker, cores)
    p_dt = time.perf_counter() - t1
    p_flops = 2.0 * r_end * (2 * I * H + H * I)
    return dict(value=dt / n * 1e6, unit="us/step", cores=cores, kind="oracle",
                sample="%d decode steps (bs=1, H=2048, I=768, 64 slots, 8/8 active) on %d threads of the C oracle, "
                       "%.1f s wall" % (n, cores, dt),
                cpu_model=cpu_model(), hardware_concurrency=os.cpu_count(), threads_used=cores,
                decode_single_thread_us_per_step=statistics.median(single) * 1e6,
                decode_single_thread_steps=len(single),
                gather_8192_rows=dict(k=7168, rows=len(mp), bytes=gbytes,
                                      single_thread_us=statistics.median(g1) * 1e6,
                                      all_cores_us=g_all * 1e6, threads=cores),
                prefill_sample=dict(routes_total=T * 6, experts="0..31", rows=r_end, gemms="gate/up (N=2048, K=4096) "
                                    "and down (N=4096, K=1024), bf16 out", jobs=len(jobs), threads=cores,
                                    seconds=p_dt, tflops=p_flops / p_dt / 1e12))


def bm_sweep(torch, m, wl, rounds=6):
    """Every M tile at six route densities (48 to 24576 routes over E = 256, top-6, H = 4096, I = 1024): the
    block-FP8 and MXFP4 gate/up (bf16 out), fused gate/up requant and down (bf16 out) GEMMs, each from a
    row-major and from a packed bank.  As on the page, each configuration's output is checked before its
    time counts: every tile and both layouts must give the output of the 16-row tile on the row-major bank
    bit for bit (a tile size or a layout changes which rows share a workgroup or where a weight byte sits,
    not the order of any output's sums), and for the plain GEMMs that output must match the oracle on the
    rows of the first and the last expert that has rows.  Times: the tiles take turns call by call with a
    sync between calls, `rounds` rounds, the first dropped; the median of the rest."""
    import numpy as np
    import oracle
    dev = torch.device("cuda")
    H, I, E = 4096, 1024, 256
    banks = {}
    res = []
    for fmt in ("fp8", "mxfp4"):
        if fmt == "fp8":
            (w13, w13_s), (w2, w2_s) = prefill_weights(torch, wl, E, H, I)
            step = 128
        else:
            (w13, w13_s), (w2, w2_s) = (wl.mxfp4_weights(E, 2 * I, H, seed=31, device=dev),
                                        wl.mxfp4_weights(E, H, I, seed=32, device=dev))
            step = 64
        p13, p2 = m.pack_weights(w13, step), m.pack_weights(w2, step)
        for T in (8, 32, 128, 256, 1024, 4096):
            R = T * 6
            rt = wl.prefill_routes(T, E, 6, seed=9)
            offs = torch.from_numpy(rt.expert_offsets).to(dev)
            a1_q, a1_s = wl.fp8_rows(R, H, seed=23, device=dev)
            a2_q, a2_s = wl.fp8_rows(R, I, seed=24, device=dev)
            nonempty = [e for e in range(E) if rt.expert_offsets[e + 1] > rt.expert_offsets[e]]
            row = dict(weights=fmt, routes=R, rows_per_expert=R / E, density_rule=m.pick_block_m(R, E), gemms={})
            for name in ("gate_up", "gate_up_act_quant", "down"):
                down = name == "down"
                a_q, a_s = (a2_q, a2_s) if down else (a1_q, a1_s)
                w_s = w2_s if down else w13_s
                N, K = (H, I) if down else (2 * I, H)
                fused = name == "gate_up_act_quant"

                def alloc():
                    if fused:
                        return (torch.empty((R, I), dtype=torch.uint8, device=dev),
                                torch.empty((R, I // 128), dtype=torch.float32, device=dev))
                    return (torch.empty((R, N), dtype=torch.bfloat16, device=dev),)

                def call(bm, packed, out):
                    w = (p2 if down else p13) if packed else (w2 if down else w13)
                    if fmt == "fp8" and fused:
                        m.bf8_grouped_gemm_act_quant(a_q, a_s, w, w_s, offs, out[0], out[1], block_m=bm, w_packed=packed)
                    elif fmt == "fp8":
                        m.bf8_grouped_gemm(a_q, a_s, w, w_s, out[0], mode=m.MOE_MODE_GROUPED, expert_offsets=offs,
                                           block_m=bm, w_packed=packed)
                    elif fused:
                        m.mxfp4_grouped_gemm_act_quant(a_q, a_s, w, w_s, offs, out[0], out[1], block_m=bm,
                                                       w_packed=packed)
                    else:
                        m.mxfp4_grouped_gemm(a_q, a_s, w, w_s, offs, out[0], block_m=bm, w_packed=packed)

                base = alloc()
                call(16, False, base)
                torch.cuda.synchronize()
                if not fused:
                    for e in (nonempty[0], nonempty[-1]):
                        r0, r1 = int(rt.expert_offsets[e]), int(rt.expert_offsets[e + 1])
                        one = np.array([0, r1 - r0], np.int32)
                        wq = (w2 if down else w13)[e:e + 1].cpu().numpy()
                        ws = w_s[e:e + 1].cpu().numpy()
                        aq, as_ = a_q[r0:r1].cpu().numpy(), a_s[r0:r1].cpu().numpy()
                        if fmt == "fp8":
                            ref = oracle.block_gemm(aq, as_, wq, ws, mode=oracle.MODE_GROUPED, expert_offsets=one,
                                                    out_dtype=np.uint16)
                        else:
                            ref = oracle.mxfp4_gemm(aq, as_, wq, ws, mode=oracle.MODE_GROUPED, expert_offsets=one,
                                                    out_dtype=np.uint16)
                        got = oracle.bf16_decode(base[0][r0:r1].view(torch.int16).cpu().numpy().view(np.uint16))
                        got, r = got.astype(float), oracle.bf16_decode(ref).astype(float)
                        rel = np.linalg.norm(got - r) / np.linalg.norm(r)
                        if not (rel <= 5e-3 and np.abs(got - r).max() <= 2e-2 * np.abs(r).max()):
                            raise RuntimeError("bm sweep: %s %s at %d routes, expert %d: rel L2 %.3e" % (
                                fmt, name, R, e, rel))
                for packed in (False, True):
                    outs = {bm: alloc() for bm in (16, 32, 64, 128)}
                    for bm in (16, 32, 64, 128):
                        call(bm, packed, outs[bm])
                        torch.cuda.synchronize()
                        for x, y in zip(outs[bm], base):
                            if not torch.equal(x.view(torch.uint8), y.view(torch.uint8)):
                                raise RuntimeError("bm sweep: %s %s at %d routes: BM=%d%s differs from BM=16" % (
                                    fmt, name, R, bm, " packed" if packed else ""))
                    ts = {bm: [] for bm in (16, 32, 64, 128)}
                    for rnd in range(rounds):
                        for bm in (16, 32, 64, 128):
                            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                            a.record()
                            call(bm, packed, outs[bm])
                            b.record()
                            torch.cuda.synchronize()
                            if rnd:
                                ts[bm].append(a.elapsed_time(b) * 1000.0)
                    times = {bm: statistics.median(v) for bm, v in ts.items()}
                    best = min(times, key=times.get)
                    lib = m.grouped_block_m(R, E, K, mxfp4=fmt == "mxfp4", packed=packed, fused=fused)
                    row["gemms"][name + ("_packed" if packed else "")] = dict(
                        us_median=times, best=best, library=lib, library_over_best=times[lib] / times[best])
                    log("bm sweep %s %s %d routes%s: %s" % (fmt, name, R, " packed" if packed else "",
                                                            " ".join("%d:%.1f" % kv for kv in times.items())))
            res.append(row)
        del w13, w2, p13, p2
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=320,
                    help="decode steps to time: max(5, ceil(steps/16)) replays of the 16-layer graph (at least "
                         "4 per window) in five windows")
    ap.add_argument("--warmup", type=int, default=3, help="untimed graph replays")
    ap.add_argument("--skip-prefill", action="store_true")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--only-headline", action="store_true",
                    help="the headline decode configuration only, without the 100 ms windows (for counter passes)")
    ap.add_argument("--active", type=int, default=8, help="active routes of the --only-headline decode (0..8)")
    ap.add_argument("--only-prefill", action="store_true", help="copy calibration and the prefill GEMMs only")
    ap.add_argument("--only-gather", action="store_true", help="copy calibration and the gather configurations only")
    ap.add_argument("--only-stream", action="store_true", help="copy calibration, input quant, requant and reduce only")
    ap.add_argument("--sweep-bm", action="store_true",
                    help="every M tile at the three prefill densities, each checked before it is timed")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only; --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import moe_routed_expert_amd as m
    import workloads as wl
    m.lib()
    torch.cuda.init()
    reps = max(5, -(-args.steps // LAYERS))
    calib = copy_calibration(torch, m)
    if args.sweep_bm:
        print(json.dumps({"metric": "prefill grouped GEMM us per M tile (checked)", "copy_calibration": calib,
                          "bm_sweep": bm_sweep(torch, m, wl)}))
        return
    if args.only_prefill:
        print(json.dumps({"metric": "prefill fp8 TFLOP/s (grouped GEMMs only)", "copy_calibration": calib,
                          "prefill_densities": prefill_all(torch, m, wl)}))
        return
    if args.only_stream:
        print(json.dumps({"metric": "bandwidth-bound steps at prefill sizes", "copy_calibration": calib,
                          "stream_ops": stream_ops_bench(torch, m, wl)}))
        return
    if args.only_gather:
        print(json.dumps({"metric": "gather us/call (gather only)", "copy_calibration": calib,
                          "gather": gather_all(torch, m, wl)}))
        return

    log("decode H=2048 I=768: building %d layer pools" % LAYERS)
    pools = decode_pools(torch, wl, 2048, 768, 64, seed=1)
    head_active = args.active if args.only_headline else 8
    log("decode H=2048 I=768 %d/8 (headline)" % head_active)
    head = decode_bench(torch, m, wl, pools, 2048, 768, 64, 8, head_active, reps, args.warmup,
                        pages_windows=not args.only_headline)
    extra = {"decode": [head]}
    if args.only_headline:
        print(json.dumps({"metric": "decode us/step (headline configuration only)", "copy_calibration": calib,
                          "decode": head}))
        return
    for active in (4, 2, 0):
        log("decode H=2048 I=768 %d/8" % active)
        extra["decode"].append(decode_bench(torch, m, wl, pools, 2048, 768, 64, 8, active, reps, args.warmup))
    del pools
    torch.cuda.empty_cache()
    log("decode H=4096 I=1024: building %d layer pools" % LAYERS)
    pools = decode_pools(torch, wl, 4096, 1024, 64, seed=2)
    for active in (8, 4, 2, 0):
        log("decode H=4096 I=1024 %d/8" % active)
        extra["decode"].append(decode_bench(torch, m, wl, pools, 4096, 1024, 64, 8, active, reps, args.warmup))
    del pools
    torch.cuda.empty_cache()
    extra["decode_fit"] = [active_fit([r for r in extra["decode"] if r["H"] == h]) for h in (2048, 4096)]
    log("gather")
    extra["gather"] = gather_all(torch, m, wl)
    extra["launch_floor"] = launch_floor(torch)
    log("input quant, requant and reduce at prefill sizes")
    extra["stream_ops"] = stream_ops_bench(torch, m, wl)
    log("route prep")
    extra["route_prep"] = [route_prep_bench(torch, m, wl, T, 256, 6, 20) for T in (256, 4096)]
    if not args.skip_prefill:
        extra["prefill_densities"] = prefill_all(torch, m, wl)
        extra["prefill"] = extra["prefill_densities"][-1]
    tr = measured_traffic()
    roof = dict(bound="hbm",
                kernel="moe_fused_decode step = one decode_step_kernel launch (gate/up and down tiles in one "
                       "grid; H=2048, I=768, 8/8 active)",
                bytes_per_launch=head["bytes_streamed"], us_per_launch=head["us_per_step_median"],
                achieved=head["hbm_gbs"], peak=HBM_PEAK_GBS, unit="GB/s", frac=head["hbm_frac"],
                traffic=tr["traffic_bytes_per_step"] if tr else None)
    extra["copy_calibration"] = calib
    cpu = None
    if not args.skip_cpu:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(wl)
    line = {
        "metric": "bs1 decode us/step & HBM GB/s (top-k 8); prefill fp8 TFLOP/s vs peak",
        "value": round(head["us_per_step_median"], 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": head["steps_timed"],
        "steps_requested": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["us_per_step_median"] / 1000.0,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic (seeded N(0,0.02) block-FP8 expert banks, N(0,1) bf16 activations)",
        "config": {"workload": "decode bs=1, H=2048, I=768, 64-slot pool per layer, top-k 8, 8/8 active; "
                               "16 chained layers per graph, weights from HBM; value = median of 5 windows of %d replays"
                               % head["replays_per_window"],
                   "hbm_gbs": round(head["hbm_gbs"], 1), "hbm_frac": round(head["hbm_frac"], 4),
                   "t0_us": round(extra["decode_fit"][0]["t0_us"], 3),
                   "tau_us_per_route": round(extra["decode_fit"][0]["tau_us_per_route"], 3)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    try:
        main()
    except RuntimeError as e:          # a failed output check or a set error word: no valid line
        print("bench.py: %s" % e, file=sys.stderr)
        sys.exit(3)
