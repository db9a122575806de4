"""GPU parity of the grouped GEMMs at the largest K the ABI accepts and at the full prefill sizes.

* K = 8192 (64 K blocks, the most a tile keeps scales for) at every M tile, fp8 and MXFP4; MXFP4 also at
  K = 4096, where a BM = 64 tile (3-step weight ring, so a 30-step scale chunk) reloads its E8M0 chunk.
* The prefill workload (E = 256, top-6, H = 4096, I = 1024) at 1536, 6144 and 24576 routes in the launch
  the picker chooses ("perf(dsfp4): pick the grouped-prefill tile from route density on sm_89",
  Measurements): the gate/up GEMM (bf16 out), the fused gate/up + SiLU requant and the down GEMM (bf16 out),
  block-FP8, and MXFP4 at 6144 and 24576 routes.  Every column of the rows of four experts is compared with the
  oracle: expert 0, expert E-1, and the experts whose rows start the third and the sixth of the eight
  per-XCD ranges of the persistent tile walk.
* At 24576 routes, the BM = 128 launch (a workgroup's tiles as one pipeline) against the BM = 64 launch
  (tiles one at a time), bit for bit, block-FP8 and MXFP4.
"""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

import moe_routed_expert_amd as m
import oracle
import workloads as wl
from gpu_util import (assert_bf16_within_bound, assert_close, assert_within_bound, check_codes_and_scales, dev,
                      gemm_abs_bound, host_out, mxfp4_abs_bound, silu_h_bound, to_dev, u16)

pytestmark = pytest.mark.gpu

XCDS = 8


def offsets_of(counts):
    offs = np.zeros(len(counts) + 1, np.int32)
    offs[1:] = np.cumsum(counts)
    return offs


# ------------------------------------------------------------- K = 8192 ---

@pytest.mark.parametrize("bm", [16, 32, 64, 128])
def test_fp8_grouped_gemm_k8192(orc, bm):
    """K = 8192 with full-range activation codes (|value| up to 448): f32 output within the per-block
    bound at every element, bf16 output within the pages' tolerance."""
    E, N, K = 3, 256, 8192
    counts = [5, 131, 40]               # ragged tails; 131 rows span two 128-row tiles
    print("fp8 grouped gemm K=8192 BM=%d" % bm, flush=True)
    w_q, w_s = wl.block_fp8_weights(E, N, K, seed=800 + bm)
    offs = offsets_of(counts)
    R = int(offs[-1])
    a_q, a_s = wl.fp8_rows(R, K, seed=801 + bm, full_range=True)
    a_q, a_s, w_q, w_s = a_q.numpy(), a_s.numpy(), w_q.numpy(), w_s.numpy()
    ref = orc.block_gemm(a_q, a_s, w_q, w_s, mode=orc.MODE_GROUPED, expert_offsets=offs, out_dtype=np.float32)
    d = dev()
    out = torch.full((R, N), float("nan"), dtype=torch.float32, device=d)
    outb = torch.full((R, N), float("nan"), dtype=torch.bfloat16, device=d)
    args = (to_dev(a_q), to_dev(a_s), to_dev(w_q), to_dev(w_s))
    m.bf8_grouped_gemm(*args, out, mode=m.MOE_MODE_GROUPED, expert_offsets=to_dev(offs), block_m=bm)
    m.bf8_grouped_gemm(*args, outb, mode=m.MOE_MODE_GROUPED, expert_offsets=to_dev(offs), block_m=bm)
    torch.cuda.synchronize()
    experts = np.repeat(np.arange(E), counts)
    bound = gemm_abs_bound(a_q, a_s, w_q, w_s, experts, np.arange(R))
    assert_within_bound(host_out(out), ref, bound, what="K=8192 f32")
    assert_bf16_within_bound(u16(outb), ref, bound, what="K=8192 bf16")
    assert_close(host_out(outb), ref.astype(np.float64), what="K=8192 bf16")


def test_fp8_grouped_gemm_k8192_integer_case_bit_exact(orc):
    """Codes of -4..4 with power-of-two scales at K = 8192: the exact result (float64, which holds every
    partial sum here) is checked to be what the oracle returns, then the device must return the same bits
    at every M tile."""
    E, N, K = 2, 256, 8192
    counts = [70, 9]
    a_q, a_s, w_q, w_s = wl.powers_of_two_case(E, N, K, sum(counts), seed=12)
    offs = offsets_of(counts)
    ref = orc.block_gemm(a_q, a_s, w_q, w_s, mode=orc.MODE_GROUPED, expert_offsets=offs)
    dec = lambda c: orc.e4m3_decode(c).astype(np.float64)
    exact = np.zeros_like(ref, dtype=np.float64)
    for e in range(E):
        r0, r1 = offs[e], offs[e + 1]
        A = dec(a_q[r0:r1]) * np.repeat(a_s[r0:r1], 128, axis=1)
        W = dec(w_q[e]) * np.repeat(np.repeat(w_s[e], 128, axis=0), 128, axis=1)
        exact[r0:r1] = A @ W.T
    assert np.array_equal(ref.astype(np.float64), exact), "the case is not exact in fp32"
    for bm in (16, 32, 64, 128):
        out = torch.empty((offs[-1], N), dtype=torch.float32, device=dev())
        m.bf8_grouped_gemm(to_dev(a_q), to_dev(a_s), to_dev(w_q), to_dev(w_s), out, mode=m.MOE_MODE_GROUPED,
                           expert_offsets=to_dev(offs), block_m=bm)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32)), bm


@pytest.mark.parametrize("K", [4096, 8192])
@pytest.mark.parametrize("bm", [16, 32, 64, 128])
def test_mxfp4_grouped_gemm_long_k(orc, K, bm):
    """MXFP4 at K = 4096 and 8192, where every tile reloads its E8M0 scale chunk (a chunk covers 30 K steps
    at BM = 64 and 32 otherwise): plain f32 output within the bound, the fused gate/up requant within the
    derived bound and equal to the device's unfused pair, and the exact case bit for bit."""
    E, I = 3, 128
    N = 2 * I
    counts = [5, 131, 40]
    print("mxfp4 long K=%d BM=%d" % (K, bm), flush=True)
    w4, w4_s = wl.mxfp4_weights(E, N, K, seed=900 + K + bm)
    w4, w4_s = w4.numpy(), w4_s.numpy()
    offs = offsets_of(counts)
    R = int(offs[-1])
    a_q, a_s = wl.fp8_rows(R, K, seed=901 + K + bm, full_range=True)
    a_q, a_s = a_q.numpy(), a_s.numpy()
    c1 = orc.mxfp4_gemm(a_q, a_s, w4, w4_s, mode=orc.MODE_GROUPED, expert_offsets=offs, out_dtype=np.float32)
    d = dev()
    aq, as_, wd, wsd, od = to_dev(a_q), to_dev(a_s), to_dev(w4), to_dev(w4_s), to_dev(offs)
    out = torch.full((R, N), float("nan"), dtype=torch.float32, device=d)
    m.mxfp4_grouped_gemm(aq, as_, wd, wsd, od, out, block_m=bm)
    q = torch.full((R, I), 0xAB, dtype=torch.uint8, device=d)
    s = torch.full((R, I // 128), float("nan"), dtype=torch.float32, device=d)
    m.mxfp4_grouped_gemm_act_quant(aq, as_, wd, wsd, od, q, s, block_m=bm)
    q2 = torch.empty_like(q)
    s2 = torch.empty_like(s)
    m.act_quant(out, q2, s2, act=m.MOE_ACT_SILU_MUL)
    torch.cuda.synchronize()
    experts = np.repeat(np.arange(E), counts)
    bound = mxfp4_abs_bound(a_q, a_s, w4, w4_s, experts, np.arange(R))
    assert_within_bound(host_out(out), c1, bound, what="mxfp4 K=%d f32" % K)
    assert torch.equal(q, q2) and torch.equal(s.view(torch.int32), s2.view(torch.int32)), "fused != unfused"
    ref_q, ref_s = orc.silu_mul_quant(c1)
    check_codes_and_scales(orc, q.cpu().numpy(), s.cpu().numpy(), ref_q, ref_s, silu_h_bound(c1, bound, I))
    # the exact case: nibble order, K order and scale-to-block pairing across the reloads
    a_q, a_s, w4, w4_s = wl.mxfp4_exact_case(E, N, K, R, seed=902 + K + bm)
    ref = orc.mxfp4_gemm(a_q, a_s, w4, w4_s, mode=orc.MODE_GROUPED, expert_offsets=offs)
    out = torch.empty((R, N), dtype=torch.float32, device=d)
    m.mxfp4_grouped_gemm(to_dev(a_q), to_dev(a_s), to_dev(w4), to_dev(w4_s), od, out, block_m=bm)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------ full prefill sizes ---

E_FULL, TOPK, H, I = 256, 6, 4096, 1024


def xcd_range_experts(offs, bm, n_tiles_n, ranges=(2, 5)):
    """Experts owning the first tile of the given per-XCD ranges of the persistent tile walk: the live tiles
    (expert M tiles x N tiles, expert-major) are cut into 8 equal contiguous ranges."""
    rows = np.diff(offs)
    tiles = (rows + bm - 1) // bm
    cum = np.concatenate([[0], np.cumsum(tiles)])
    live = int(cum[-1]) * n_tiles_n
    out = []
    for x in ranges:
        m_tile = (live * x // XCDS) // n_tiles_n
        out.append(int(np.searchsorted(cum, m_tile, side="right") - 1))
    return out


def sampled_experts(offs, bm, n_tiles_n):
    ex = [0, E_FULL - 1] + xcd_range_experts(offs, bm, n_tiles_n)
    ex = [e for e in dict.fromkeys(ex) if offs[e + 1] > offs[e]]
    assert len(ex) >= 3
    return ex


def expert_slice(t, e):
    return t[e:e + 1].cpu().numpy()


def oracle_rows(fn, jobs):
    """Per-expert oracle calls on the host's cores (the C oracle releases the GIL)."""
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        return list(ex.map(lambda a: fn(*a), jobs))


@pytest.mark.parametrize("T", [256, 1024, 4096])
def test_prefill_full_size_fp8_vs_oracle(orc, T):
    R = T * TOPK
    # the tiles the launches take (block_m = 0): gate/up and the fused form at K = H, down at K = I
    bms = {"gate/up": m.grouped_block_m(R, E_FULL, H), "fused": m.grouped_block_m(R, E_FULL, H, fused=True),
           "down": m.grouped_block_m(R, E_FULL, I)}
    print("prefill fp8 full size: %d routes, BM %s" % (R, bms), flush=True)
    d = dev()
    w13_q, w13_s = wl.block_fp8_weights(E_FULL, 2 * I, H, 21, device=d, chunk_experts=32)
    w2_q, w2_s = wl.block_fp8_weights(E_FULL, H, I, 22, device=d, chunk_experts=32)
    rt = wl.prefill_routes(T, E_FULL, TOPK, seed=9)
    offs = rt.expert_offsets
    od = to_dev(offs)
    a1_q, a1_s = wl.fp8_rows(R, H, seed=23, device=d, full_range=True)
    a2_q, a2_s = wl.fp8_rows(R, I, seed=24, device=d, full_range=True)
    c1 = torch.full((R, 2 * I), float("nan"), dtype=torch.bfloat16, device=d)
    aq = torch.full((R, I), 0xAB, dtype=torch.uint8, device=d)
    as_ = torch.full((R, I // 128), float("nan"), dtype=torch.float32, device=d)
    c2 = torch.full((R, H), float("nan"), dtype=torch.bfloat16, device=d)
    m.bf8_grouped_gemm(a1_q, a1_s, w13_q, w13_s, c1, mode=m.MOE_MODE_GROUPED, expert_offsets=od)
    m.bf8_grouped_gemm_act_quant(a1_q, a1_s, w13_q, w13_s, od, aq, as_)
    m.bf8_grouped_gemm(a2_q, a2_s, w2_q, w2_s, c2, mode=m.MOE_MODE_GROUPED, expert_offsets=od)
    torch.cuda.synchronize()
    for name, n_tiles_n in (("gate/up", 2 * I // 256), ("fused", I // 128), ("down", H // 256)):
        experts = sampled_experts(offs, bms[name], n_tiles_n)
        print("  %s: experts %s" % (name, experts), flush=True)
        jobs = []
        for e in experts:
            r0, r1 = int(offs[e]), int(offs[e + 1])
            one = np.array([0, r1 - r0], np.int32)
            if name == "down":
                jobs.append((a2_q[r0:r1].cpu().numpy(), a2_s[r0:r1].cpu().numpy(), expert_slice(w2_q, e),
                             expert_slice(w2_s, e), one))
            else:
                jobs.append((a1_q[r0:r1].cpu().numpy(), a1_s[r0:r1].cpu().numpy(), expert_slice(w13_q, e),
                             expert_slice(w13_s, e), one))
        refs = oracle_rows(lambda a, s_, w, ws, o: orc.block_gemm(a, s_, w, ws, mode=orc.MODE_GROUPED,
                                                                   expert_offsets=o, out_dtype=np.float32), jobs)
        for e, job, ref in zip(experts, jobs, refs):
            r0, r1 = int(offs[e]), int(offs[e + 1])
            bound = gemm_abs_bound(job[0], job[1], job[2], job[3], np.zeros(r1 - r0, np.int64), np.arange(r1 - r0))
            what = "%d routes %s expert %d" % (R, name, e)
            if name == "fused":
                ref_q, ref_s = orc.silu_mul_quant(ref)
                check_codes_and_scales(orc, aq[r0:r1].cpu().numpy(), as_[r0:r1].cpu().numpy(), ref_q, ref_s,
                                       silu_h_bound(ref, bound, I))
            else:
                got = u16(c2[r0:r1] if name == "down" else c1[r0:r1])
                assert_bf16_within_bound(got, ref, bound, what=what)
                assert_close(host_out(c2[r0:r1] if name == "down" else c1[r0:r1]),
                             oracle.bf16_decode(orc.bf16_encode(ref)).astype(np.float64), what=what)
    # rows past the last expert stay untouched; every routed row was written
    assert not torch.isnan(c1.float()).any() and not torch.isnan(c2.float()).any()
    assert not torch.isnan(as_).any()


@pytest.mark.parametrize("T", [1024, 4096])
def test_prefill_full_size_mxfp4_vs_oracle(orc, T):
    R = T * TOPK
    bms = {"gate/up": m.grouped_block_m(R, E_FULL, H, mxfp4=True),
           "fused": m.grouped_block_m(R, E_FULL, H, mxfp4=True, fused=True),
           "down": m.grouped_block_m(R, E_FULL, I, mxfp4=True)}
    print("prefill mxfp4 full size: %d routes, BM %s" % (R, bms), flush=True)
    d = dev()
    w13, w13_s = wl.mxfp4_weights(E_FULL, 2 * I, H, seed=31, device=d)
    w2, w2_s = wl.mxfp4_weights(E_FULL, H, I, seed=32, device=d)
    rt = wl.prefill_routes(T, E_FULL, TOPK, seed=9)
    offs = rt.expert_offsets
    od = to_dev(offs)
    a1_q, a1_s = wl.fp8_rows(R, H, seed=33, device=d, full_range=True)
    a2_q, a2_s = wl.fp8_rows(R, I, seed=34, device=d, full_range=True)
    c1 = torch.full((R, 2 * I), float("nan"), dtype=torch.bfloat16, device=d)
    aq = torch.full((R, I), 0xAB, dtype=torch.uint8, device=d)
    as_ = torch.full((R, I // 128), float("nan"), dtype=torch.float32, device=d)
    c2 = torch.full((R, H), float("nan"), dtype=torch.bfloat16, device=d)
    m.mxfp4_grouped_gemm(a1_q, a1_s, w13, w13_s, od, c1)
    m.mxfp4_grouped_gemm_act_quant(a1_q, a1_s, w13, w13_s, od, aq, as_)
    m.mxfp4_grouped_gemm(a2_q, a2_s, w2, w2_s, od, c2)
    torch.cuda.synchronize()
    for name, n_tiles_n in (("gate/up", 2 * I // 256), ("fused", I // 128), ("down", H // 256)):
        experts = sampled_experts(offs, bms[name], n_tiles_n)
        print("  %s: experts %s" % (name, experts), flush=True)
        jobs = []
        for e in experts:
            r0, r1 = int(offs[e]), int(offs[e + 1])
            one = np.array([0, r1 - r0], np.int32)
            if name == "down":
                jobs.append((a2_q[r0:r1].cpu().numpy(), a2_s[r0:r1].cpu().numpy(), expert_slice(w2, e),
                             expert_slice(w2_s, e), one))
            else:
                jobs.append((a1_q[r0:r1].cpu().numpy(), a1_s[r0:r1].cpu().numpy(), expert_slice(w13, e),
                             expert_slice(w13_s, e), one))
        refs = oracle_rows(lambda a, s_, w, ws, o: orc.mxfp4_gemm(a, s_, w, ws, mode=orc.MODE_GROUPED,
                                                                   expert_offsets=o, out_dtype=np.float32), jobs)
        for e, job, ref in zip(experts, jobs, refs):
            r0, r1 = int(offs[e]), int(offs[e + 1])
            bound = mxfp4_abs_bound(job[0], job[1], job[2], job[3], np.zeros(r1 - r0, np.int64), np.arange(r1 - r0))
            what = "mxfp4 %d routes %s expert %d" % (R, name, e)
            if name == "fused":
                ref_q, ref_s = orc.silu_mul_quant(ref)
                check_codes_and_scales(orc, aq[r0:r1].cpu().numpy(), as_[r0:r1].cpu().numpy(), ref_q, ref_s,
                                       silu_h_bound(ref, bound, I))
            else:
                got = u16(c2[r0:r1] if name == "down" else c1[r0:r1])
                assert_bf16_within_bound(got, ref, bound, what=what)
    assert not torch.isnan(c1.float()).any() and not torch.isnan(c2.float()).any()
    assert not torch.isnan(as_).any()


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_block_m_128_tile_walk_equals_single_tiles(fmt):
    """At 24576 routes each BM = 128 workgroup runs many tiles back to back as one K-step pipeline (the next
    tile's first steps and scales in flight during a tile's last steps and epilogue; with MXFP4 weights
    only for the down GEMM, whose tiles have 8 K steps).  Each output element takes the same K order at
    every tile size, so the gate/up GEMM (f32 out), its fused SiLU requant and the down GEMM (bf16 out)
    must equal the BM = 64 launch, whose tiles run one at a time, bit for bit."""
    T = 4096
    R = T * TOPK
    assert m.pick_block_m(R, E_FULL) == 128
    print("BM=128 walk vs BM=64 tiles, %s, %d routes" % (fmt, R), flush=True)
    d = dev()
    if fmt == "fp8":
        w13, w13_s = wl.block_fp8_weights(E_FULL, 2 * I, H, 41, device=d, chunk_experts=32)
        w2, w2_s = wl.block_fp8_weights(E_FULL, H, I, 42, device=d, chunk_experts=32)
        gemm = lambda a, s_, w, ws, od, out, bm: m.bf8_grouped_gemm(a, s_, w, ws, out, mode=m.MOE_MODE_GROUPED,
                                                                     expert_offsets=od, block_m=bm)
        fused = lambda a, s_, w, ws, od, q, s, bm: m.bf8_grouped_gemm_act_quant(a, s_, w, ws, od, q, s, block_m=bm)
    else:
        w13, w13_s = wl.mxfp4_weights(E_FULL, 2 * I, H, seed=43, device=d)
        w2, w2_s = wl.mxfp4_weights(E_FULL, H, I, seed=44, device=d)
        gemm = lambda a, s_, w, ws, od, out, bm: m.mxfp4_grouped_gemm(a, s_, w, ws, od, out, block_m=bm)
        fused = lambda a, s_, w, ws, od, q, s, bm: m.mxfp4_grouped_gemm_act_quant(a, s_, w, ws, od, q, s,
                                                                                  block_m=bm)
    rt = wl.prefill_routes(T, E_FULL, TOPK, seed=45)
    od = to_dev(rt.expert_offsets)
    a1_q, a1_s = wl.fp8_rows(R, H, seed=46, device=d, full_range=True)
    a2_q, a2_s = wl.fp8_rows(R, I, seed=47, device=d, full_range=True)
    res = {}
    for bm in (128, 64):
        c1 = torch.full((R, 2 * I), float("nan"), dtype=torch.float32, device=d)
        q = torch.full((R, I), 0xAB, dtype=torch.uint8, device=d)
        s = torch.full((R, I // 128), float("nan"), dtype=torch.float32, device=d)
        c2 = torch.full((R, H), float("nan"), dtype=torch.bfloat16, device=d)
        gemm(a1_q, a1_s, w13, w13_s, od, c1, bm)
        fused(a1_q, a1_s, w13, w13_s, od, q, s, bm)
        gemm(a2_q, a2_s, w2, w2_s, od, c2, bm)
        res[bm] = (c1.view(torch.int32), q, s.view(torch.int32), c2.view(torch.int16))
    torch.cuda.synchronize()
    assert not torch.isnan(res[128][0].view(torch.float32)).any()
    for name, x, y in zip(("gate/up", "codes", "scales", "down"), res[128], res[64]):
        bad = (x != y).nonzero()
        assert bad.numel() == 0, "%s %s: %d elements differ, first at %s" % (fmt, name, bad.shape[0],
                                                                              bad[0].tolist())
