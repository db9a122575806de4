"""GPU tests of packed expert banks (moe_pack_weights) and of the grouped GEMMs reading them.

The packed order is this library's own layout, not a step of the pages' method: the pack must give the bytes
the header's formula names, and every grouped GEMM must return, from a packed bank, the bits it returns from
the row-major bank (which the other GEMM tests compare with the oracle).  One small case is also compared
with the oracle directly.
"""
import numpy as np
import pytest
import torch

import moe_routed_expert_amd as m
import workloads as wl
from gpu_util import assert_within_bound, dev, gemm_abs_bound, host_out, to_dev

pytestmark = pytest.mark.gpu


def packed_order(w: np.ndarray, step: int) -> np.ndarray:
    """The packed bank of w [E, N, RB] as moe_routed.h states it: per expert, per 16-row group g and K step
    s, a block of `step` 16-byte pieces; piece p is row 16g + p%16, bytes s*step + 64*(p/64) +
    16*((p%64)/16) .. +15."""
    E, N, RB = w.shape
    ns = RB // step
    r = np.arange(N * RB // 16)
    blk, p = r // step, r % step
    g, s = blk // ns, blk % ns
    row = 16 * g + (p % 16)
    col = s * step + 64 * (p // 64) + 16 * ((p % 64) // 16)
    idx = col[:, None] + np.arange(16)[None, :]
    out = np.empty((E, N * RB // 16, 16), np.uint8)
    for e in range(E):
        out[e] = w[e][row[:, None], idx]
    return out.reshape(E, N, RB)


@pytest.mark.parametrize("step", [128, 64])
def test_pack_matches_the_stated_order(step):
    """Strided source (padded rows and experts), several experts and groups."""
    E, N, RB = 3, 48, 4 * step
    rng = np.random.default_rng(5 + step)
    src = rng.integers(0, 256, size=(E, N + 5, RB + 32), dtype=np.uint8)
    d = dev()
    big = to_dev(src)
    w = big[:, :N, :RB]
    out = m.pack_weights(w, step)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), packed_order(src[:, :N, :RB], step))


def offsets_of(counts):
    offs = np.zeros(len(counts) + 1, np.int32)
    offs[1:] = np.cumsum(counts)
    return offs


@pytest.mark.parametrize("bm", [16, 32, 64, 128])
def test_bf8_packed_equals_row_major(orc, bm):
    """Plain GEMM (f32 and bf16 out) and the fused gate/up requant: packed bank == row-major bank, bit for bit;
    the f32 output also against the oracle within the per-block bound."""
    E, I, K = 5, 256, 640
    N = 2 * I
    counts = [3, 0, 40, 129, 17]
    print("packed bf8 BM=%d" % bm, flush=True)
    w_q, w_s = wl.block_fp8_weights(E, N, K, seed=60 + bm)
    offs = offsets_of(counts)
    R = int(offs[-1])
    a_q, a_s = wl.fp8_rows(R, K, seed=61 + bm, full_range=True)
    d = dev()
    aq, as_, wq, ws, od = to_dev(a_q), to_dev(a_s), to_dev(w_q), to_dev(w_s), to_dev(offs)
    wp = m.pack_weights(wq, 128)
    res = {}
    for packed, w in ((False, wq), (True, wp)):
        f = torch.empty((R, N), dtype=torch.float32, device=d)
        b = torch.empty((R, N), dtype=torch.bfloat16, device=d)
        q = torch.empty((R, I), dtype=torch.uint8, device=d)
        s = torch.empty((R, I // 128), dtype=torch.float32, device=d)
        m.bf8_grouped_gemm(aq, as_, w, ws, f, mode=m.MOE_MODE_GROUPED, expert_offsets=od, block_m=bm, w_packed=packed)
        m.bf8_grouped_gemm(aq, as_, w, ws, b, mode=m.MOE_MODE_GROUPED, expert_offsets=od, block_m=bm, w_packed=packed)
        m.bf8_grouped_gemm_act_quant(aq, as_, w, ws, od, q, s, block_m=bm, w_packed=packed)
        res[packed] = (f.view(torch.int32), b.view(torch.int16), q, s.view(torch.int32))
    torch.cuda.synchronize()
    for name, x, y in zip(("f32", "bf16", "codes", "scales"), res[True], res[False]):
        assert torch.equal(x, y), "packed != row-major: " + name
    ref = orc.block_gemm(a_q.numpy(), a_s.numpy(), w_q.numpy(), w_s.numpy(), mode=orc.MODE_GROUPED,
                         expert_offsets=offs, out_dtype=np.float32)
    experts = np.repeat(np.arange(E), counts)
    bound = gemm_abs_bound(a_q.numpy(), a_s.numpy(), w_q.numpy(), w_s.numpy(), experts, np.arange(R))
    assert_within_bound(host_out(res[True][0].view(torch.float32)), ref, bound, what="packed f32")


@pytest.mark.parametrize("bm,K", [(16, 640), (64, 640), (128, 640), (64, 4096), (128, 4096)])
def test_mxfp4_packed_equals_row_major(bm, K):
    """MXFP4 plain and fused, short K (BM = 128 runs its tiles as one pipeline) and K = 4096 (tiles one at a
    time; BM = 64 reloads its E8M0 chunk): packed == row-major, bit for bit."""
    E, I = 4, 128
    N = 2 * I
    counts = [5, 131, 0, 40]
    print("packed mxfp4 BM=%d K=%d" % (bm, K), flush=True)
    w4, w4_s = wl.mxfp4_weights(E, N, K, seed=70 + bm + K)
    offs = offsets_of(counts)
    R = int(offs[-1])
    a_q, a_s = wl.fp8_rows(R, K, seed=71 + bm + K, full_range=True)
    d = dev()
    aq, as_, w, ws, od = to_dev(a_q), to_dev(a_s), to_dev(w4), to_dev(w4_s), to_dev(offs)
    wp = m.pack_weights(w, 64)
    res = {}
    for packed, wt in ((False, w), (True, wp)):
        f = torch.empty((R, N), dtype=torch.float32, device=d)
        q = torch.empty((R, I), dtype=torch.uint8, device=d)
        s = torch.empty((R, I // 128), dtype=torch.float32, device=d)
        m.mxfp4_grouped_gemm(aq, as_, wt, ws, od, f, block_m=bm, w_packed=packed)
        m.mxfp4_grouped_gemm_act_quant(aq, as_, wt, ws, od, q, s, block_m=bm, w_packed=packed)
        res[packed] = (f.view(torch.int32), q, s.view(torch.int32))
    torch.cuda.synchronize()
    for name, x, y in zip(("f32", "codes", "scales"), res[True], res[False]):
        assert torch.equal(x, y), "packed != row-major: " + name


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_packed_prefill_full_size(fmt):
    """The 24576-route prefill (E = 256, top-6, H = 4096, I = 1024) in the picker's launch: gate/up (bf16),
    the fused requant and down (bf16) from packed banks equal the row-major ones bit for bit."""
    E, topk, H, I, T = 256, 6, 4096, 1024, 4096
    R = T * topk
    print("packed %s prefill, %d routes" % (fmt, R), flush=True)
    d = dev()
    if fmt == "fp8":
        w13, w13_s = wl.block_fp8_weights(E, 2 * I, H, 81, device=d, chunk_experts=32)
        w2, w2_s = wl.block_fp8_weights(E, H, I, 82, device=d, chunk_experts=32)
        step = 128

        def run(a, s_, w, ws, od, out, packed):
            m.bf8_grouped_gemm(a, s_, w, ws, out, mode=m.MOE_MODE_GROUPED, expert_offsets=od, w_packed=packed)

        def fused(a, s_, w, ws, od, q, s, packed):
            m.bf8_grouped_gemm_act_quant(a, s_, w, ws, od, q, s, w_packed=packed)
    else:
        w13, w13_s = wl.mxfp4_weights(E, 2 * I, H, seed=83, device=d)
        w2, w2_s = wl.mxfp4_weights(E, H, I, seed=84, device=d)
        step = 64

        def run(a, s_, w, ws, od, out, packed):
            m.mxfp4_grouped_gemm(a, s_, w, ws, od, out, w_packed=packed)

        def fused(a, s_, w, ws, od, q, s, packed):
            m.mxfp4_grouped_gemm_act_quant(a, s_, w, ws, od, q, s, w_packed=packed)
    p13, p2 = m.pack_weights(w13, step), m.pack_weights(w2, step)
    rt = wl.prefill_routes(T, E, topk, seed=85)
    od = to_dev(rt.expert_offsets)
    a1_q, a1_s = wl.fp8_rows(R, H, seed=86, device=d, full_range=True)
    a2_q, a2_s = wl.fp8_rows(R, I, seed=87, device=d, full_range=True)
    res = {}
    for packed, (wa, wb) in ((False, (w13, w2)), (True, (p13, p2))):
        c1 = torch.empty((R, 2 * I), dtype=torch.bfloat16, device=d)
        q = torch.empty((R, I), dtype=torch.uint8, device=d)
        s = torch.empty((R, I // 128), dtype=torch.float32, device=d)
        c2 = torch.empty((R, H), dtype=torch.bfloat16, device=d)
        run(a1_q, a1_s, wa, w13_s, od, c1, packed)
        fused(a1_q, a1_s, wa, w13_s, od, q, s, packed)
        run(a2_q, a2_s, wb, w2_s, od, c2, packed)
        res[packed] = (c1.view(torch.int16), q, s.view(torch.int32), c2.view(torch.int16))
    torch.cuda.synchronize()
    for name, x, y in zip(("gate/up", "codes", "scales", "down"), res[True], res[False]):
        bad = (x != y).nonzero()
        assert bad.numel() == 0, "%s %s: %d elements differ, first at %s" % (fmt, name, bad.shape[0],
                                                                              bad[0].tolist())
