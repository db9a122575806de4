"""GPU parity of the block-FP8 GEMM (slot mode and grouped mode) against the CPU oracle."""
import numpy as np
import pytest
import torch

import moe_routed_expert_amd as m
import oracle
import workloads as wl
from gpu_util import (NP_OUT, assert_bf16_close, assert_close, assert_within_bound, check_codes_and_scales, dev,
                      gemm_abs_bound, host_out, ref_as_f64, silu_h_bound, to_dev, u16)

pytestmark = pytest.mark.gpu

# --------------------------------------------------------------- slot mode ---

@pytest.mark.parametrize("N,K,rows,topk", [(256, 256, 2, 2), (1536, 2048, 8, 8), (2048, 768, 8, 1),
                                           (2048, 4096, 16, 8), (64, 1024, 5, 1)])
@pytest.mark.parametrize("odt", [torch.float32, torch.bfloat16, torch.float16])
def test_slot_gemm_vs_oracle(orc, N, K, rows, topk, odt):
    print("slot gemm N=%d K=%d rows=%d %s" % (N, K, rows, odt), flush=True)
    E = 6
    w_q, w_s = wl.block_fp8_weights(E, N, K, seed=N + K)
    T = max(1, rows // topk)
    a_q, a_s = wl.fp8_rows(T, K, seed=K)
    rng = np.random.default_rng(N)
    slots = rng.integers(-1, E, size=rows).astype(np.int32)
    slots[0] = 2
    ref = orc.block_gemm(a_q.numpy(), a_s.numpy(), w_q.numpy(), w_s.numpy(), mode=orc.MODE_SLOT,
                         slot_ids=slots, a_row_div=topk, out_dtype=NP_OUT[odt])
    out = torch.full((rows, N), float("nan"), dtype=odt, device=dev())
    m.bf8_grouped_gemm(a_q.to(dev()), a_s.to(dev()), w_q.to(dev()), w_s.to(dev()), out, mode=m.MOE_MODE_SLOT,
                       slot_ids=to_dev(slots), a_row_div=topk)
    torch.cuda.synchronize()
    got = host_out(out)
    inactive = slots < 0
    assert np.all(got[inactive] == 0) and not np.any(np.signbit(got[inactive]))
    if odt == torch.float32:
        bound = gemm_abs_bound(a_q.numpy(), a_s.numpy(), w_q.numpy(), w_s.numpy(), slots, np.arange(rows) // topk)
        assert_within_bound(got, ref, bound, what="slot gemm f32")
    assert_close(got, ref_as_f64(ref, odt), what="slot gemm")


def test_slot_gemm_integer_case_bit_exact(orc):
    E, N, K, rows = 3, 512, 1024, 6
    a_q, a_s, w_q, w_s = wl.powers_of_two_case(E, N, K, rows, seed=9)
    slots = np.array([0, 2, -1, 1, 1, 0], np.int32)
    ref = orc.block_gemm(a_q, a_s, w_q, w_s, mode=orc.MODE_SLOT, slot_ids=slots)
    out = torch.empty((rows, N), dtype=torch.float32, device=dev())
    m.bf8_grouped_gemm(to_dev(a_q), to_dev(a_s), to_dev(w_q), to_dev(w_s), out, mode=m.MOE_MODE_SLOT,
                       slot_ids=to_dev(slots))
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_slot_gemm_empty_bank_all_inactive():
    K, N = 256, 128
    a_q = torch.zeros((1, K), dtype=torch.uint8, device=dev())
    a_s = torch.zeros((1, 2), dtype=torch.float32, device=dev())
    out = torch.full((4, N), float("nan"), dtype=torch.float32, device=dev())
    slots = torch.full((4,), -1, dtype=torch.int32, device=dev())
    st = m.lib().moe_bf8_grouped_gemm(a_q.data_ptr(), K, a_s.data_ptr(), 2, None, 0, K, None, 0, 2, 0, N, K,
                                      m.MOE_MODE_SLOT, None, slots.data_ptr(), 4, 4, 0, out.data_ptr(), m.MOE_F32,
                                      N, m._stream())
    assert st == m.MOE_OK
    torch.cuda.synchronize()
    assert torch.all(out == 0)


# ------------------------------------------------------------ grouped mode ---

def grouped_case(E, N, K, counts, seed):
    w_q, w_s = wl.block_fp8_weights(E, N, K, seed=seed)
    R = int(sum(counts))
    a_q, a_s = wl.fp8_rows(R, K, seed=seed + 1)
    offs = np.zeros(E + 1, np.int32)
    offs[1:] = np.cumsum(counts)
    return w_q, w_s, a_q, a_s, offs


@pytest.mark.parametrize("bm", [16, 32, 64, 128])
@pytest.mark.parametrize("odt", [torch.bfloat16, torch.float32])
def test_grouped_gemm_vs_oracle(orc, bm, odt):
    E, N, K = 5, 256, 512
    counts = [3, 0, 40, 129, 17]        # empty expert, ragged tails, several M tiles
    print("grouped gemm BM=%d %s" % (bm, odt), flush=True)
    w_q, w_s, a_q, a_s, offs = grouped_case(E, N, K, counts, seed=bm)
    ref = orc.block_gemm(a_q.numpy(), a_s.numpy(), w_q.numpy(), w_s.numpy(), mode=orc.MODE_GROUPED,
                         expert_offsets=offs, out_dtype=NP_OUT[odt])
    R = offs[-1]
    out = torch.full((R + 3, N), float("nan"), dtype=odt, device=dev())   # 3 spare rows stay untouched
    m.bf8_grouped_gemm(a_q.to(dev()), a_s.to(dev()), w_q.to(dev()), w_s.to(dev()), out, mode=m.MOE_MODE_GROUPED,
                       expert_offsets=to_dev(offs), m_rows=R + 3, block_m=bm)
    torch.cuda.synchronize()
    got = host_out(out)
    assert np.all(np.isnan(got[R:]))
    if odt == torch.float32:
        experts = np.repeat(np.arange(E), np.diff(offs))
        bound = gemm_abs_bound(a_q.numpy(), a_s.numpy(), w_q.numpy(), w_s.numpy(), experts, np.arange(R))
        assert_within_bound(got[:R], ref, bound, what="grouped gemm f32")
    assert_close(got[:R], ref_as_f64(ref, odt), what="grouped gemm")


@pytest.mark.parametrize("w4", [False, True])
@pytest.mark.parametrize("bm", [16, 32, 64, 128])
def test_grouped_gemm_2byte_outputs_are_the_rounded_f32(bm, w4):
    """bf16 and f16 outputs equal torch's round-to-nearest-even of the same launch's f32 output, bit for bit,
    at an output row stride that takes the 16-byte stores (lane swaps), one that takes 8-byte stores and
    one that takes 2-byte stores; N = 384 leaves the second 256-column tile half empty, and nothing outside
    the output is written."""
    E, N, K = 5, 384, 512
    counts = [3, 0, 40, 129, 17]
    print("2-byte outputs BM=%d %s" % (bm, "mxfp4" if w4 else "bf8"), flush=True)
    offs = np.zeros(E + 1, np.int32)
    offs[1:] = np.cumsum(counts)
    R = int(offs[-1])
    a_q, a_s = wl.fp8_rows(R, K, seed=71 + bm, full_range=True)
    aq, as_, od = a_q.to(dev()), a_s.to(dev()), to_dev(offs)
    if w4:
        w, ws = wl.mxfp4_weights(E, N, K, seed=72 + bm)
        w, ws = w.to(dev()), ws.to(dev())
        run = lambda out: m.mxfp4_grouped_gemm(aq, as_, w, ws, od, out, m_rows=R, block_m=bm)
    else:
        w, ws = wl.block_fp8_weights(E, N, K, seed=72 + bm)
        w, ws = w.to(dev()), ws.to(dev())
        run = lambda out: m.bf8_grouped_gemm(aq, as_, w, ws, out, mode=m.MOE_MODE_GROUPED, expert_offsets=od,
                                             m_rows=R, block_m=bm)
    ref = torch.empty((R, N), dtype=torch.float32, device=dev())
    run(ref)
    for odt in (torch.bfloat16, torch.float16):
        want = ref.to(odt)
        for pad in (0, 4, 1):
            big = torch.full((R + 2, N + pad), float("nan"), dtype=odt, device=dev())
            out = big[:R, :N]
            run(out)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), want.view(torch.int16)), (odt, pad)
            assert torch.all(torch.isnan(big[:, N:])) and torch.all(torch.isnan(big[R:])), (odt, pad)


def test_grouped_gemm_integer_case_bit_exact(orc):
    E, N, K = 4, 384, 640
    counts = [20, 1, 0, 33]
    a_q, a_s, w_q, w_s = wl.powers_of_two_case(E, N, K, sum(counts), seed=10)
    offs = np.zeros(E + 1, np.int32)
    offs[1:] = np.cumsum(counts)
    ref = orc.block_gemm(a_q, a_s, w_q, w_s, mode=orc.MODE_GROUPED, expert_offsets=offs)
    for bm in (16, 32, 64, 128):
        out = torch.empty((offs[-1], N), dtype=torch.float32, device=dev())
        m.bf8_grouped_gemm(to_dev(a_q), to_dev(a_s), to_dev(w_q), to_dev(w_s), out, mode=m.MOE_MODE_GROUPED,
                           expert_offsets=to_dev(offs), block_m=bm)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32)), bm


def test_grouped_prefill_routes_chain(orc):
    """gather -> grouped gate/up (bf16) -> SiLU-mul requant -> grouped down (bf16) -> reduce, small shape."""
    T, E, topk, H, I = 64, 16, 4, 512, 256
    rt = wl.prefill_routes(T, E, topk, seed=3)
    x = wl.bf16_normal((T, H), seed=4)
    w13_q, w13_s = wl.block_fp8_weights(E, 2 * I, H, seed=5)
    w2_q, w2_s = wl.block_fp8_weights(E, H, I, seed=6)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    # oracle chain
    xq, xs = orc.quant_groups(xb)
    gq, gs = orc.gather_rows_scales(xq, xs, rt.dst2src)
    c1 = orc.block_gemm(gq, gs, w13_q.numpy(), w13_s.numpy(), mode=orc.MODE_GROUPED,
                        expert_offsets=rt.expert_offsets, out_dtype=np.uint16)
    aq, as_ = orc.silu_mul_quant(c1)
    c2 = orc.block_gemm(aq, as_, w2_q.numpy(), w2_s.numpy(), mode=orc.MODE_GROUPED,
                        expert_offsets=rt.expert_offsets, out_dtype=np.uint16)
    ref = orc.topk_reduce(c2, rt.expert_ids, rt.weights, route_rows=rt.route_rows)
    # device chain
    R = T * topk
    d = dev()
    xq_d = torch.empty((T, H), dtype=torch.uint8, device=d)
    xs_d = torch.empty((T, H // 128), dtype=torch.float32, device=d)
    m.act_quant(x.to(d), xq_d, xs_d)
    gq_d = torch.empty((R, H), dtype=torch.uint8, device=d)
    gs_d = torch.empty((R, H // 128), dtype=torch.float32, device=d)
    m.gather_rows_scales(xq_d, xs_d, to_dev(rt.dst2src), gq_d, gs_d)
    c1_d = torch.empty((R, 2 * I), dtype=torch.bfloat16, device=d)
    offs = to_dev(rt.expert_offsets)
    m.bf8_grouped_gemm(gq_d, gs_d, w13_q.to(d), w13_s.to(d), c1_d, mode=m.MOE_MODE_GROUPED, expert_offsets=offs)
    aq_d = torch.empty((R, I), dtype=torch.uint8, device=d)
    as_d = torch.empty((R, I // 128), dtype=torch.float32, device=d)
    m.act_quant(c1_d, aq_d, as_d, act=m.MOE_ACT_SILU_MUL)
    c2_d = torch.empty((R, H), dtype=torch.bfloat16, device=d)
    m.bf8_grouped_gemm(aq_d, as_d, w2_q.to(d), w2_s.to(d), c2_d, mode=m.MOE_MODE_GROUPED, expert_offsets=offs)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=d)
    m.topk_reduce(c2_d, to_dev(rt.expert_ids), to_dev(rt.weights), out, route_rows=to_dev(rt.route_rows))
    torch.cuda.synchronize()
    assert np.array_equal(xq_d.cpu().numpy(), xq)
    assert np.array_equal(gq_d.cpu().numpy(), gq)
    assert_bf16_close(u16(c1_d), c1, what="prefill c1")
    assert_bf16_close(u16(out), ref, what="prefill out")


# ------------------------------------------------- fused SiLU-mul requant ---

@pytest.mark.parametrize("bm,act", [(0, 1), (16, 1), (32, 1), (64, 1), (128, 1), (64, 2), (128, 3), (32, 4),
                                    (16, 5)])
def test_grouped_silu_quant_vs_oracle_and_unfused(orc, bm, act):
    """The fused gate/up + gated-activation requant equals the oracle's fp32 GEMM followed by its requant
    (within the derived bound), and the device's own unfused pair (fp32 GEMM, then act_quant) bit for bit;
    every tile size with SwiGLU, and each other activation once."""
    E, I, K = 5, 256, 640
    counts = [3, 0, 40, 129, 17]        # empty expert, ragged tails, several M tiles
    print("fused gate/up act-quant BM=%d act=%d" % (bm, act), flush=True)
    w_q, w_s, a_q, a_s, offs = grouped_case(E, 2 * I, K, counts, seed=100 + bm + act)
    R = int(offs[-1])
    c1 = orc.block_gemm(a_q.numpy(), a_s.numpy(), w_q.numpy(), w_s.numpy(), mode=orc.MODE_GROUPED,
                        expert_offsets=offs, out_dtype=np.float32)
    ref_q, ref_s = orc.gated_act_quant(c1, act)
    d = dev()
    q = torch.full((R + 2, I), 0xAB, dtype=torch.uint8, device=d)          # 2 spare rows stay untouched
    s = torch.full((R + 2, I // 128), float("nan"), dtype=torch.float32, device=d)
    wq, ws, aq, as_, od = w_q.to(d), w_s.to(d), a_q.to(d), a_s.to(d), to_dev(offs)
    m.bf8_grouped_gemm_act_quant(aq, as_, wq, ws, od, q, s, m_rows=R + 2, block_m=bm, act=act)
    # the unfused device pair
    c1_d = torch.empty((R, 2 * I), dtype=torch.float32, device=d)
    m.bf8_grouped_gemm(aq, as_, wq, ws, c1_d, mode=m.MOE_MODE_GROUPED, expert_offsets=od, block_m=bm)
    q2 = torch.empty((R, I), dtype=torch.uint8, device=d)
    s2 = torch.empty((R, I // 128), dtype=torch.float32, device=d)
    m.act_quant(c1_d, q2, s2, act=act)
    torch.cuda.synchronize()
    hq, hs = q.cpu().numpy(), s.cpu().numpy()
    assert np.all(hq[R:] == 0xAB) and np.all(np.isnan(hs[R:]))
    assert np.array_equal(hq[:R], q2.cpu().numpy()) and np.array_equal(hs[:R].view(np.uint32),
                                                                      s2.cpu().numpy().view(np.uint32))
    experts = np.repeat(np.arange(E), np.diff(offs))
    c1_bound = gemm_abs_bound(a_q.numpy(), a_s.numpy(), w_q.numpy(), w_s.numpy(), experts, np.arange(R))
    check_codes_and_scales(orc, hq[:R], hs[:R], ref_q, ref_s, silu_h_bound(c1, c1_bound, I, act))


def test_grouped_silu_quant_zero_rows():
    """Rows whose activation is all zero (an inactive route's tile) give zero codes and +0 scales."""
    E, I, K = 2, 128, 256
    w_q, w_s, a_q, a_s, offs = grouped_case(E, 2 * I, K, [5, 7], seed=9)
    a_q[3] = 0
    a_s[3] = 0
    d = dev()
    q = torch.full((12, I), 0xAB, dtype=torch.uint8, device=d)
    s = torch.full((12, 1), float("nan"), dtype=torch.float32, device=d)
    m.bf8_grouped_gemm_act_quant(a_q.to(d), a_s.to(d), w_q.to(d), w_s.to(d), to_dev(offs), q, s)
    torch.cuda.synchronize()
    assert np.all(q.cpu().numpy()[3] == 0) and s.cpu().numpy()[3, 0] == 0.0 and not np.signbit(s.cpu().numpy()[3, 0])


def test_grouped_silu_quant_full_prefill_size(orc):
    """At the 24576-route prefill size (E=256, top-6, H=4096, I=1024) in the picker's launch: fused equals the
    unfused device pair bit for bit, and one sampled expert's rows match the oracle."""
    E, topk, H, I, T = 256, 6, 4096, 1024, 4096
    print("fused gate/up silu-quant at 24576 routes", flush=True)
    d = dev()
    w_q, w_s = wl.block_fp8_weights(E, 2 * I, H, 21, device=d, chunk_experts=32)
    rt = wl.prefill_routes(T, E, topk, seed=9)
    R = T * topk
    od = to_dev(rt.expert_offsets)
    a_q, a_s = wl.fp8_rows(R, H, seed=23, device=d)
    q = torch.empty((R, I), dtype=torch.uint8, device=d)
    s = torch.empty((R, I // 128), dtype=torch.float32, device=d)
    m.bf8_grouped_gemm_act_quant(a_q, a_s, w_q, w_s, od, q, s)
    c1_d = torch.empty((R, 2 * I), dtype=torch.float32, device=d)
    m.bf8_grouped_gemm(a_q, a_s, w_q, w_s, c1_d, mode=m.MOE_MODE_GROUPED, expert_offsets=od)
    q2 = torch.empty_like(q)
    s2 = torch.empty_like(s)
    m.act_quant(c1_d, q2, s2, act=m.MOE_ACT_SILU_MUL)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s.view(torch.int32), s2.view(torch.int32))
    e = 77
    r0, r1 = int(rt.expert_offsets[e]), int(rt.expert_offsets[e + 1])
    wq_e, ws_e = w_q[e:e + 1].cpu().numpy(), w_s[e:e + 1].cpu().numpy()
    aq_e, as_e = a_q[r0:r1].cpu().numpy(), a_s[r0:r1].cpu().numpy()
    offs_e = np.array([0, r1 - r0], np.int32)
    c1 = orc.block_gemm(aq_e, as_e, wq_e, ws_e, mode=orc.MODE_GROUPED, expert_offsets=offs_e, out_dtype=np.float32)
    ref_q, ref_s = orc.silu_mul_quant(c1)
    bound = gemm_abs_bound(aq_e, as_e, wq_e, ws_e, np.zeros(r1 - r0, np.int64), np.arange(r1 - r0))
    check_codes_and_scales(orc, q[r0:r1].cpu().numpy(), s[r0:r1].cpu().numpy(), ref_q, ref_s,
                           silu_h_bound(c1, bound, I))
