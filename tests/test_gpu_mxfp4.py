"""GPU parity of the grouped GEMM with MXFP4 expert weights (plain output and the fused gate/up gated-activation
requant) against the CPU oracle."""
import numpy as np
import pytest
import torch

import moe_routed_expert_amd as m
import workloads as wl
from gpu_util import (NP_OUT, assert_close, assert_within_bound, check_codes_and_scales, dev, host_out,
                      mxfp4_abs_bound, ref_as_f64, silu_h_bound, to_dev)

pytestmark = pytest.mark.gpu


def mx_case(E, N, K, counts, seed):
    w4, w4_s = wl.mxfp4_weights(E, N, K, seed=seed)
    R = int(sum(counts))
    a_q, a_s = wl.fp8_rows(R, K, seed=seed + 1)
    offs = np.zeros(E + 1, np.int32)
    offs[1:] = np.cumsum(counts)
    return w4.numpy(), w4_s.numpy(), a_q.numpy(), a_s.numpy(), offs


@pytest.mark.parametrize("bm", [0, 16, 32, 64, 128])
@pytest.mark.parametrize("odt", [torch.bfloat16, torch.float32, torch.float16])
def test_mxfp4_grouped_gemm_vs_oracle(orc, bm, odt):
    E, N, K = 5, 384, 640
    counts = [3, 0, 40, 129, 17]        # empty expert, ragged tails, several M tiles, a 128-column N tail tile
    print("mxfp4 grouped gemm BM=%d %s" % (bm, odt), flush=True)
    w4, w4_s, a_q, a_s, offs = mx_case(E, N, K, counts, seed=200 + bm)
    ref = orc.mxfp4_gemm(a_q, a_s, w4, w4_s, mode=orc.MODE_GROUPED, expert_offsets=offs, out_dtype=NP_OUT[odt])
    R = int(offs[-1])
    out = torch.full((R + 3, N), float("nan"), dtype=odt, device=dev())   # 3 spare rows stay untouched
    m.mxfp4_grouped_gemm(to_dev(a_q), to_dev(a_s), to_dev(w4), to_dev(w4_s), to_dev(offs), out, m_rows=R + 3,
                         block_m=bm)
    torch.cuda.synchronize()
    got = host_out(out)
    assert np.all(np.isnan(got[R:]))
    if odt == torch.float32:
        experts = np.repeat(np.arange(E), np.diff(offs))
        bound = mxfp4_abs_bound(a_q, a_s, w4, w4_s, experts, np.arange(R))
        assert_within_bound(got[:R], ref, bound, what="mxfp4 gemm f32")
    assert_close(got[:R], ref_as_f64(ref, odt), what="mxfp4 gemm")


def test_mxfp4_grouped_gemm_exact_case_bit_exact(orc):
    """Operands whose every partial sum is exact in fp32: the device equals the oracle bit for bit at every
    tile, which pins the nibble order, the K order of both MFMA operands and the scale-to-block pairing."""
    E, N, K = 4, 256, 1024
    counts = [20, 1, 0, 70]
    a_q, a_s, w4, w4_s = wl.mxfp4_exact_case(E, N, K, sum(counts), seed=11)
    offs = np.zeros(E + 1, np.int32)
    offs[1:] = np.cumsum(counts)
    ref = orc.mxfp4_gemm(a_q, a_s, w4, w4_s, mode=orc.MODE_GROUPED, expert_offsets=offs)
    assert np.abs(ref).max() > 100.0
    for bm in (16, 32, 64, 128):
        out = torch.empty((offs[-1], N), dtype=torch.float32, device=dev())
        m.mxfp4_grouped_gemm(to_dev(a_q), to_dev(a_s), to_dev(w4), to_dev(w4_s), to_dev(offs), out, block_m=bm)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32)), bm


def test_mxfp4_strided_operands(orc):
    """Padded rows and expert strides (bytes) are honoured: a view into larger buffers gives the same bits as
    the packed call."""
    E, N, K = 3, 256, 512
    counts = [9, 33, 5]
    w4, w4_s, a_q, a_s, offs = mx_case(E, N, K, counts, seed=7)
    d = dev()
    R = int(offs[-1])
    big_w = torch.zeros((E, N + 8, K // 2 + 48), dtype=torch.uint8, device=d)
    big_w[:, :N, :K // 2] = to_dev(w4)
    big_s = torch.zeros((E, N + 4, K // 32 + 12), dtype=torch.uint8, device=d)
    big_s[:, :N, :K // 32] = to_dev(w4_s)
    big_a = torch.zeros((R, K + 32), dtype=torch.uint8, device=d)
    big_a[:, :K] = to_dev(a_q)
    out = torch.empty((R, N + 64), dtype=torch.float32, device=d)
    m.mxfp4_grouped_gemm(big_a[:, :K], to_dev(a_s), big_w[:, :N, :K // 2], big_s[:, :N, :K // 32], to_dev(offs),
                         out[:, :N])
    ref_out = torch.empty((R, N), dtype=torch.float32, device=d)
    m.mxfp4_grouped_gemm(to_dev(a_q), to_dev(a_s), to_dev(w4), to_dev(w4_s), to_dev(offs), ref_out)
    torch.cuda.synchronize()
    assert torch.equal(out[:, :N].view(torch.int32), ref_out.view(torch.int32))


@pytest.mark.parametrize("bm,act", [(0, 1), (16, 1), (32, 1), (64, 1), (128, 1), (64, 2), (128, 3), (32, 4),
                                    (16, 5)])
def test_mxfp4_gate_up_act_quant_vs_oracle_and_unfused(orc, bm, act):
    """The fused MXFP4 gate/up + gated-activation requant equals the oracle's fp32 MXFP4 GEMM followed by its
    requant (within the derived bound), and the device's unfused pair bit for bit."""
    E, I, K = 5, 256, 640
    counts = [3, 0, 40, 129, 17]
    print("mxfp4 fused gate/up act-quant BM=%d act=%d" % (bm, act), flush=True)
    w4, w4_s, a_q, a_s, offs = mx_case(E, 2 * I, K, counts, seed=300 + bm + act)
    R = int(offs[-1])
    c1 = orc.mxfp4_gemm(a_q, a_s, w4, w4_s, mode=orc.MODE_GROUPED, expert_offsets=offs, out_dtype=np.float32)
    ref_q, ref_s = orc.gated_act_quant(c1, act)
    d = dev()
    q = torch.full((R + 2, I), 0xAB, dtype=torch.uint8, device=d)          # 2 spare rows stay untouched
    s = torch.full((R + 2, I // 128), float("nan"), dtype=torch.float32, device=d)
    w4d, w4sd, aq, as_, od = to_dev(w4), to_dev(w4_s), to_dev(a_q), to_dev(a_s), to_dev(offs)
    m.mxfp4_grouped_gemm_act_quant(aq, as_, w4d, w4sd, od, q, s, m_rows=R + 2, block_m=bm, act=act)
    c1_d = torch.empty((R, 2 * I), dtype=torch.float32, device=d)
    m.mxfp4_grouped_gemm(aq, as_, w4d, w4sd, od, c1_d, block_m=bm)
    q2 = torch.empty((R, I), dtype=torch.uint8, device=d)
    s2 = torch.empty((R, I // 128), dtype=torch.float32, device=d)
    m.act_quant(c1_d, q2, s2, act=act)
    torch.cuda.synchronize()
    hq, hs = q.cpu().numpy(), s.cpu().numpy()
    assert np.all(hq[R:] == 0xAB) and np.all(np.isnan(hs[R:]))
    assert np.array_equal(hq[:R], q2.cpu().numpy()) and np.array_equal(hs[:R].view(np.uint32),
                                                                      s2.cpu().numpy().view(np.uint32))
    experts = np.repeat(np.arange(E), np.diff(offs))
    c1_bound = mxfp4_abs_bound(a_q, a_s, w4, w4_s, experts, np.arange(R))
    assert_within_bound(c1_d.cpu().numpy(), c1, c1_bound, what="mxfp4 c1")
    check_codes_and_scales(orc, hq[:R], hs[:R], ref_q, ref_s, silu_h_bound(c1, c1_bound, I, act))


def test_mxfp4_prefill_layer_full_size(orc):
    """At the 24576-route prefill size (E=256, top-6, H=4096, I=1024) in the picker's launch: the fused gate/up
    equals the unfused device pair bit for bit, and rows of one sampled expert match the oracle in the gate/up
    codes and the down output."""
    E, topk, H, I, T = 256, 6, 4096, 1024, 4096
    print("mxfp4 prefill layer at 24576 routes", flush=True)
    d = dev()
    w13, w13_s = wl.mxfp4_weights(E, 2 * I, H, seed=31, device=d)
    w2, w2_s = wl.mxfp4_weights(E, H, I, seed=32, device=d)
    rt = wl.prefill_routes(T, E, topk, seed=9)
    R = T * topk
    od = to_dev(rt.expert_offsets)
    a_q, a_s = wl.fp8_rows(R, H, seed=33, device=d)
    q = torch.empty((R, I), dtype=torch.uint8, device=d)
    s = torch.empty((R, I // 128), dtype=torch.float32, device=d)
    m.mxfp4_grouped_gemm_act_quant(a_q, a_s, w13, w13_s, od, q, s)
    c1_d = torch.empty((R, 2 * I), dtype=torch.float32, device=d)
    m.mxfp4_grouped_gemm(a_q, a_s, w13, w13_s, od, c1_d)
    q2 = torch.empty_like(q)
    s2 = torch.empty_like(s)
    m.act_quant(c1_d, q2, s2, act=m.MOE_ACT_SILU_MUL)
    y = torch.empty((R, H), dtype=torch.bfloat16, device=d)
    m.mxfp4_grouped_gemm(q, s, w2, w2_s, od, y)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s.view(torch.int32), s2.view(torch.int32))
    e = 141
    r0, r1 = int(rt.expert_offsets[e]), int(rt.expert_offsets[e + 1])
    assert r1 - r0 > 40
    r1 = r0 + 40           # the first 40 of its rows: three 16-row MFMA tiles with a ragged one
    offs_e = np.array([0, r1 - r0], np.int32)
    rows = np.arange(r1 - r0)
    w13_e, w13s_e = w13[e:e + 1].cpu().numpy(), w13_s[e:e + 1].cpu().numpy()
    aq_e, as_e = a_q[r0:r1].cpu().numpy(), a_s[r0:r1].cpu().numpy()
    c1 = orc.mxfp4_gemm(aq_e, as_e, w13_e, w13s_e, mode=orc.MODE_GROUPED, expert_offsets=offs_e,
                        out_dtype=np.float32)
    ref_q, ref_s = orc.silu_mul_quant(c1)
    bound = mxfp4_abs_bound(aq_e, as_e, w13_e, w13s_e, np.zeros(r1 - r0, np.int64), rows)
    check_codes_and_scales(orc, q[r0:r1].cpu().numpy(), s[r0:r1].cpu().numpy(), ref_q, ref_s,
                           silu_h_bound(c1, bound, I))
    # the down rows of this expert from the device's own codes
    w2_e, w2s_e = w2[e:e + 1].cpu().numpy(), w2_s[e:e + 1].cpu().numpy()
    ref_y = orc.mxfp4_gemm(q[r0:r1].cpu().numpy(), s[r0:r1].cpu().numpy(), w2_e, w2s_e, mode=orc.MODE_GROUPED,
                           expert_offsets=offs_e, out_dtype=np.uint16)
    assert_close(host_out(y[r0:r1]), ref_as_f64(ref_y, torch.bfloat16), what="mxfp4 down")
