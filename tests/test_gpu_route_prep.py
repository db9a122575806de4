"""GPU parity of the routing prep (top-k, renormalized weights, (expert, token) route maps) against
the CPU oracle: expert ids and all three maps bit-exact, weights within a derived fp32 bound."""
import numpy as np
import pytest
import torch

import moe_routed_expert_amd as m
import workloads as wl
from gpu_util import dev, to_dev

pytestmark = pytest.mark.gpu


def weight_bound(lg, ids, topk):
    """Per-weight relative bound between the device (fp32: expf, a wave sum, one divide) and the
    oracle (fp64, rounded once to fp32).  Each term e_j = exp(d_j), d_j = l_j - l_max: the fp32
    difference rounds with relative 2^-24, i.e. absolute |d_j| 2^-24 in the exponent, and expf adds
    at most 2 ulp (4 * 2^-24), so e_j is within (4 + |d_j|) 2^-24.  The sum of topk terms is within
    the worst term's error plus (topk - 1) 2^-24; the divide and the oracle's final rounding add
    2^-24 each.  A 1% margin covers the second-order terms."""
    l_sel = np.take_along_axis(lg.astype(np.float64), ids.astype(np.int64), axis=1)
    d = np.abs(l_sel - l_sel[:, :1])
    return 1.01 * (4.0 + d + 4.0 + d.max(axis=1, keepdims=True) + (topk - 1) + 2.0) * 2.0 ** -24


def run(lg, topk, stride=None):
    T, E = lg.shape
    if stride is not None and stride > E:
        buf = np.full((T, stride), np.float32(1e30))
        buf[:, :E] = lg
        x = to_dev(buf)[:, :E]
    else:
        x = to_dev(lg)
    ids, w, d2s, rr, offs = m.route_prep(x, topk)
    torch.cuda.synchronize()
    return dict(expert_ids=ids.cpu().numpy(), weights=w.cpu().numpy(), dst2src=d2s.cpu().numpy(),
                route_rows=rr.cpu().numpy(), expert_offsets=offs.cpu().numpy())


def check(orc, lg, topk, stride=None):
    T, E = lg.shape
    print("route_prep T=%d E=%d topk=%d stride=%s" % (T, E, topk, stride), flush=True)
    got = run(lg, topk, stride)
    ref = orc.route_prep(lg, topk)
    for key in ("expert_ids", "dst2src", "route_rows", "expert_offsets"):
        assert np.array_equal(got[key].reshape(ref[key].shape), ref[key]), key
    if T:
        rel = np.abs(got["weights"].astype(np.float64) - ref["weights"]) / ref["weights"]
        bound = weight_bound(lg, ref["expert_ids"], topk)
        assert np.all(rel <= bound), "weights: worst rel %.3e" % rel.max()
    return got


@pytest.mark.parametrize("T,E,topk,skew", [(4096, 256, 8, 0.0), (4096, 256, 8, 1.0), (1, 256, 8, 0.0),
                                           (65, 256, 8, 0.5), (127, 64, 6, 0.0), (3000, 128, 4, 2.0),
                                           (200, 1024, 16, 0.0), (33, 7, 3, 0.0), (64, 64, 64, 0.0),
                                           (5, 1, 1, 0.0), (1024, 160, 6, 1.0)])
def test_route_prep_matches_oracle(orc, T, E, topk, skew):
    check(orc, wl.router_logits(T, E, seed=T + 31 * E + topk, skew=skew), topk)


def test_route_prep_strided_logits(orc):
    check(orc, wl.router_logits(300, 96, seed=3), 6, stride=100)


def test_route_prep_ties_and_signed_zero(orc):
    lg = np.zeros((70, 40), np.float32)
    lg[5, 7] = 1.0
    lg[9, :] = -0.0
    lg[9, 3] = 0.0
    lg[10, ::2] = 2.5                    # half the experts tie at the top
    got = check(orc, lg, 5)
    assert got["expert_ids"][0].tolist() == [0, 1, 2, 3, 4]
    assert np.all(got["weights"][0] == np.float32(0.2))
    assert got["expert_ids"][10].tolist() == [0, 2, 4, 6, 8]


def test_route_prep_no_tokens():
    offs = torch.full((9,), 77, dtype=torch.int32, device=dev())
    size = m.lib().moe_route_prep_workspace_size(0, 8)
    ws = torch.empty(size, dtype=torch.uint8, device=dev())
    rc = m.lib().moe_route_prep(None, 8, 0, 8, 2, None, None, None, None, offs.data_ptr(), ws.data_ptr(), size, None)
    torch.cuda.synchronize()
    assert rc == m.MOE_OK and np.all(offs.cpu().numpy() == 0)


def test_route_prep_feeds_the_gather_and_reduce_maps(orc):
    """The device maps are consistent with each other: dst2src[route_rows[t, j]] == t, rows of
    expert e carry expert id e, and each expert's rows hold increasing tokens."""
    T, E, topk = 2048, 256, 8
    got = run(wl.router_logits(T, E, seed=9, skew=1.0), topk)
    rr = got["route_rows"].reshape(T, topk)
    assert np.array_equal(got["dst2src"][rr], np.repeat(np.arange(T)[:, None], topk, axis=1))
    offs = got["expert_offsets"]
    ids = got["expert_ids"]
    row_e = np.empty(T * topk, np.int64)
    row_e[rr.ravel()] = ids.ravel()
    for e in range(E):
        seg = slice(offs[e], offs[e + 1])
        assert np.all(row_e[seg] == e)
        assert np.all(np.diff(got["dst2src"][seg]) > 0)


def test_prefill_layer_on_device_from_logits(orc):
    """Routing prep -> input quant -> gather -> fused gate/up + SiLU-mul requant -> down -> top-k reduce,
    every step on the device, against the oracle's chain on the same logits, activations and weights."""
    from gpu_util import assert_bf16_close, u16
    T, E, topk, H, I = 200, 16, 4, 512, 256
    lg = wl.router_logits(T, E, seed=3, skew=1.0)
    x = wl.bf16_normal((T, H), seed=4)
    w13_q, w13_s = wl.block_fp8_weights(E, 2 * I, H, seed=5)
    w2_q, w2_s = wl.block_fp8_weights(E, H, I, seed=6)
    # oracle chain (c1 in fp32, as the fused step keeps it)
    r = orc.route_prep(lg, topk)
    xq, xs = orc.quant_groups(x.view(torch.int16).numpy().view(np.uint16))
    gq, gs = orc.gather_rows_scales(xq, xs, r["dst2src"])
    c1 = orc.block_gemm(gq, gs, w13_q.numpy(), w13_s.numpy(), mode=orc.MODE_GROUPED,
                        expert_offsets=r["expert_offsets"], out_dtype=np.float32)
    aq, as_ = orc.silu_mul_quant(c1)
    c2 = orc.block_gemm(aq, as_, w2_q.numpy(), w2_s.numpy(), mode=orc.MODE_GROUPED,
                        expert_offsets=r["expert_offsets"], out_dtype=np.uint16)
    ref = orc.topk_reduce(c2, r["expert_ids"], r["weights"], route_rows=r["route_rows"])
    # device chain
    d = dev()
    R = T * topk
    ids, w, d2s, rr, offs = m.route_prep(to_dev(lg), topk)
    xq_d = torch.empty((T, H), dtype=torch.uint8, device=d)
    xs_d = torch.empty((T, H // 128), dtype=torch.float32, device=d)
    m.act_quant(x.to(d), xq_d, xs_d)
    gq_d = torch.empty((R, H), dtype=torch.uint8, device=d)
    gs_d = torch.empty((R, H // 128), dtype=torch.float32, device=d)
    m.gather_rows_scales(xq_d, xs_d, d2s, gq_d, gs_d)
    aq_d = torch.empty((R, I), dtype=torch.uint8, device=d)
    as_d = torch.empty((R, I // 128), dtype=torch.float32, device=d)
    m.bf8_grouped_gemm_act_quant(gq_d, gs_d, w13_q.to(d), w13_s.to(d), offs, aq_d, as_d)
    c2_d = torch.empty((R, H), dtype=torch.bfloat16, device=d)
    m.bf8_grouped_gemm(aq_d, as_d, w2_q.to(d), w2_s.to(d), c2_d, mode=m.MOE_MODE_GROUPED, expert_offsets=offs)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=d)
    m.topk_reduce(c2_d, ids, w, out, route_rows=rr)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), r["expert_ids"]) and np.array_equal(d2s.cpu().numpy(), r["dst2src"])
    assert np.array_equal(gq_d.cpu().numpy(), gq)
    assert_bf16_close(u16(out), ref, what="prefill layer out")
