"""GPU check of moe_fused_decode_noalloc (the decode step on the library's fixed device scratch) through the
C ABI: on consecutive calls, the second with a smaller input, it must give the same bits as moe_fused_decode
with a caller workspace, and match the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import moe_routed_expert_amd as m
import oracle
import workloads as wl
from gpu_util import assert_bf16_close, dev, to_dev, u16

pytestmark = pytest.mark.gpu


def run_both(c, act=1):
    """One step through each entry point on the same inputs; returns (noalloc bits, workspace bits)."""
    d = dev()
    L = m.lib()
    x = c.x.to(d)
    slots, w = to_dev(c.slot_ids), to_dev(c.weights)
    w13_q, w13_s, w2_q, w2_s = (t.to(d) for t in (c.w13_q, c.w13_s, c.w2_q, c.w2_s))
    I = c.I
    out_na = torch.full((c.T, c.H), float("nan"), dtype=torch.bfloat16, device=d)
    out_ws = torch.full((c.T, c.H), float("nan"), dtype=torch.bfloat16, device=d)
    st = m._stream()
    print("noalloc decode T=%d H=%d I=%d topk=%d" % (c.T, c.H, I, c.topk), flush=True)
    rc = L.moe_fused_decode_noalloc(x.data_ptr(), c.T, c.H, I, c.topk, act, slots.data_ptr(), w.data_ptr(), c.n_slots,
                                    w13_q.data_ptr(), w13_s.data_ptr(), w2_q.data_ptr(), w2_s.data_ptr(),
                                    out_na.data_ptr(), st)
    assert rc == m.MOE_OK, L.moe_status_string(rc)
    size = m.fused_decode_workspace_size(c.T, c.H, I, c.topk)
    ws = torch.empty(size, dtype=torch.uint8, device=d)
    assert L.moe_fused_decode_workspace_init(ws.data_ptr(), size, c.T, c.H, I, c.topk, st) == m.MOE_OK
    rc = L.moe_fused_decode(x.data_ptr(), c.T, c.H, I, c.topk, act, slots.data_ptr(), w.data_ptr(), c.n_slots,
                            w13_q.data_ptr(), w13_s.data_ptr(), w2_q.data_ptr(), w2_s.data_ptr(), ws.data_ptr(),
                            size, out_ws.data_ptr(), st)
    assert rc == m.MOE_OK
    torch.cuda.synchronize()
    return u16(out_na), u16(out_ws)


def check(c, act=1):
    got, want = run_both(c, act)
    assert np.array_equal(got, want), "noalloc and workspace outputs differ"
    ref = oracle.fused_decode(c.x.view(torch.int16).numpy().view(np.uint16), c.slot_ids, c.weights,
                              *(t.numpy() for t in (c.w13_q, c.w13_s, c.w2_q, c.w2_s)), act=act)
    assert_bf16_close(got, ref, what="noalloc decode")


def test_noalloc_decode_matches_the_workspace_entry_point(orc):
    # two tokens, then one (a smaller input: the control block is cleared for the new shape), then the
    # same shape again with new inputs (its call counters continue), then the two-launch shape and back
    check(wl.decode_case(H=2048, I=768, topk=8, n_slots=16, active=6, seed=61, T=2))
    check(wl.decode_case(H=2048, I=768, topk=8, n_slots=16, active=5, seed=62, T=1))
    check(wl.decode_case(H=2048, I=768, topk=8, n_slots=16, active=8, seed=63, T=1))
    check(wl.decode_case(H=4096, I=1024, topk=8, n_slots=12, active=3, seed=64, T=1))
    check(wl.decode_case(H=2048, I=768, topk=8, n_slots=16, active=2, seed=65, T=1), act=2)


def test_noalloc_decode_rejects_steps_beyond_its_scratch():
    L = m.lib()
    d = dev()
    x = torch.zeros((32, 4096), dtype=torch.bfloat16, device=d)
    out = torch.full((32, 4096), float("nan"), dtype=torch.bfloat16, device=d)
    z = torch.zeros(16, dtype=torch.int32, device=d)
    rc = L.moe_fused_decode_noalloc(x.data_ptr(), 32, 4096, 1024, 8, 1, z.data_ptr(), z.data_ptr(), 0, None, None,
                                    None, None, out.data_ptr(), m._stream())
    assert rc == m.MOE_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()            # nothing was launched
