"""GPU parity of the fused decode step against the CPU oracle, including inactive (-1)
routes, NaN-poisoned workspaces and hipGraph replay with inputs changed in place
("perf(moe): skip inactive block-fp8 decode routes", Validation)."""
import numpy as np
import pytest
import torch

import moe_routed_expert_amd as m
import oracle
import workloads as wl
from gpu_util import assert_bf16_close, assert_close, assert_within_bound, dev, gemm_abs_bound, to_dev, u16


pytestmark = pytest.mark.gpu


class DevDecode:
    """A decode case resident on the GPU, with its workspace and output."""

    def __init__(self, c: wl.DecodeCase):
        d = dev()
        self.c = c
        self.x = c.x.to(d)
        self.slots = to_dev(c.slot_ids)
        self.w = to_dev(c.weights)
        self.wts = [t.to(d) for t in (c.w13_q, c.w13_s, c.w2_q, c.w2_s)]
        self.ws = m.fused_decode_workspace(c.T, c.H, c.I, c.topk, device=d)
        self.lay = m.fused_decode_workspace_layout(c.T, c.H, c.I, c.topk)
        self.out = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=d)

    def run(self, act=1):
        m.fused_decode(self.x, self.slots, self.w, *self.wts, self.ws, self.out, act=act)

    def region(self, name, dtype, shape):
        nbytes = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        return self.ws[self.lay[name]:self.lay[name] + nbytes].view(dtype).view(shape)

    def poison(self):
        self.ws[:self.lay["ctl"]].fill_(0xFF)          # NaN in every fp32 word, 0xFF codes
        self.out.fill_(float("nan"))


def oracle_decode(c: wl.DecodeCase, slots=None, weights=None, host_weights=None, act=1):
    xb = c.x.view(torch.int16).numpy().view(np.uint16)
    hw = host_weights or [t.cpu().numpy() for t in (c.w13_q, c.w13_s, c.w2_q, c.w2_s)]
    return oracle.fused_decode(xb, c.slot_ids if slots is None else slots, c.weights if weights is None else weights,
                               *hw, intermediates=True, act=act)


def gate64(act, g):
    """Gate functions of the five gated activations in float64 (scipy's erf and expit)."""
    from scipy.special import erf, expit
    return {1: lambda x: x * expit(x), 2: lambda x: x * 0.5 * (1 + erf(x / np.sqrt(2))),
            3: lambda x: np.maximum(x, 0), 4: expit, 5: lambda x: x}[act](g)


def one_launch_epoch_words(T, H, I, topk):
    """Epoch words of the one-launch step's control block (0 for shapes it never takes): one per
    gate/up tile of 8*M act columns and one per (token, 8-row down tile, route)."""
    g = I // 8
    if not (1 <= I // 128 <= 8 and (g % 2 == 0 or g % 3 == 0) and H // 128 <= 16 and H % 8 == 0
            and T * topk * (H // 8) <= 1 << 18):
        return 0
    M = 3 if g % 3 == 0 else 2
    return T * topk * (I // (8 * M)) + T * (H // 8) * topk


def check_ctl(dd: DevDecode):
    """The error word is clear, and every tile's epoch word holds the same call count (all zero when
    the step ran as several launches)."""
    c = dd.c
    ctl = dd.ws[dd.lay["ctl"]:dd.lay["total"]].view(torch.int32).cpu().numpy()
    assert ctl[0] == 0, "a hand-off wait gave up"
    n = one_launch_epoch_words(c.T, c.H, c.I, c.topk)
    ep = ctl[32:32 + n]
    assert n == 0 or np.all(ep == ep[0]), "tiles disagree on the call count"
    return int(ep[0]) if n else None


def one_launch_flag_words(T, H, I, topk):
    """(first word, word count) of the one-launch step's ready-word copies inside the control block:
    8 copies x routes x the route's gate/up tiles padded to 32 words, after the line-aligned epoch
    words; 0 words for shapes the step never takes."""
    n = one_launch_epoch_words(T, H, I, topk)
    if n == 0:
        return 0, 0
    g = I // 8
    tiles = I // (8 * (3 if g % 3 == 0 else 2))
    first = (32 + n + 31) // 32 * 32
    return first, 8 * T * topk * ((tiles + 31) // 32 * 32)


def check_against_oracle(dd: DevDecode, ref, im, host_weights=None, act=1):
    c = dd.c
    R = c.T * c.topk
    got = u16(dd.out)
    assert_bf16_close(got, ref, what="fused decode out")
    c1 = dd.region("c1", torch.float32, (R, 2 * c.I)).cpu().numpy()
    hh = dd.region("h", torch.float32, (R, c.I)).cpu().numpy()
    c2 = dd.region("c2", torch.float32, (R, c.H)).cpu().numpy()
    aq = dd.region("aq", torch.uint8, (R, c.I)).cpu().numpy()
    as_ = dd.region("as", torch.float32, (R, c.I // 128)).cpu().numpy()
    inactive = c.slot_ids.reshape(-1) < 0
    stores_h = c.I <= 1024                      # the four-launch form (wider I) never writes h
    for name, arr in (("c1", c1), ("h", hh), ("c2", c2), ("as", as_)):
        if name == "h" and not stores_h:
            continue
        assert np.all(arr[inactive].view(np.uint32) == 0), name + ": inactive rows must be +0.0"
    assert np.all(aq[inactive] == 0)
    check_ctl(dd)
    if (~inactive).any():
        hw = host_weights or [t.cpu().numpy() for t in (c.w13_q, c.w13_s)]
        bound = gemm_abs_bound(im["xq"], im["xs"], hw[0], hw[1], c.slot_ids.reshape(-1), np.arange(R) // c.topk)
        assert_within_bound(c1, im["c1"], bound, what="c1")
        g, u = im["c1"][:, :c.I].astype(np.float64), im["c1"][:, c.I:].astype(np.float64)
        if stores_h:
            assert_close(hh[~inactive], (gate64(act, g) * u)[~inactive], rel_l2=1e-4, max_abs=1e-4, what="h")
        assert_close(c2[~inactive], im["c2"][~inactive], what="c2")


@pytest.mark.parametrize("active", [1])
def test_fused_decode_tiny(orc, active):
    c = wl.decode_case(H=256, I=128, topk=2, n_slots=8, active=active, seed=0)
    dd = DevDecode(c)
    dd.poison()
    dd.run()
    torch.cuda.synchronize()
    ref, im = oracle_decode(c)
    check_against_oracle(dd, ref, im)


@pytest.mark.parametrize("H,I", [(2048, 768), (4096, 1024)])
@pytest.mark.parametrize("active", [8, 4, 2, 0])
def test_fused_decode_full_configs(orc, H, I, active):
    print("fused decode H=%d I=%d active=%d/8" % (H, I, active), flush=True)
    c = wl.decode_case(H=H, I=I, topk=8, n_slots=64, active=active, seed=H + active, device="cuda")
    host = [t.cpu().numpy() for t in (c.w13_q, c.w13_s, c.w2_q, c.w2_s)]
    c.x = c.x.cpu()
    dd = DevDecode(c)
    dd.poison()
    dd.run()
    torch.cuda.synchronize()
    ref, im = oracle_decode(c, host_weights=host)
    check_against_oracle(dd, ref, im, host_weights=host)
    if active == 0:
        assert np.all(u16(dd.out) == 0)


@pytest.mark.parametrize("act", [2, 3, 4, 5])
@pytest.mark.parametrize("H,I,T", [(256, 128, 1), (2048, 768, 1), (4096, 1024, 1), (256, 1152, 2)])
def test_fused_decode_gated_activations(orc, act, H, I, T):
    """The other four gated activations (GEGLU, ReGLU, GLU, bilinear) through every form of the fused
    decode: one launch (256/128, 2048/768), two launches (H = 4096) and four (I = 1152 > 1024)."""
    print("fused decode act=%d H=%d I=%d T=%d" % (act, H, I, T), flush=True)
    c = wl.decode_case(H=H, I=I, topk=4, n_slots=12, active=3, seed=act + H, T=T)
    dd = DevDecode(c)
    dd.poison()
    dd.run(act=act)
    torch.cuda.synchronize()
    ref, im = oracle_decode(c, act=act)
    check_against_oracle(dd, ref, im, act=act)


@pytest.mark.parametrize("T,H,I,topk,active", [(2, 512, 256, 4, 3), (3, 256, 384, 2, 1), (1, 1024, 128, 1, 1),
                                                (2, 1024, 768, 4, 3)])
def test_fused_decode_one_launch_shapes(orc, T, H, I, topk, active):
    """Shapes the one-launch step takes beyond batch 1 and top-8: several tokens (down tiles and
    epoch words per token), top-1, I/8 a multiple of 3 (24-column tiles) and of 2 only (16-column),
    a 128-wide I (one act group); every one checked against the oracle, twice in a row."""
    print("fused decode T=%d H=%d I=%d topk=%d" % (T, H, I, topk), flush=True)
    c = wl.decode_case(H=H, I=I, topk=topk, n_slots=12, active=active, seed=T * 100 + H + I, T=T)
    dd = DevDecode(c)
    ref, im = oracle_decode(c)
    for _ in range(2):
        dd.poison()
        dd.run()
        torch.cuda.synchronize()
        check_against_oracle(dd, ref, im)
    assert check_ctl(dd) == 2, "the step did not run as one launch"


def test_fused_decode_batch_of_tokens(orc):
    c = wl.decode_case(H=512, I=256, topk=4, n_slots=10, active=3, seed=11, T=5)
    dd = DevDecode(c)
    dd.poison()
    dd.run()
    torch.cuda.synchronize()
    ref, im = oracle_decode(c)
    check_against_oracle(dd, ref, im)


def test_negative_slots_match_clamped_zero_weight_path_on_gpu(orc):
    """The old path (inactive -> slot 0, weight 0) gives exactly the same output."""
    c = wl.decode_case(H=2048, I=768, topk=8, n_slots=16, active=2, seed=21)
    dd = DevDecode(c)
    dd.run()
    torch.cuda.synchronize()
    new = u16(dd.out).copy()
    dd.slots.copy_(to_dev(np.where(c.slot_ids < 0, 0, c.slot_ids).astype(np.int32)))
    dd.w.copy_(to_dev(np.where(c.slot_ids < 0, 0.0, c.weights).astype(np.float32)))
    dd.run()
    torch.cuda.synchronize()
    assert np.array_equal(u16(dd.out), new)


def test_inactive_routing_weights_never_read(orc):
    c = wl.decode_case(H=2048, I=768, topk=8, n_slots=16, active=3, seed=22)
    dd = DevDecode(c)
    dd.run()
    torch.cuda.synchronize()
    base = u16(dd.out).copy()
    w = c.weights.copy()
    w[c.slot_ids < 0] = np.nan
    dd.w.copy_(to_dev(w))
    dd.run()
    torch.cuda.synchronize()
    assert np.array_equal(u16(dd.out), base)


def test_graph_replay_with_changing_inputs_and_poison(orc):
    """One captured graph serves all-active, mixed and all-inactive steps; inputs change in place,
    workspaces are NaN-poisoned before each replay, and every replay equals the eager result."""
    H, I, S, topk = 2048, 768, 32, 8
    base = wl.decode_case(H=H, I=I, topk=topk, n_slots=S, active=8, seed=31)
    dd = DevDecode(base)
    host_w = [t.cpu().numpy() for t in (base.w13_q, base.w13_s, base.w2_q, base.w2_s)]
    steps = []
    for i, active in enumerate((8, 3, 0, 5, 8, 1)):
        x = wl.bf16_normal((1, H), seed=100 + i)
        slots, w = wl.decode_slots(1, topk, S, active, seed=200 + i, tail=(i == 3))
        steps.append((x, slots, w))
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    dd.run()                                   # warm-up outside capture
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        dd.run()
    for i, (x, slots, w) in enumerate(steps):
        dd.x.copy_(x.to(dev()))
        dd.slots.copy_(to_dev(slots))
        dd.w.copy_(to_dev(w))
        dd.poison()
        g.replay()
        torch.cuda.synchronize()
        replay_out = u16(dd.out).copy()
        c = wl.DecodeCase(1, H, I, topk, S, x, slots, w, base.w13_q, base.w13_s, base.w2_q, base.w2_s)
        dd.c = c
        ref, im = oracle_decode(c, host_weights=host_w)
        check_against_oracle(dd, ref, im, host_weights=host_w)
        dd.poison()
        dd.run()                               # eager, same inputs
        torch.cuda.synchronize()
        assert np.array_equal(u16(dd.out), replay_out), "replay %d differs from eager" % i
        if (slots < 0).all():
            assert np.all(replay_out == 0)
    # one warm-up call, then a replay and an eager call per step: the one-launch step counts each
    assert check_ctl(dd) in (None, 0, 1 + 2 * len(steps))


def test_chained_layers_in_one_graph_like_the_benchmark(orc):
    """The benchmark's launch configuration: chained decode layers (each with its own 64-slot pool,
    layer l+1 reading layer l's output) captured in one graph; every layer checked against the oracle
    on the token row the device actually fed it."""
    H, I, S, topk, L = 2048, 768, 64, 8, 4
    d = dev()
    pools = [wl.block_fp8_weights(S, 2 * I, H, 900 + 2 * l, device="cuda") +
             wl.block_fp8_weights(S, H, I, 901 + 2 * l, device="cuda") for l in range(L)]
    x0 = wl.bf16_normal((1, H), seed=5, device="cuda")
    outs = [torch.empty((1, H), dtype=torch.bfloat16, device=d) for _ in range(L)]
    routes = [wl.decode_slots(1, topk, S, (8, 3, 8, 0)[l], seed=40 + l) for l in range(L)]
    routes_d = [(to_dev(sl), to_dev(w)) for sl, w in routes]
    ws = m.fused_decode_workspace(1, H, I, topk, device=d)

    def step_all():
        x = x0
        for l in range(L):
            m.fused_decode(x, routes_d[l][0], routes_d[l][1], *pools[l], ws, outs[l])
            x = outs[l]

    step_all()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        step_all()
    for o in outs:
        o.fill_(float("nan"))
    g.replay()
    g.replay()
    torch.cuda.synchronize()
    x_in = u16(x0)
    for l in range(L):
        host = [t.cpu().numpy() for t in pools[l]]
        ref = oracle.fused_decode(x_in, routes[l][0], routes[l][1], *host)
        got = u16(outs[l])
        assert_bf16_close(got, ref, what="layer %d" % l)
        x_in = got
    assert np.all(u16(outs[3]) == 0)                 # layer 3 has no active route
    ctl = ws[m.fused_decode_workspace_layout(1, H, I, topk)["ctl"]:].view(torch.int32)
    assert int(ctl[0]) == 0, "a hand-off wait gave up"
    # one eager call, then two replays of L layers sharing the workspace: each call bumps every epoch
    assert int(ctl[32]) == 3 * L


@pytest.mark.parametrize("active", [8, 5, 0])
def test_fused_decode_narrow_two_launch_down_tiles(orc, active):
    """H = 3072 (H/128 = 24 > 16, so never one launch; 3072/16 = 192 wide tiles would not fill the CUs, so the
    8-row down tiles run): against the oracle with a NaN-poisoned workspace, and the one-launch step's epoch
    words stay 0."""
    print("fused decode H=3072 I=768 active=%d/8" % active, flush=True)
    c = wl.decode_case(H=3072, I=768, topk=8, n_slots=16, active=active, seed=3072 + active)
    dd = DevDecode(c)
    assert one_launch_epoch_words(c.T, c.H, c.I, c.topk) == 0
    dd.poison()
    dd.run()
    torch.cuda.synchronize()
    ref, im = oracle_decode(c)
    check_against_oracle(dd, ref, im)
    ctl = dd.ws[dd.lay["ctl"]:dd.lay["total"]].view(torch.int32).cpu().numpy()
    assert np.all(ctl[2:] == 0) and ctl[0] == 0


@pytest.mark.parametrize("T,I,topk,active", [(1, 1024, 3, 2), (2, 512, 8, 5)])
def test_fused_decode_wide_two_launch_down_tiles_other_shapes(orc, T, I, topk, active):
    """H = 4096 beyond the 4096/1024 top-8 step: top-3 of one token and two tokens at I = 512, both run as
    two launches with 16-row down tiles: against the oracle with a NaN-poisoned workspace, and the control
    block is never written past its shape word."""
    H = 4096
    print("fused decode two launches T=%d H=%d I=%d topk=%d" % (T, H, I, topk), flush=True)
    assert one_launch_epoch_words(T, H, I, topk) == 0
    c = wl.decode_case(H=H, I=I, topk=topk, n_slots=12, active=active, seed=4096 + T + I + topk, T=T)
    dd = DevDecode(c)
    dd.poison()
    dd.run()
    torch.cuda.synchronize()
    ref, im = oracle_decode(c)
    check_against_oracle(dd, ref, im)
    ctl = dd.ws[dd.lay["ctl"]:dd.lay["total"]].view(torch.int32).cpu().numpy()
    assert np.all(ctl[2:] == 0) and ctl[0] == 0


def test_workspace_of_another_shape_sets_the_error_word(orc):
    """A workspace initialized for one shape and passed with another (large enough for both): the one-launch
    step sees the shape word disagree, waits on no hand-off word and sets the error word to 2; a fresh init
    for the right shape clears it and the step matches the oracle again."""
    c = wl.decode_case(H=1024, I=768, topk=8, n_slots=12, active=6, seed=51)
    d = dev()
    size = max(m.fused_decode_workspace_size(1, 2048, 768, 8), m.fused_decode_workspace_size(1, 1024, 768, 8))
    dd = DevDecode(c)
    dd.ws = torch.empty(size, dtype=torch.uint8, device=d)
    assert m.lib().moe_fused_decode_workspace_init(dd.ws.data_ptr(), size, 1, 2048, 768, 8,
                                                   m._stream()) == m.MOE_OK
    dd.run()
    torch.cuda.synchronize()
    assert int(dd.ws[dd.lay["ctl"]:dd.lay["ctl"] + 4].view(torch.int32)[0]) == 2
    assert m.lib().moe_fused_decode_workspace_init(dd.ws.data_ptr(), size, 1, 1024, 768, 8,
                                                   m._stream()) == m.MOE_OK
    dd.poison()
    dd.run()
    torch.cuda.synchronize()
    ref, im = oracle_decode(c)
    check_against_oracle(dd, ref, im)
    assert check_ctl(dd) == 1, "the step did not run as one launch"


def test_ready_words_ahead_of_h_fall_back_to_coherent_loads(orc):
    """A ready word seen before its tile's h: every ready word is set to the next call's tag before the
    call, so the down tiles read h at once, find the previous call's tags (and, on each XCD, stale L2
    lines), and must wait on coherent loads of h itself; the output still equals the oracle's."""
    c = wl.decode_case(H=2048, I=768, topk=8, n_slots=16, active=6, seed=41)
    dd = DevDecode(c)
    dd.run()
    torch.cuda.synchronize()
    calls = check_ctl(dd)
    if calls is None or calls == 0:
        pytest.skip("the step did not run as one launch on this device")
    first, count = one_launch_flag_words(c.T, c.H, c.I, c.topk)
    ctl = dd.ws[dd.lay["ctl"]:dd.lay["total"]].view(torch.int32)
    ctl[first:first + count] = calls + 1
    dd.poison()
    dd.run()
    torch.cuda.synchronize()
    ref, im = oracle_decode(c)
    check_against_oracle(dd, ref, im)
    assert check_ctl(dd) == calls + 1
