"""GPU parity of the gather, the 1x128 quantizer and the top-k reduce against the CPU oracle."""
import numpy as np
import pytest
import torch

import moe_routed_expert_amd as m
import oracle
import workloads as wl
from gpu_util import assert_bf16_close, assert_close, dev, to_dev, u16

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ gather ---

@pytest.mark.parametrize("k,tokens", [(7168, 1), (2048, 1), (7168, 8), (7168, 64), (7168, 1024),
                                      (896, 16), (896, 1), (4096, 100), (100, 7), (16, 33)])
def test_gather_bit_exact(orc, k, tokens):
    print("gather k=%d tokens=%d" % (k, tokens), flush=True)
    src_q, src_s, mp = wl.gather_case(k, tokens, 8, seed=1000 + k + tokens)
    g = src_s.shape[1]
    ref_q, ref_s = orc.gather_rows_scales(src_q, src_s.view(np.float32), mp)
    dq = torch.full((len(mp), k), 0xAB, dtype=torch.uint8, device=dev())
    ds = torch.full((len(mp), g), -1, dtype=torch.int32, device=dev())
    m.gather_rows_scales(to_dev(src_q), to_dev(src_s).view(torch.float32), to_dev(mp), dq, ds.view(torch.float32))
    torch.cuda.synchronize()
    assert np.array_equal(dq.cpu().numpy(), ref_q)
    assert np.array_equal(ds.cpu().numpy(), ref_s.view(np.int32))
    assert np.array_equal(dq.cpu().numpy(), src_q[mp])     # the plain-indexing oracle too


def test_gather_strided_negative_and_empty(orc):
    k, tokens = 896, 5
    src_q, src_s, _ = wl.gather_case(k, tokens, 8, seed=77)
    mp = np.array([4, -1, 0, 0, 3, -7, 2, 1], np.int32)
    # destination rows padded to 1024 bytes and 9 scale words
    dq = torch.full((8, 1024), 0xCD, dtype=torch.uint8, device=dev())
    ds = torch.full((8, 9), 12345, dtype=torch.int32, device=dev())
    m.gather_rows_scales(to_dev(src_q), to_dev(src_s).view(torch.float32), to_dev(mp),
                         dq, ds.view(torch.float32), k=k, g=7)
    torch.cuda.synchronize()
    ref_q, ref_s = orc.gather_rows_scales(src_q, src_s.view(np.float32), mp)
    hq, hs = dq.cpu().numpy(), ds.cpu().numpy()
    assert np.array_equal(hq[:, :k], ref_q) and np.all(hq[:, k:] == 0xCD)
    assert np.array_equal(hs[:, :7], ref_s.view(np.int32)) and np.all(hs[:, 7:] == 12345)
    # empty map: nothing written
    e = torch.zeros(0, dtype=torch.int32, device=dev())
    m.gather_rows_scales(to_dev(src_q), to_dev(src_s).view(torch.float32), e, dq, ds.view(torch.float32))
    torch.cuda.synchronize()
    assert np.array_equal(dq.cpu().numpy(), hq)


@pytest.mark.parametrize("tokens", [8, 300])
def test_gather_without_scales_and_out_of_range_entries(orc, tokens):
    """g = 0 with NULL scale buffers reads and writes no scale word; map entries >= n_src write a zero row
    like negative ones.  Short maps (row per wave) and long ones (XCD-aware kernel)."""
    k = 4096
    src_q, src_s, mp = wl.gather_case(k, tokens, 8, seed=90 + tokens)
    rng = np.random.default_rng(tokens)
    bad = rng.random(len(mp)) < 0.2
    mp = np.where(bad, tokens + rng.integers(0, 1 << 20, len(mp)), mp).astype(np.int32)
    mp[0] = 2 ** 31 - 1
    d = dev()
    dq = torch.full((len(mp), k), 0xAB, dtype=torch.uint8, device=d)
    sq = to_dev(src_q)
    st = m.lib().moe_gather_rows_scales(sq.data_ptr(), k, None, 0, tokens, k, 0, to_dev(mp).data_ptr(), len(mp),
                                        dq.data_ptr(), k, None, 0, m._stream())
    assert st == m.MOE_OK
    ds = torch.full((len(mp), src_s.shape[1]), -1, dtype=torch.int32, device=d)
    dq2 = torch.full((len(mp), k), 0xAB, dtype=torch.uint8, device=d)
    m.gather_rows_scales(sq, to_dev(src_s).view(torch.float32), to_dev(mp), dq2, ds.view(torch.float32))
    torch.cuda.synchronize()
    in_range = np.where(mp >= tokens, -1, mp).astype(np.int32)
    ref_q, ref_s = orc.gather_rows_scales(src_q, src_s.view(np.float32), in_range)
    assert np.array_equal(dq.cpu().numpy(), ref_q)
    assert np.array_equal(dq2.cpu().numpy(), ref_q)
    assert np.array_equal(ds.cpu().numpy(), ref_s.view(np.int32))


@pytest.mark.parametrize("case", ["ragged_strided_negative", "one_source", "identity"])
def test_gather_long_maps(orc, case):
    """Maps of 1024 rows and more: every copy of a source row is made on one XCD.  Ragged map
    lengths, negative entries, more than 64 scale words, padded destination rows, a map whose
    rows all name one source, and the identity map."""
    print("gather long map case=%s" % case, flush=True)
    rng = np.random.default_rng({"ragged_strided_negative": 11, "one_source": 12, "identity": 13}[case])
    if case == "ragged_strided_negative":
        k, n_src, n_dst, pad_q, pad_s = 16400, 300, 1027, 32, 3      # g = 129, 1025 vectors per row
        mp = rng.integers(-2, n_src, n_dst).astype(np.int32)
    elif case == "one_source":
        k, n_src, n_dst, pad_q, pad_s = 7168, 5, 2048, 0, 0
        mp = np.full(n_dst, 3, np.int32)
    else:
        k, n_src, n_dst, pad_q, pad_s = 4096, 1536, 1536, 0, 0
        mp = np.arange(n_dst, dtype=np.int32)
    g = (k + 127) // 128
    src_q = rng.integers(0, 256, (n_src, k), dtype=np.uint8)
    src_s = rng.integers(0, 2**32, (n_src, g), dtype=np.uint32).view(np.int32)
    dq = torch.full((n_dst, k + pad_q), 0xCD, dtype=torch.uint8, device=dev())
    ds = torch.full((n_dst, g + pad_s), 12345, dtype=torch.int32, device=dev())
    m.gather_rows_scales(to_dev(src_q), to_dev(src_s).view(torch.float32), to_dev(mp),
                         dq, ds.view(torch.float32), k=k, g=g)
    torch.cuda.synchronize()
    ref_q, ref_s = orc.gather_rows_scales(src_q, src_s.view(np.float32), mp)
    hq, hs = dq.cpu().numpy(), ds.cpu().numpy()
    assert np.array_equal(hq[:, :k], ref_q) and np.all(hq[:, k:] == 0xCD)
    assert np.array_equal(hs[:, :g], ref_s.view(np.int32)) and np.all(hs[:, g:] == 12345)


@pytest.mark.parametrize("k,tokens,topk", [(4096, 4096, 6), (896, 256, 8)])
def test_gather_prefill_size_route_map(orc, k, tokens, topk):
    """A route map of the prefill shape (every token once per routed expert, rows in expert order) at
    full size (24576 rows of 4096 bytes) and at the 896-byte width, both on the XCD-aware kernel."""
    print("gather route map k=%d tokens=%d top-%d" % (k, tokens, topk), flush=True)
    rng = np.random.default_rng(k + tokens)
    g = (k + 127) // 128
    src_q = rng.integers(0, 256, (tokens, k), dtype=np.uint8)
    src_s = rng.integers(0, 2**32, (tokens, g), dtype=np.uint32).view(np.int32)
    experts = np.stack([rng.choice(256, topk, replace=False) for _ in range(tokens)])   # [T, topk]
    order = np.lexsort((np.repeat(np.arange(tokens), topk), experts.ravel()))          # (expert, token)
    mp = np.repeat(np.arange(tokens, dtype=np.int32), topk)[order]
    dq = torch.empty((len(mp), k), dtype=torch.uint8, device=dev())
    ds = torch.empty((len(mp), g), dtype=torch.int32, device=dev())
    m.gather_rows_scales(to_dev(src_q), to_dev(src_s).view(torch.float32), to_dev(mp), dq, ds.view(torch.float32))
    torch.cuda.synchronize()
    ref_q, ref_s = orc.gather_rows_scales(src_q, src_s.view(np.float32), mp)
    assert np.array_equal(dq.cpu().numpy(), ref_q)
    assert np.array_equal(ds.cpu().numpy(), ref_s.view(np.int32))
    assert np.array_equal(dq.cpu().numpy(), src_q[mp])


def test_gather_unaligned_source_takes_byte_path(orc):
    k, tokens = 256, 6
    src_q, src_s, mp = wl.gather_case(k, tokens, 8, seed=78)
    big = torch.zeros(tokens * k + 1, dtype=torch.uint8, device=dev())
    big[1:] = to_dev(src_q).reshape(-1)
    src_view = big[1:].view(tokens, k)                       # 1-byte misaligned base
    dq = torch.empty((len(mp), k), dtype=torch.uint8, device=dev())
    ds = torch.empty((len(mp), 2), dtype=torch.float32, device=dev())
    m.gather_rows_scales(src_view, to_dev(src_s).view(torch.float32), to_dev(mp), dq, ds)
    torch.cuda.synchronize()
    assert np.array_equal(dq.cpu().numpy(), src_q[mp])


# --------------------------------------------------------------- act quant ---

def _ref_quant(orc, x_host):
    return orc.quant_groups(x_host)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("rows,n", [(1, 2048), (1, 4096), (7, 768), (3, 896), (5, 200), (2, 7), (64, 1024)])
def test_act_quant_identity_bit_exact(orc, dtype, rows, n):
    print("act_quant identity %s %dx%d" % (dtype, rows, n), flush=True)
    g = torch.Generator().manual_seed(rows * 10007 + n)
    x = (torch.randn((rows, n), generator=g) * torch.exp2(torch.randint(-8, 8, (rows, 1), generator=g).float()))
    x = x.to(dtype)
    if rows > 2:
        x[1] = 0
    host = x.view(torch.int16).numpy().view(np.uint16) if dtype == torch.bfloat16 else x.numpy()
    ref_q, ref_s = orc.quant_groups(host)
    gq = (n + 127) // 128
    q = torch.full((rows, n), 0x55, dtype=torch.uint8, device=dev())
    s = torch.full((rows, gq), float("nan"), dtype=torch.float32, device=dev())
    m.act_quant(x.to(dev()), q, s)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), ref_q)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))


def test_act_quant_identity_rounding_edges(orc):
    # rows whose values sit exactly on e4m3 rounding midpoints after scaling by s = 448/448 = 1
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    vals = orc.e4m3_decode(codes).astype(np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    row = np.zeros(128 * 2, np.float32)
    row[0] = 448.0
    row[1:1 + len(mids)] = mids
    row[128] = -448.0
    row[129:129 + len(mids)] = -mids
    x = np.stack([row, row * 0.75, row * 1e-3])
    ref_q, ref_s = orc.quant_groups(x)
    q = torch.empty((3, 256), dtype=torch.uint8, device=dev())
    s = torch.empty((3, 2), dtype=torch.float32, device=dev())
    m.act_quant(to_dev(x), q, s)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), ref_q)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))


def test_act_quant_identity_quotients_near_code_boundaries(orc):
    """Groups with arbitrary scales whose values divide to within a few ulp of an e4m3 rounding midpoint
    (and to midpoints exactly): the kernel's quotients (the division's steps without its range scaling)
    must give the codes of the correctly rounded division, bit for bit."""
    rng = np.random.default_rng(5)
    rows, n = 64, 1024
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    vals = orc.e4m3_decode(codes).astype(np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = np.empty((rows, n), np.float32)
    for r in range(rows):
        for g in range(n // 128):
            amax = np.float32(448.0 * 2.0 ** rng.uniform(-40, 40))
            s = np.float32(amax / np.float32(448.0))
            q = rng.choice(mids, 127).astype(np.float32)
            q = (q.view(np.int32) + rng.integers(-6, 7, 127).astype(np.int32)).view(np.float32)   # +- a few ulp
            v = (q * s).astype(np.float32) * rng.choice([-1.0, 1.0], 127).astype(np.float32)
            v = np.clip(v, -amax, amax)
            x[r, g * 128:(g + 1) * 128] = np.concatenate([[amax], v])
    ref_q, ref_s = orc.quant_groups(x)
    q = torch.empty((rows, n), dtype=torch.uint8, device=dev())
    s = torch.empty((rows, n // 128), dtype=torch.float32, device=dev())
    m.act_quant(to_dev(x), q, s)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), ref_q)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))


def test_act_quant_more_rows_than_one_grid_column(orc):
    """70000 rows: more than the 65535 rows one launch column covers, so rows are taken in strides."""
    rows, n = 70000, 128
    g = torch.Generator().manual_seed(11)
    x = torch.randn((rows, n), generator=g).to(torch.bfloat16)
    ref_q, ref_s = orc.quant_groups(x.view(torch.int16).numpy().view(np.uint16))
    q = torch.full((rows, n), 0x55, dtype=torch.uint8, device=dev())
    s = torch.full((rows, 1), float("nan"), dtype=torch.float32, device=dev())
    m.act_quant(x.to(dev()), q, s)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), ref_q)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,n", [(8, 768), (8, 1024), (37, 1024), (4, 200)])
def test_act_quant_silu_mul_within_one_step(orc, dtype, rows, n):
    g = torch.Generator().manual_seed(rows + n)
    c1 = (torch.randn((rows, 2 * n), generator=g) * 2).to(dtype)
    c1[0] = 0                                                       # an inactive route's zero tile
    host = c1.view(torch.int16).numpy().view(np.uint16) if dtype == torch.bfloat16 else c1.numpy()
    ref_q, ref_s = orc.silu_mul_quant(host)
    gq = (n + 127) // 128
    q = torch.empty((rows, n), dtype=torch.uint8, device=dev())
    s = torch.empty((rows, gq), dtype=torch.float32, device=dev())
    m.act_quant(c1.to(dev()), q, s, act=m.MOE_ACT_SILU_MUL)
    torch.cuda.synchronize()
    hq, hs = q.cpu().numpy(), s.cpu().numpy()
    assert np.all(hq[0] == 0) and np.all(hs[0].view(np.uint32) == 0)   # zero tile stays exactly zero
    assert np.allclose(hs, ref_s, rtol=1e-6, atol=0)
    # the device's sigmoid (hardware exp2 and reciprocal) is within a few ulp of libm's: codes differ by at
    # most one step, rarely
    dec = lambda c: orc.e4m3_decode(c).astype(np.float64)
    diff = hq != ref_q
    assert diff.mean() < 2e-3
    d = np.abs(dec(hq) - dec(ref_q))[diff]
    assert np.all(d <= np.abs(dec(ref_q))[diff] * 0.125 + 2.0 ** -9)


@pytest.mark.parametrize("act", [2, 3, 4, 5])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_act_quant_other_gated_activations(orc, act, dtype):
    """GEGLU, ReGLU, GLU and bilinear against the oracle on the same input: ReGLU and bilinear are exact
    fp32 products, so codes and scales match bit for bit; GEGLU and GLU go through the device erff/expf,
    so scales match to a few ulp and a code may move by one e4m3 step, rarely (GLU's sigmoid is the
    hardware exp2 and reciprocal)."""
    rows, n = 37, 640
    g = torch.Generator().manual_seed(rows + n + act)
    c1 = (torch.randn((rows, 2 * n), generator=g) * 2).to(dtype)
    c1[0] = 0                                                       # an inactive route's zero tile
    c1[1, :n] = -c1[1, :n].abs()                                     # non-positive gates: ReGLU zeros
    host = c1.view(torch.int16).numpy().view(np.uint16) if dtype == torch.bfloat16 else c1.numpy()
    ref_q, ref_s = orc.gated_act_quant(host, act)
    q = torch.empty((rows, n), dtype=torch.uint8, device=dev())
    s = torch.empty((rows, n // 128), dtype=torch.float32, device=dev())
    m.act_quant(c1.to(dev()), q, s, act=act)
    torch.cuda.synchronize()
    hq, hs = q.cpu().numpy(), s.cpu().numpy()
    assert np.all(hq[0] == 0) and np.all(hs[0].view(np.uint32) == 0)
    if act in (3, 5):
        assert np.array_equal(hq, ref_q) and np.array_equal(hs.view(np.uint32), ref_s.view(np.uint32))
        return
    assert np.allclose(hs, ref_s, rtol=4e-7, atol=0)
    dec = lambda c: orc.e4m3_decode(c).astype(np.float64)
    diff = hq != ref_q
    assert diff.mean() < 2e-3
    d = np.abs(dec(hq) - dec(ref_q))[diff]
    assert np.all(d <= np.abs(dec(ref_q))[diff] * 0.125 + 2.0 ** -9)


# ------------------------------------------------------------------ reduce ---

def assert_reduce_bound(got, ref, y, slots, w, rr):
    """Both sides sum the active routes in ascending order in fp32 (the device may fuse each multiply-add),
    so each fp32 sum is within (topk + 1) * 2^-24 * sum|w*y| of the exact one; one bf16 rounding each adds
    half a bf16 ulp of the result."""
    from gpu_util import bf16_bits_to_f64
    T, topk = slots.shape
    rows = np.arange(T * topk).reshape(T, topk) if rr is None else rr
    act = (slots >= 0).astype(np.float64)
    wa = np.where(slots >= 0, np.nan_to_num(w.astype(np.float64)), 0.0)
    S = np.einsum("tj,tjh->th", np.abs(wa) * act, np.abs(y.astype(np.float64)[rows]))
    g, r = bf16_bits_to_f64(got), bf16_bits_to_f64(ref)
    mag = np.maximum(np.abs(g), np.abs(r))
    ulp = np.where(mag > 0, 2.0 ** (np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 7), 2.0 ** -133)
    bound = 2 * (topk + 1) * 2.0 ** -24 * S + ulp
    assert np.all(np.abs(g - r) <= bound), "reduce beyond its fp32 + bf16 rounding bound"


@pytest.mark.parametrize("ydt", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("H,topk", [(2048, 8), (100, 6), (4096, 6), (24, 11)])
def test_topk_reduce(orc, ydt, H, topk):
    """8-column vector path (H % 8 == 0) and the 4-column path (H = 100); topk above one 8-route pass."""
    print("topk_reduce %s H=%d topk=%d" % (ydt, H, topk), flush=True)
    rng = np.random.default_rng(5 + H + topk)
    T = 6
    y = torch.from_numpy(rng.standard_normal((T * topk, H)).astype(np.float32)).to(ydt)
    slots = rng.integers(0, 64, size=(T, topk)).astype(np.int32)
    slots[1, [0, 3, 5]] = -1
    slots[2, :] = -1
    slots[3, topk - 1] = -1
    w = rng.random((T, topk)).astype(np.float32)
    w[slots < 0] = np.nan                                     # never read
    perm = rng.permutation(T * topk).astype(np.int32).reshape(T, topk)
    host_y = y.view(torch.int16).numpy().view(np.uint16) if ydt == torch.bfloat16 else y.numpy()
    if ydt == torch.float16:
        host_y = y.numpy()
    for rr in (None, perm):
        ref = orc.topk_reduce(host_y, slots, w, route_rows=rr)
        out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=dev())
        m.topk_reduce(y.to(dev()), to_dev(slots), to_dev(w), out, route_rows=None if rr is None else to_dev(rr))
        torch.cuda.synchronize()
        got = u16(out)
        assert np.all(got[2] == 0)
        assert_bf16_close(got, ref, what="topk_reduce")
        assert_reduce_bound(got, ref, y.float().numpy(), slots, w, rr)


def test_topk_reduce_strided_rows_take_the_4_column_path(orc):
    """y rows with a stride that breaks 16-byte alignment of every row: the 4-column path, same results."""
    rng = np.random.default_rng(11)
    T, topk, H = 5, 6, 64
    ypad = torch.from_numpy(rng.standard_normal((T * topk, H + 4)).astype(np.float32)).to(torch.bfloat16)
    y = ypad[:, :H]
    slots = rng.integers(0, 8, size=(T, topk)).astype(np.int32)
    w = rng.random((T, topk)).astype(np.float32)
    ref = orc.topk_reduce(np.ascontiguousarray(y.view(torch.int16).numpy()).view(np.uint16), slots, w)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev())
    m.topk_reduce(ypad.to(dev())[:, :H], to_dev(slots), to_dev(w), out)
    torch.cuda.synchronize()
    got = u16(out)
    assert_reduce_bound(got, ref, y.float().numpy(), slots, w, None)
