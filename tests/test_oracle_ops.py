"""Pins of the oracle's operations (quantize, gather, block GEMM, activation, reduce, fused decode).

Each test checks the oracle against something fixed outside it: numpy
indexing and matmul in float64, torch's fp8/bf16 casts, exact integer
arithmetic, closed-form invariants and the behaviour the pages state.
"""
import json
import os

import numpy as np
import pytest
import torch

import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def t_dec(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float32).numpy()


def t_enc(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    return x.contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- O1 -------

@pytest.mark.parametrize("n", [128, 256, 768, 896, 200, 7])
def test_quant_groups_against_numpy_division_and_torch_cast(orc, n):
    rng = np.random.default_rng(n)
    x = (rng.standard_normal((9, n)) * np.exp2(rng.integers(-6, 6, size=(9, 1)))).astype(np.float32)
    x[3, :] = 0.0                                   # an all-zero row: s = 0, q = 0
    x[4, :min(n, 128)] = -0.0
    q, s = orc.quant_groups(x)
    g = (n + 127) // 128
    for r in range(9):
        for gi in range(g):
            seg = x[r, gi * 128:(gi + 1) * 128]
            amax = np.max(np.abs(seg))
            s_want = np.float32(amax) / np.float32(448.0)  # numpy: one correctly rounded division
            assert s[r, gi].view(np.uint32) == np.float32(s_want).view(np.uint32)
            if s_want == 0:
                assert np.all(q[r, gi * 128:(gi + 1) * 128] == 0)
            else:
                want = t_enc(seg / np.float32(s_want))
                assert np.array_equal(q[r, gi * 128:(gi + 1) * 128], want)
                # the element achieving amax lands exactly on the top code, +-448
                assert np.max(np.abs(t_dec(q[r, gi * 128:(gi + 1) * 128]))) == 448.0


def test_quant_groups_bf16_input_is_exact_widening(orc):
    x = wl.bf16_normal((5, 384), seed=1)
    q1, s1 = orc.quant_groups(bf16_bits(x))
    q2, s2 = orc.quant_groups(x.to(torch.float32).numpy())
    assert np.array_equal(q1, q2) and np.array_equal(s1.view(np.uint32), s2.view(np.uint32))


def test_quant_groups_dequant_error_within_half_step(orc):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((64, 1024)).astype(np.float32)
    q, s = orc.quant_groups(x)
    deq = t_dec(q).astype(np.float64) * np.repeat(s, 128, axis=1).astype(np.float64)
    # e4m3 has 3 mantissa bits: relative half-step 2^-4 for normals, absolute 2^-10 * s below 2^-6
    err = np.abs(deq - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * np.repeat(s, 128, axis=1)) * (1 + 1e-6)
    assert np.all(err <= bound)


# ---------------------------------------------------------------- O2 -------

@pytest.mark.parametrize("k,tokens", [(7168, 1), (2048, 1), (7168, 8), (896, 16), (896, 1), (100, 5)])
def test_gather_matches_numpy_indexing_and_two_pass(orc, k, tokens):
    src_q, src_s, m = wl.gather_case(k, tokens, 8, seed=k + tokens)
    dq, ds = orc.gather_rows_scales(src_q, src_s.view(np.float32), m)
    # the page's plain-indexing oracle, on integer views (random bytes are often NaN)
    assert np.array_equal(dq, src_q[m])
    assert np.array_equal(ds.view(np.int32), src_s[m])
    # two-pass form: rows with g = 0, then scales with k = 0
    dq2, _ = orc.gather_rows_scales(src_q, src_s.view(np.float32), m, g=0)
    _, ds2 = orc.gather_rows_scales(src_q, src_s.view(np.float32), m, k=0)
    assert np.array_equal(dq2, dq) and np.array_equal(ds2.view(np.int32), ds.view(np.int32))


def test_gather_shapes_from_page(orc):
    spec = json.load(open(os.path.join(GOLD, "gather_scale_groups.json")))
    for c in spec["cases"]:
        assert (c["k"] + 127) // 128 == c["groups"] == c["k"] // 128 or c["k"] % 128 == 0
        assert c["rows"] == 8 * c["tokens"]
        assert 4 * c["groups"] / c["k"] == spec["scale_bytes_over_row_bytes"]
    src_q, src_s, m = wl.gather_case(896, 16, 8, seed=3)
    assert src_s.shape[1] == 7
    assert len(np.unique(m)) < len(m)                 # randint maps repeat sources


def test_gather_empty_and_negative_entries(orc):
    src_q, src_s, _ = wl.gather_case(256, 4, 8, seed=4)
    dq, ds = orc.gather_rows_scales(src_q, src_s.view(np.float32), np.zeros(0, np.int32))
    assert dq.shape == (0, 256) and ds.shape == (0, 2)
    m = np.array([2, -1, 0, -5], np.int32)
    dq, ds = orc.gather_rows_scales(src_q, src_s.view(np.float32), m)
    assert np.all(dq[[1, 3]] == 0) and np.all(ds[[1, 3]].view(np.uint32) == 0)
    assert np.array_equal(dq[[0, 2]], src_q[[2, 0]])


# ---------------------------------------------------------------- O3 -------

def brute_gemm(a_q, a_s, w_q, w_s, experts_of_rows, a_rows):
    """float64 reference: dequantize both operands with torch's fp8 decode and multiply."""
    R = len(experts_of_rows)
    E, N, K = w_q.shape
    out = np.zeros((R, N))
    A = t_dec(a_q).astype(np.float64) * np.repeat(a_s, 128, axis=1)[:, :K]
    for r in range(R):
        e = experts_of_rows[r]
        if e < 0:
            continue
        W = t_dec(w_q[e]).astype(np.float64) * np.repeat(np.repeat(w_s[e], 128, axis=0), 128, axis=1)[:N, :K]
        out[r] = W @ A[a_rows[r]]
    return out


def error_bound(a_q, a_s, w_q, w_s, experts_of_rows, a_rows):
    """|fp32 result - exact| <= (K/128 + 130) * 2^-24 * sum|terms| (one rounding per add/mul)."""
    E, N, K = w_q.shape
    A = np.abs(t_dec(a_q).astype(np.float64)) * np.repeat(a_s, 128, axis=1)[:, :K]
    out = np.zeros((len(experts_of_rows), N))
    for r, e in enumerate(experts_of_rows):
        if e < 0:
            continue
        W = np.abs(t_dec(w_q[e]).astype(np.float64)) * np.repeat(np.repeat(w_s[e], 128, axis=0), 128, axis=1)[:N, :K]
        out[r] = W @ A[a_rows[r]]
    return out * (K / 128 + 130) * 2.0 ** -24


def test_block_gemm_slot_mode_vs_float64_brute_force(orc):
    E, N, K, T, topk = 5, 384, 640, 3, 4
    w_q, w_s = wl.block_fp8_weights(E, N, K, seed=21)
    w_q, w_s = w_q.numpy(), w_s.numpy()
    a_q, a_s = wl.fp8_rows(T, K, seed=22)
    a_q, a_s = a_q.numpy(), a_s.numpy()
    slots = np.array([[0, 4, -1, 2], [3, -1, -1, 1], [4, 4, 0, -1]], np.int32).reshape(-1)
    out = orc.block_gemm(a_q, a_s, w_q, w_s, mode=orc.MODE_SLOT, slot_ids=slots, a_row_div=topk)
    ref = brute_gemm(a_q, a_s, w_q, w_s, slots, np.arange(T * topk) // topk)
    bound = error_bound(a_q, a_s, w_q, w_s, slots, np.arange(T * topk) // topk)
    assert np.all(np.abs(out - ref) <= bound)
    inactive = slots < 0
    assert np.all(out[inactive].view(np.uint32) == 0)          # +0.0 rows
    assert np.abs(out[~inactive]).max() > 0


def test_block_gemm_integer_special_case_is_exact(orc):
    # values -4..4 with power-of-two scales: every step is exact in fp32
    E, N, K, rows = 3, 256, 512, 10
    a_q, a_s, w_q, w_s = wl.powers_of_two_case(E, N, K, rows, seed=5)
    offs = np.array([0, 4, 4, 10], np.int32)  # expert 1 is empty
    out = orc.block_gemm(a_q, a_s, w_q, w_s, mode=orc.MODE_GROUPED, expert_offsets=offs)
    ia = t_dec(a_q).astype(np.int64)
    iw = t_dec(w_q).astype(np.int64)
    ref = np.zeros((rows, N))
    for e in range(E):
        for r in range(offs[e], offs[e + 1]):
            for kb in range(K // 128):
                part = iw[e][:, kb * 128:(kb + 1) * 128] @ ia[r, kb * 128:(kb + 1) * 128]
                ref[r] += part * a_s[r, kb] * np.repeat(w_s[e][:, kb], 128)[:N]
    assert np.array_equal(out.astype(np.float64), ref)


def test_block_gemm_grouped_equals_slot_with_same_experts(orc):
    E, N, K = 4, 256, 384
    w_q, w_s = wl.block_fp8_weights(E, N, K, seed=31)
    w_q, w_s = w_q.numpy(), w_s.numpy()
    a_q, a_s = wl.fp8_rows(11, K, seed=32)
    a_q, a_s = a_q.numpy(), a_s.numpy()
    offs = np.array([0, 3, 3, 9, 11], np.int32)
    grouped = orc.block_gemm(a_q, a_s, w_q, w_s, mode=orc.MODE_GROUPED, expert_offsets=offs)
    experts = np.repeat(np.arange(E), np.diff(offs)).astype(np.int32)
    slot = orc.block_gemm(a_q, a_s, w_q, w_s, mode=orc.MODE_SLOT, slot_ids=experts, a_row_div=1)
    assert np.array_equal(grouped.view(np.uint32), slot.view(np.uint32))
    ref = brute_gemm(a_q, a_s, w_q, w_s, experts, np.arange(11))
    assert np.all(np.abs(grouped - ref) <= error_bound(a_q, a_s, w_q, w_s, experts, np.arange(11)))


@pytest.mark.parametrize("dt", [np.uint16, np.float16])
def test_block_gemm_narrow_outputs_are_rounded_fp32(orc, dt):
    E, N, K = 2, 128, 256
    w_q, w_s = wl.block_fp8_weights(E, N, K, seed=41)
    a_q, a_s = wl.fp8_rows(4, K, seed=42)
    args = (a_q.numpy(), a_s.numpy(), w_q.numpy(), w_s.numpy())
    slots = np.array([1, 0, -1, 1], np.int32)
    f32 = orc.block_gemm(*args, mode=orc.MODE_SLOT, slot_ids=slots)
    nar = orc.block_gemm(*args, mode=orc.MODE_SLOT, slot_ids=slots, out_dtype=dt)
    if dt == np.uint16:
        want = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    else:
        want = f32.astype(np.float16)
    assert np.array_equal(nar.view(np.uint16), want.view(np.uint16))


# ---------------------------------------------------------------- O4 -------

def test_silu_mul_quant_vs_float64(orc):
    rng = np.random.default_rng(51)
    rows, n = 16, 768
    c1 = (rng.standard_normal((rows, 2 * n)) * 3).astype(np.float32)
    q, s = orc.silu_mul_quant(c1)
    g64, u64 = c1[:, :n].astype(np.float64), c1[:, n:].astype(np.float64)
    h64 = g64 / (1 + np.exp(-g64)) * u64
    deq = t_dec(q).astype(np.float64) * np.repeat(s, 128, axis=1)
    sc = np.repeat(s, 128, axis=1).astype(np.float64)
    bound = np.maximum(np.abs(h64) * 2.0 ** -4, 2.0 ** -10 * sc) * (1 + 1e-4) + 1e-6 * sc
    assert np.all(np.abs(deq - h64) <= bound)
    # quantizing the float64 h with torch's cast flips few codes (only near rounding midpoints)
    s64 = (np.abs(h64).reshape(rows, -1, 128).max(axis=2) / 448.0).astype(np.float32)
    want = t_enc((h64 / np.repeat(s64, 128, axis=1)).astype(np.float32))
    assert np.mean(want != q) < 1e-3
    # gate and up are not swapped: silu(u)*g differs from silu(g)*u
    h_sw = u64 / (1 + np.exp(-u64)) * g64
    assert np.abs(deq - h_sw).max() > 10 * np.abs(deq - h64).max()


def test_silu_mul_quant_of_zero_tile_is_zero(orc):
    c1 = np.zeros((3, 512), np.float32)
    q, s = orc.silu_mul_quant(c1)
    assert np.all(q == 0) and np.all(s.view(np.uint32) == 0)


def _act64(act, g, u):
    """The five GLU variants in float64 from independent library routines."""
    from scipy.special import erf, expit
    if act == 1:
        return g * expit(g) * u                          # Swish_1(g) * u
    if act == 2:
        return g * 0.5 * (1.0 + erf(g / np.sqrt(2.0))) * u   # GELU(g) * u, GELU = x Phi(x)
    if act == 3:
        return np.maximum(g, 0.0) * u
    if act == 4:
        return expit(g) * u
    return g * u


@pytest.mark.parametrize("act", [1, 2, 3, 4, 5])
def test_gated_act_quant_vs_float64(orc, act):
    """Each gated activation against its float64 definition: every dequantized value within half an e4m3
    step of the float64 h, codes equal to torch's cast of the float64 h except near rounding midpoints,
    and gate/up not swapped."""
    rng = np.random.default_rng(70 + act)
    rows, n = 12, 512
    c1 = (rng.standard_normal((rows, 2 * n)) * 3).astype(np.float32)
    q, s = orc.gated_act_quant(c1, act)
    g64, u64 = c1[:, :n].astype(np.float64), c1[:, n:].astype(np.float64)
    h64 = _act64(act, g64, u64)
    sc = np.repeat(s, 128, axis=1).astype(np.float64)
    deq = t_dec(q).astype(np.float64) * sc
    bound = np.maximum(np.abs(h64) * 2.0 ** -4, 2.0 ** -10 * sc) * (1 + 1e-4) + 1e-6 * sc
    assert np.all(np.abs(deq - h64) <= bound)
    s64 = (np.abs(h64).reshape(rows, -1, 128).max(axis=2) / 448.0).astype(np.float32)
    want = t_enc((h64 / np.repeat(s64, 128, axis=1)).astype(np.float32))
    assert np.mean(want != q) < 1e-3
    if act != 5:                                 # g * u is symmetric in gate and up
        h_sw = _act64(act, u64, g64)
        assert np.abs(deq - h_sw).max() > 10 * np.abs(deq - h64).max()
    z = orc.gated_act_quant(np.zeros((2, 256), np.float32), act)
    assert np.all(z[0] == 0) and np.all(z[1].view(np.uint32) == 0)


@pytest.mark.parametrize("act", [3, 5])
def test_relu_and_bilinear_are_exact_products(orc, act):
    """ReGLU and bilinear form h with one exact-rounded fp32 product, so the codes and scales equal O1's
    definition applied to numpy's fp32 product bit for bit (a non-positive gate gives +0, and +0 times a
    negative up is -0, code 0x80)."""
    rng = np.random.default_rng(80 + act)
    rows, n = 6, 384
    c1 = (rng.standard_normal((rows, 2 * n)) * 2).astype(np.float32)
    c1[0, :n] = -np.abs(c1[0, :n])              # row 0: every gate <= 0 ...
    c1[0, 5] = 1.5                               # ... but one
    q, s = orc.gated_act_quant(c1, act)
    g, u = c1[:, :n], c1[:, n:]
    h = (np.where(g > 0, g, np.float32(0)) * u if act == 3 else g * u).astype(np.float32)
    s_want = (np.abs(h).reshape(rows, -1, 128).max(axis=2) / np.float32(448)).astype(np.float32)
    assert np.array_equal(s.view(np.uint32), s_want.view(np.uint32))
    with np.errstate(invalid="ignore", divide="ignore"):
        v = h / np.repeat(s_want, 128, axis=1)
    v = np.where(np.repeat(s_want, 128, axis=1) == 0, 0, v).astype(np.float32)
    assert np.array_equal(q, t_enc(v))
    if act == 3:
        # group 0 of row 0 holds the one positive gate, so its scale is nonzero and the zeros keep their
        # sign; groups 1 and 2 are all zero (s = 0) and give 0x00 codes whatever the sign
        c = np.arange(128)
        neg_u = (u[0, :128] < 0) & (c != 5)
        assert np.all(q[0, :128][neg_u] == 0x80) and np.all(q[0, :128][~neg_u & (c != 5)] == 0x00)
        assert np.all(q[0, 128:] == 0) and np.all(s[0, 1:] == 0)


def test_gelu_gate_closed_form(orc):
    """GELU(x) - GELU(-x) = x: with up = 1, the GEGLU rows of x and -x dequantize to values whose
    difference is x within the two rows' half steps."""
    x = np.linspace(-6, 6, 256).astype(np.float32)
    c1 = np.stack([np.concatenate([x, np.ones_like(x)]), np.concatenate([-x, np.ones_like(x)])])
    q, s = orc.gated_act_quant(c1, 2)
    d = t_dec(q).astype(np.float64) * np.repeat(s, 128, axis=1)
    step = np.maximum(np.abs(d) * 2.0 ** -4, 2.0 ** -10 * np.repeat(s, 128, axis=1))
    assert np.all(np.abs((d[0] - d[1]) - x) <= step[0] + step[1] + 1e-6)


# ---------------------------------------------------------------- O5 -------

def test_topk_reduce_one_hot_all_inactive_and_float64(orc):
    rng = np.random.default_rng(61)
    T, topk, H = 4, 8, 256
    y = rng.standard_normal((T * topk, H)).astype(np.float32)
    slots = rng.integers(0, 64, size=(T, topk)).astype(np.int32)
    slots[1, [0, 3, 5]] = -1
    slots[2, :] = -1
    w = rng.random((T, topk)).astype(np.float32)
    w[slots < 0] = np.nan                              # never read
    w[3, :] = 0.0
    w[3, 6] = 1.0                                      # one-hot
    out = orc.topk_reduce(y, slots, w)
    assert np.all(out[2] == 0)                          # no active route -> +0.0
    want3 = torch.from_numpy(y[3 * topk + 6]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out[3], want3)
    for t in (0, 1):
        act = slots[t] >= 0
        ref = (w[t, act].astype(np.float64)[:, None] * y[t * topk:(t + 1) * topk][act]).sum(0)
        got = bits_to_f32(out[t]).astype(np.float64)
        assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6)


def test_topk_reduce_route_rows_indirection(orc):
    rng = np.random.default_rng(62)
    T, topk, H = 5, 3, 128
    perm = rng.permutation(T * topk).astype(np.int32)
    y = rng.standard_normal((T * topk, H)).astype(np.float32)
    slots = np.zeros((T, topk), np.int32)
    w = rng.random((T, topk)).astype(np.float32)
    direct = orc.topk_reduce(y[perm], slots, w)
    via = orc.topk_reduce(y, slots, w, route_rows=perm.reshape(T, topk))
    assert np.array_equal(direct, via)


# ---------------------------------------------------------------- O6 -------

def _case(H=256, I=128, topk=2, n_slots=8, active=1, seed=0, T=1, tail=False):
    c = wl.decode_case(H, I, topk, n_slots, active, seed, T=T, tail=tail)
    return c, (bf16_bits(c.x), c.slot_ids, c.weights, c.w13_q.numpy(), c.w13_s.numpy(),
               c.w2_q.numpy(), c.w2_s.numpy())


@pytest.mark.parametrize("act", [1, 2, 3, 4, 5])
def test_fused_decode_vs_float64_layer(orc, act):
    """Whole layer in float64 from dequantized operands, for each gated activation; only the two
    quantization points (x and the activation) are kept, done with numpy division and torch's fp8
    cast."""
    c, args = _case(H=512, I=256, topk=4, n_slots=6, active=3, seed=3, T=2)
    out = orc.fused_decode(*args, act=act)
    x = c.x.to(torch.float32).numpy()
    xs = (np.abs(x).reshape(c.T, -1, 128).max(2) / np.float32(448)).astype(np.float32)
    xq = t_enc(x / np.repeat(xs, 128, axis=1))
    X = t_dec(xq).astype(np.float64) * np.repeat(xs, 128, axis=1)
    W13 = t_dec(args[3]).astype(np.float64) * np.repeat(np.repeat(args[4], 128, 1), 128, 2)
    W2 = t_dec(args[5]).astype(np.float64) * np.repeat(np.repeat(args[6], 128, 1), 128, 2)
    ref = np.zeros((c.T, c.H))
    for t in range(c.T):
        for j in range(c.topk):
            sl = c.slot_ids[t, j]
            if sl < 0:
                continue
            h = W13[sl] @ X[t]
            g, u = h[:c.I], h[c.I:]
            a = _act64(act, g, u)
            a_s = (np.abs(a).reshape(-1, 128).max(1) / 448.0).astype(np.float32)
            aq = t_enc((a / np.repeat(a_s, 128)).astype(np.float32))
            A = t_dec(aq).astype(np.float64) * np.repeat(a_s, 128)
            ref[t] += c.weights[t, j] * (W2[sl] @ A)
    got = bits_to_f32(out).astype(np.float64)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel < 1e-2, rel


def test_fused_decode_negative_slots_equal_clamped_zero_weight_path(orc):
    """-1 routes give exactly the output of the old path: slot 0 with routing weight 0."""
    for active, seed in ((1, 0), (4, 1), (0, 2), (8, 3)):
        c, args = _case(H=256, I=128, topk=8, n_slots=8, active=active, seed=seed, T=2)
        out_new = orc.fused_decode(*args)
        clamped = np.where(c.slot_ids < 0, 0, c.slot_ids).astype(np.int32)
        w_old = np.where(c.slot_ids < 0, 0.0, c.weights).astype(np.float32)
        out_old = orc.fused_decode(args[0], clamped, w_old, *args[3:])
        assert np.array_equal(out_new, out_old)


def test_fused_decode_all_inactive_is_exact_zero(orc):
    c, args = _case(H=256, I=128, topk=2, n_slots=8, active=0, seed=5)
    w = args[2].copy()
    w[:] = np.nan                                   # routing weights are never read
    out, im = orc.fused_decode(args[0], args[1], w, *args[3:], intermediates=True)
    assert np.all(out == 0)
    for key in ("c1", "aq", "as_", "c2"):
        assert np.all(im[key].view(np.uint8) == 0), key


def test_fused_decode_route_permutation_invariance(orc):
    c, args = _case(H=256, I=128, topk=8, n_slots=16, active=6, seed=7)
    out = orc.fused_decode(*args)
    perm = np.random.default_rng(0).permutation(8)
    out_p = orc.fused_decode(args[0], args[1][:, perm].copy(), args[2][:, perm].copy(), *args[3:])
    a, b = bits_to_f32(out), bits_to_f32(out_p)
    ulp = np.abs(a) * 2.0 ** -7 + 1e-30
    assert np.all(np.abs(a - b) <= ulp)


def test_fused_decode_tiny_config(orc):
    """1 token, H=256, I=128, 8 slots, top-2 with one slot -1: the active route alone decides."""
    c, args = _case(H=256, I=128, topk=2, n_slots=8, active=1, seed=0)
    out, im = orc.fused_decode(*args, intermediates=True)
    j = int(np.nonzero(c.slot_ids[0] >= 0)[0][0])
    only = np.full_like(c.slot_ids, -1)
    only[0, j] = c.slot_ids[0, j]
    out_only = orc.fused_decode(args[0], only, args[2], *args[3:])
    assert np.array_equal(out, out_only)
    assert np.all(im["c1"][1 - j] == 0) and np.abs(im["c1"][j]).max() > 0


# ---- O7: routing prep -------------------------------------------------------------------------

def _routing_logits(T, E, seed):
    return np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32)


@pytest.mark.parametrize("T,E,topk", [(1, 8, 2), (37, 16, 4), (300, 256, 6), (64, 64, 64), (5, 1, 1)])
def test_route_prep_selection_and_maps_vs_numpy_sort(orc, T, E, topk):
    """Top-k equals numpy's stable argsort of -logits (ties to the lower index); the route maps equal a
    stable numpy sort of the (expert, token) keys, and the offsets a bincount prefix sum."""
    lg = _routing_logits(T, E, seed=T * 7 + E)
    r = orc.route_prep(lg, topk)
    want_ids = np.argsort(-lg, axis=1, kind="stable")[:, :topk].astype(np.int32)
    assert np.array_equal(r["expert_ids"], want_ids)
    keys = (want_ids.astype(np.int64) * T + np.arange(T)[:, None]).ravel()
    order = np.argsort(keys, kind="stable")
    assert np.array_equal(r["dst2src"], (order // topk).astype(np.int32))
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    assert np.array_equal(r["route_rows"], inv.astype(np.int32))
    offs = np.concatenate([[0], np.cumsum(np.bincount(want_ids.ravel(), minlength=E))]).astype(np.int32)
    assert np.array_equal(r["expert_offsets"], offs)


def test_route_prep_weights_vs_scipy_softmax_and_closed_form(orc):
    from scipy.special import softmax
    lg = _routing_logits(200, 64, seed=5)
    r = orc.route_prep(lg, 6)
    p = softmax(lg.astype(np.float64), axis=1)
    sel = np.take_along_axis(p, r["expert_ids"].astype(np.int64), axis=1)
    want = sel / sel.sum(axis=1, keepdims=True)
    assert np.allclose(r["weights"], want, rtol=2e-7, atol=0)
    # closed form: the ratio of two routes' weights is exp of their logit difference; weights sum to 1
    l_sel = np.take_along_axis(lg.astype(np.float64), r["expert_ids"].astype(np.int64), axis=1)
    ratio = r["weights"][:, 1:].astype(np.float64) / r["weights"][:, :1]
    assert np.allclose(ratio, np.exp(l_sel[:, 1:] - l_sel[:, :1]), rtol=1e-6)
    assert np.allclose(r["weights"].sum(axis=1, dtype=np.float64), 1.0, rtol=1e-6)


def test_route_prep_ties_all_experts_and_empty(orc):
    # all-equal logits: experts 0..topk-1, each weight exactly 1/topk
    r = orc.route_prep(np.zeros((3, 10), np.float32), 4)
    assert np.array_equal(r["expert_ids"], np.tile(np.arange(4, dtype=np.int32), (3, 1)))
    assert np.all(r["weights"] == np.float32(0.25))
    # +0 and -0 tie as well: the lower index wins
    lg = np.array([[-0.0, 0.0, -1.0]], np.float32)
    assert r is not None and orc.route_prep(lg, 2)["expert_ids"].tolist() == [[0, 1]]
    # topk == E: every expert, weights = plain softmax
    lg = _routing_logits(4, 5, seed=1)
    r = orc.route_prep(lg, 5)
    assert np.array_equal(np.sort(r["expert_ids"], axis=1), np.tile(np.arange(5), (4, 1)))
    # no tokens: empty maps, all offsets zero
    r = orc.route_prep(np.zeros((0, 8), np.float32), 2)
    assert r["dst2src"].size == 0 and np.all(r["expert_offsets"] == 0)


def test_route_prep_matches_the_workload_generator(orc):
    """workloads.routing draws N(0,1) logits with torch in float64 and routes them in numpy (softmax,
    stable top-k, renormalization); the oracle on the same logits in fp32 picks the same experts and
    weights within fp32 rounding."""
    import torch
    T, E, topk, seed = 256, 64, 6, 11
    ids, w = wl.routing(T, E, topk, seed)
    lg = torch.randn((T, E), generator=wl._gen(seed), dtype=torch.float64).numpy()
    r = orc.route_prep(lg.astype(np.float32), topk)
    assert np.array_equal(r["expert_ids"], ids)
    assert np.allclose(r["weights"], w, rtol=1e-6, atol=0)
