"""Pins of the oracle's MXFP4 weight path (O8): the E2M1 and E8M0 decoders against their closed forms and
torch, and the GEMM against float64 brute force and against the block-FP8 GEMM (O3) on weights that both
formats hold exactly."""
import numpy as np
import pytest
import torch

import workloads as wl


def e2m1_closed_form(c):
    """OCP MX element FP4 E2M1: (-1)^s * (e == 0 ? 0.5 m : 2^(e-1) (1 + m/2))."""
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    v = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
    return -v if s else v


def unpack_e2m1(w4):
    """[..., K/2] bytes -> [..., K] codes, element 2i in the low nibble."""
    lo, hi = w4 & 15, w4 >> 4
    return np.stack([lo, hi], axis=-1).reshape(*w4.shape[:-1], 2 * w4.shape[-1])


def test_e2m1_decode_matches_the_element_definition(orc):
    got = orc.e2m1_decode(np.arange(16, dtype=np.uint8))
    want = np.array([e2m1_closed_form(c) for c in range(16)], np.float32)
    assert np.array_equal(got, want)
    assert sorted(set(np.abs(got).tolist())) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.signbit(got[8]) and got[8] == 0.0          # code 0b1000 is -0


def test_e8m0_decode_matches_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    got = orc.e8m0_decode(codes)
    want = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float32).numpy()
    assert np.isnan(got[255]) and np.isnan(want[255])
    assert np.array_equal(got[:255], want[:255])


def dense_mx(w4, w4_s):
    codes = unpack_e2m1(w4)
    vals = np.vectorize(e2m1_closed_form)(codes).astype(np.float64)
    return vals * np.repeat(np.ldexp(1.0, w4_s.astype(np.int64) - 127), 32, axis=-1)


def test_mxfp4_gemm_vs_float64_brute_force(orc):
    E, N, K = 3, 48, 384
    counts = [5, 0, 11]
    w4, w4_s = (t.numpy() for t in wl.mxfp4_weights(E, N, K, seed=1))
    a_q, a_s = (t.numpy() for t in wl.fp8_rows(sum(counts), K, seed=2))
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    got = orc.mxfp4_gemm(a_q, a_s, w4, w4_s, mode=orc.MODE_GROUPED, expert_offsets=offs).astype(np.float64)
    A = torch.from_numpy(a_q).view(torch.float8_e4m3fn).double().numpy() * np.repeat(a_s, 128, axis=1)
    W = dense_mx(w4, w4_s)
    for e in range(E):
        rows = slice(offs[e], offs[e + 1])
        exact = A[rows] @ W[e].T
        terms = np.abs(A[rows]) @ np.abs(W[e]).T
        bound = (K + 4 * K / 128 + 4) * 2.0 ** -23 * terms
        assert np.all(np.abs(got[rows] - exact) <= bound)


def test_mxfp4_gemm_equals_fp8_gemm_on_shared_values(orc):
    """Weights 2^(e-127) * E2M1 with e in [120, 127] are exact e4m3 values; an fp8 bank of those values with
    unit block scales gives the same products in the same order, so O8 and the pinned O3 agree bit for bit."""
    E, N, K = 2, 32, 256
    w4, w4_s = (t.numpy() for t in wl.mxfp4_weights(E, N, K, seed=3, e_lo=120, e_hi=127))
    W = dense_mx(w4, w4_s).astype(np.float32)
    w8 = torch.from_numpy(W).to(torch.float8_e4m3fn)
    assert np.array_equal(w8.float().numpy(), W)                   # exactly representable
    w8 = w8.view(torch.uint8).numpy()
    w8_s = np.ones((E, (N + 127) // 128, K // 128), np.float32)
    a_q, a_s = (t.numpy() for t in wl.fp8_rows(9, K, seed=4))
    offs = np.array([0, 4, 9], np.int32)
    mx = orc.mxfp4_gemm(a_q, a_s, w4, w4_s, mode=orc.MODE_GROUPED, expert_offsets=offs)
    f8 = orc.block_gemm(a_q, a_s, w8, w8_s, mode=orc.MODE_GROUPED, expert_offsets=offs)
    assert np.array_equal(mx.view(np.uint32), f8.view(np.uint32))


def test_mxfp4_slot_mode_inactive_rows_and_grouped_equivalence(orc):
    E, N, K = 4, 32, 128
    w4, w4_s = (t.numpy() for t in wl.mxfp4_weights(E, N, K, seed=5))
    a_q, a_s = (t.numpy() for t in wl.fp8_rows(6, K, seed=6))
    slots = np.array([2, -1, 0, 3, -1, 1], np.int32)
    out = orc.mxfp4_gemm(a_q, a_s, w4, w4_s, mode=orc.MODE_SLOT, slot_ids=slots)
    assert np.all(out[slots < 0].view(np.uint32) == 0)
    for r, sl in enumerate(slots):
        if sl < 0:
            continue
        one = orc.mxfp4_gemm(a_q[r:r + 1], a_s[r:r + 1], w4[sl:sl + 1], w4_s[sl:sl + 1], mode=orc.MODE_GROUPED,
                             expert_offsets=np.array([0, 1], np.int32))
        assert np.array_equal(one.view(np.uint32), out[r:r + 1].view(np.uint32))


def test_mxfp4_integer_case_is_exact(orc):
    """Codes with integer values (E2M1 1, 2, 3, 4, 6 and their negatives), E8M0 = 1, activations that are
    small integers with unit scales: every partial sum is an integer below 2^24, so the result is exact."""
    rng = np.random.default_rng(7)
    N, K, R = 16, 256, 5
    int_codes = np.array([0x2, 0x4, 0x5, 0x6, 0x7, 0xA, 0xC, 0xD, 0xE, 0xF], np.uint8)
    codes = rng.choice(int_codes, size=(1, N, K))
    w4 = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    w4_s = np.full((1, N, K // 32), 127, np.uint8)
    ints = rng.integers(-4, 5, size=(R, K)).astype(np.float32)
    a_q = torch.from_numpy(ints).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    a_s = np.ones((R, K // 128), np.float32)
    got = orc.mxfp4_gemm(a_q, a_s, w4, w4_s, mode=orc.MODE_GROUPED, expert_offsets=np.array([0, R], np.int32))
    want = ints.astype(np.int64) @ np.vectorize(e2m1_closed_form)(codes[0]).astype(np.int64).T
    assert np.array_equal(got, want.astype(np.float32))
