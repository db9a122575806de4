"""Helpers shared by the GPU parity tests (comparison rules, error bounds and tensor moves)."""
import numpy as np
import torch

import oracle

REL_L2 = 5e-3       # bf16 outputs: relative L2 error bound
MAX_ABS = 2e-2      # and max-abs error bound, relative to max |oracle|


def dev():
    return torch.device("cuda:0")


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)) if isinstance(a, np.ndarray) else a
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev())


def u16(t: torch.Tensor) -> np.ndarray:
    """bf16/f16 tensor -> raw uint16 bits on the host."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_close(got: np.ndarray, ref: np.ndarray, rel_l2=REL_L2, max_abs=MAX_ABS, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    peak = np.abs(ref).max() if ref.size else 0.0
    if peak == 0.0:
        assert np.all(got == 0.0), what + ": oracle is all zero, output is not"
        return
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    mad = np.abs(got - ref).max()
    assert rel <= rel_l2, "%s: rel L2 %.3e > %.1e" % (what, rel, rel_l2)
    assert mad <= max_abs * peak, "%s: max abs %.3e > %.1e * %.3e" % (what, mad, max_abs, peak)


def assert_bf16_close(got_bits, ref_bits, what=""):
    assert_close(bf16_bits_to_f64(got_bits), bf16_bits_to_f64(ref_bits), what=what)


def _t_dec(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64)


BLOCK_ROUNDINGS = 136   # per side: 127 additions inside a 128-wide K block, 2 scale roundings, and slack
MFMA_BLOCK_SUM = 2.0 ** -11   # the device's sum of one K block's 128 products, as a fraction of their sum |p|


def bound_factor(K):
    """Per-output bound on |device - oracle| of an fp32 block-scaled GEMM, in units of sum_k |a_k w_k s|.

    Each side sums K exact products, 128 at a time.  The oracle adds a block's products in ascending k in
    fp32, within 127 u sum|p| of their exact sum (u = 2^-23: any order, rounding or truncating).  The
    device's fp8 MFMA does not add them in fp32: like other fp8 matrix units it keeps only about 13-14
    significant bits of the block sum (its products are aligned to the largest one and truncated, which
    biases all-positive sums downward).  Measured on MI355X over 2M block sums against the exact sum, its
    error reached 2^-12.5 of the block's sum|p| with all products positive and 2^-13.2 with random signs;
    the bound takes 2^-11 for it.  Per block, each side also rounds the scale product and p * s and
    accumulates once in fp32; split-K forms add at most 8 accumulates.  So the two sides are within
    (2^-11 + 2 (136 + 3 K/128) u) sum|a w s| of each other."""
    return MFMA_BLOCK_SUM + 2.0 * (BLOCK_ROUNDINGS + 3 * K / 128) * 2.0 ** -23


def _rows_by_expert(experts_of_rows):
    ex = np.asarray(experts_of_rows)
    return {int(e): np.nonzero(ex == e)[0] for e in np.unique(ex) if e >= 0}


def gemm_abs_bound(a_q, a_s, w_q, w_s, experts_of_rows, a_rows):
    """Per-element bound on |device - oracle| for an fp32 block-FP8 GEMM output: bound_factor(K) times
    sum_k |a_k| |w_k| sA sW (dequantized magnitudes, float64)."""
    E, N, K = w_q.shape
    A = _t_dec(a_q).abs() * torch.from_numpy(np.repeat(a_s, 128, axis=1)[:, :K]).double()
    out = np.zeros((len(experts_of_rows), N))
    a_rows = np.asarray(a_rows)
    for e, rows in _rows_by_expert(experts_of_rows).items():
        W = _t_dec(w_q[e]).abs() * torch.from_numpy(
            np.repeat(np.repeat(w_s[e], 128, axis=0), 128, axis=1)[:N, :K]).double()
        out[rows] = (A[torch.from_numpy(a_rows[rows])] @ W.T).numpy()
    return out * bound_factor(K)


E2M1_ABS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0] * 2)   # |value| of each E2M1 code


def mxfp4_abs_bound(a_q, a_s, w4, w4_s, experts_of_rows, a_rows):
    """gemm_abs_bound for MXFP4 weights: the same per-block form, with
    |w[e, n, k]| = |e2m1(nibble)| * 2^(w4_s[e, n, k/32] - 127) (the E8M0 scale is applied exactly)."""
    E, N, K2 = w4.shape
    K = 2 * K2
    A = _t_dec(a_q).abs() * torch.from_numpy(np.repeat(a_s, 128, axis=1)[:, :K]).double()
    out = np.zeros((len(experts_of_rows), N))
    a_rows = np.asarray(a_rows)
    for e, rows in _rows_by_expert(experts_of_rows).items():
        codes = np.stack([w4[e] & 15, w4[e] >> 4], axis=2).reshape(N, K)
        W = torch.from_numpy(E2M1_ABS[codes] * np.exp2(np.repeat(w4_s[e].astype(np.float64), 32, axis=1) - 127.0))
        out[rows] = (A[torch.from_numpy(a_rows[rows])] @ W.T).numpy()
    return out * bound_factor(K)


def assert_bf16_within_bound(got_bits, ref32, bound, what=""):
    """Element-wise check of a bf16 output against the oracle's fp32 accumulator: the device's own fp32
    value is within `bound` of it, and its rounding to bf16 moves it by at most half a bf16 step
    (2^-8 of its magnitude); the oracle's bf16 output is bf16(ref32), so this also bounds the two outputs'
    difference."""
    got = bf16_bits_to_f64(got_bits)
    ref = np.asarray(ref32, np.float64)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    allowed = bound + 2.0 ** -8 * (np.abs(ref) + bound) + 1e-38
    bad = np.abs(got - ref) > allowed
    assert not bad.any(), "%s: %d bf16 elements beyond the bound (worst excess %.3e)" % (
        what, bad.sum(), (np.abs(got - ref) - allowed)[bad].max())


def assert_within_bound(got, ref, bound, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    err = np.abs(got - ref)
    bad = err > bound
    assert not bad.any(), "%s: %d elements beyond the fp32 accumulation bound (worst %.3e vs %.3e)" % (
        what, bad.sum(), err[bad].max(), bound[bad][np.argmax(err[bad])])


NP_OUT = {torch.float32: np.float32, torch.bfloat16: np.uint16, torch.float16: np.float16}


def host_out(t):
    if t.dtype == torch.float32:
        return t.cpu().numpy().astype(np.float64)
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def ref_as_f64(ref, dtype):
    if dtype == torch.bfloat16:
        return oracle.bf16_decode(ref).astype(np.float64)
    return ref.astype(np.float64)


def act64(act, g):
    """The gate functions of the five gated activations in float64 (scipy's erf and expit)."""
    from scipy.special import erf, expit
    return {1: lambda x: x * expit(x), 2: lambda x: x * 0.5 * (1 + erf(x / np.sqrt(2))),
            3: lambda x: np.maximum(x, 0), 4: expit, 5: lambda x: x}[act](g)


def silu_h_bound(c1_ref, c1_bound, I, act=1):
    """|h_gpu - h_oracle| bound from the two sides' fp32 c1 bound: every gate function here has slope at most
    1.13 (GELU's maximum; SiLU 1.1, ReLU and identity 1, sigmoid 0.25), so |dh| <= 1.13 |dg| (|u| + |du|) +
    |act(g)| |du|, plus a few fp32 roundings of h itself (the device erff/expf within a few ulp)."""
    g, u = c1_ref[:, :I].astype(np.float64), c1_ref[:, I:].astype(np.float64)
    dg, du = c1_bound[:, :I], c1_bound[:, I:]
    sg = act64(act, g)
    return 1.13 * dg * (np.abs(u) + du) + np.abs(sg) * du + 16 * 2.0 ** -24 * np.abs(sg * u) + 1e-30


def check_codes_and_scales(orc, q, s, ref_q, ref_s, h_bound):
    """Scales within the h bound / 448 of the oracle's.  Each side's dequantized value is within half an
    e4m3 step of its own h (a step is at most 1/8 of the value, or 2^-9 scale units below the normal
    range), and the two h are within h_bound of each other, so the dequantized values may differ by
    h_bound plus both half steps.  Codes rarely differ at all."""
    groups = ref_s.shape[1]
    hb = h_bound.reshape(h_bound.shape[0], groups, 128).max(axis=2)
    assert np.all(np.abs(s.astype(np.float64) - ref_s) <= hb / 448 * 1.01 + 2.0 ** -24 * np.abs(ref_s)), "scales"
    diff = q != ref_q
    assert diff.mean() < 1e-2, "codes differ at %.3g of positions" % diff.mean()
    dec = lambda c: orc.e4m3_decode(c).astype(np.float64)
    sg = np.repeat(s.astype(np.float64), 128, axis=1)
    sr = np.repeat(ref_s.astype(np.float64), 128, axis=1)
    dq, dr = dec(q) * sg, dec(ref_q) * sr
    allowed = 1.01 * h_bound + 0.0625 * (np.abs(dq) + np.abs(dr)) + 2.0 ** -10 * (sg + sr)
    bad = np.abs(dq - dr) > allowed
    assert not bad.any(), "%d dequantized values beyond the bound" % bad.sum()
