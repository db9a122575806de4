"""Helpers shared by the GPU parity tests (comparison rules and tensor moves)."""
import numpy as np
import torch

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


def gemm_abs_bound(a_q, a_s, w_q, w_s, experts_of_rows, a_rows):
    """Per-element bound on |device - oracle| for an fp32 block-FP8 GEMM output.

    Recursive summation of n terms in any order, each addition rounded or truncated to fp32
    (unit 2^-23), is within n * 2^-23 * sum|terms| of the exact sum.  Each output sums K exact
    products plus two scale multiplies and one accumulate per 128-wide block, so each side is within
    (K + 4K/128 + 4) * 2^-23 * sum_k |a_k w_k s| of the exact result; the MFMA's internal K reduction
    is covered whatever its order or rounding.  The two sides are within twice that of each other."""
    E, N, K = w_q.shape
    A = _t_dec(a_q).abs() * torch.from_numpy(np.repeat(a_s, 128, axis=1)[:, :K]).double()
    out = np.zeros((len(experts_of_rows), N))
    for r, e in enumerate(experts_of_rows):
        if e < 0:
            continue
        W = _t_dec(w_q[e]).abs() * torch.from_numpy(
            np.repeat(np.repeat(w_s[e], 128, axis=0), 128, axis=1)[:N, :K]).double()
        out[r] = (W @ A[a_rows[r]]).numpy()
    return 2.0 * out * (K + 4 * K / 128 + 4) * 2.0 ** -23


def assert_within_bound(got, ref, bound, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    err = np.abs(got - ref)
    bad = err > bound
    assert not bad.any(), "%s: %d elements beyond the fp32 accumulation bound (worst %.3e vs %.3e)" % (
        what, bad.sum(), err[bad].max(), bound[bad][np.argmax(err[bad])])
