"""Seeded synthetic inputs for the routed-expert hot path.

This module only draws inputs.  It holds none of the path's arithmetic
(no GEMM, activation, requantization or reduction) and serves the CPU oracle
and the HIP library alike.  Every generator is deterministic in its seed and
uses torch's own RNG, on the CPU for test-sized inputs or on a GPU for the
full-size benchmark inputs.

The recipe follows the workloads the pages describe:
  * expert weights N(0, 0.02), stored as fp8 e4m3 codes with one fp32 scale
    per 128x128 block, scale = block amax / 448 ("perf(moe): skip inactive
    block-fp8 decode routes", GPU decode A/B: synthetic block-quantized expert
    banks with padded block scales);
  * token activations N(0, 1) in bf16;
  * routing weights: softmax over N(0, 1) logits, top-k by value (ties to the
    lower index), renormalized over the top-k;
  * decode: batch 1, top-k 8 with 8/4/2/0 routes active, the rest -1;
  * gather: random fp8 bytes (NaN codes included) with k/128 random 32-bit
    scale words per row, dst2src drawn with randint so sources repeat
    ("[MoE] Gather the cutlass MoE activation and its scales in one launch",
    Accuracy Tests);
  * grouped prefill: E experts, each token picks top-k distinct experts
    uniformly, rows sorted by (expert, token) ("perf(dsfp4): pick the
    grouped-prefill tile from route density on sm_89", Measurements).
The weight quantization below is input synthesis done with torch's own fp8
cast; the hot path never quantizes weights.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch


def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def block_fp8_weights(E: int, N: int, K: int, seed: int, std: float = 0.02, device="cpu",
                      chunk_experts: int = 8):
    """Random expert bank: (w_q uint8 [E,N,K], w_s float32 [E,ceil(N/128),ceil(K/128)]) on `device`."""
    nb, kb = (N + 127) // 128, (K + 127) // 128
    w_q = torch.empty((E, N, K), dtype=torch.uint8, device=device)
    w_s = torch.empty((E, nb, kb), dtype=torch.float32, device=device)
    g = _gen(seed, device)
    for e0 in range(0, E, chunk_experts):
        e1 = min(E, e0 + chunk_experts)
        w = torch.randn((e1 - e0, N, K), generator=g, device=device, dtype=torch.float32) * std
        wp = torch.zeros((e1 - e0, nb * 128, kb * 128), dtype=torch.float32, device=device)
        wp[:, :N, :K] = w
        blocks = wp.view(e1 - e0, nb, 128, kb, 128)
        amax = blocks.abs().amax(dim=(2, 4))
        s = amax / 448.0
        safe = torch.where(s == 0, torch.ones_like(s), s)
        q = (blocks / safe[:, :, None, :, None]).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
        q = q.view(torch.uint8).view(e1 - e0, nb * 128, kb * 128)[:, :N, :K]
        w_q[e0:e1] = q
        w_s[e0:e1] = s
        del w, wp, blocks, q
    return w_q, w_s


def mxfp4_weights(E: int, N: int, K: int, seed: int, device="cpu", e_lo: int = 120, e_hi: int = 122):
    """MXFP4 expert weights drawn directly as codes: w4 [E, N, K/2] uint8 (two E2M1 codes per byte,
    every nibble uniform over the 16 codes) and w4_s [E, N, K/32] uint8 E8M0 exponents uniform in
    [e_lo, e_hi] (2^-7 .. 2^-5 by default, so weights span about +-0.2 like N(0, 0.02) banks' tails)."""
    g = _gen(seed, device)
    w4 = torch.randint(0, 256, (E, N, K // 2), generator=g, device=device, dtype=torch.int32).to(torch.uint8)
    w4_s = torch.randint(e_lo, e_hi + 1, (E, N, K // 32), generator=g, device=device,
                         dtype=torch.int32).to(torch.uint8)
    return w4, w4_s


def bf16_normal(shape, seed: int, device="cpu", std: float = 1.0) -> torch.Tensor:
    g = _gen(seed, device)
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)


def routing(T: int, E: int, topk: int, seed: int):
    """Softmax over N(0,1) logits, top-k (ties -> lower index), renormalized: (ids int32, w float32) [T,topk]."""
    g = _gen(seed)
    logits = torch.randn((T, E), generator=g, dtype=torch.float64).numpy()
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    ids = np.argsort(-p, axis=1, kind="stable")[:, :topk].astype(np.int32)
    w = np.take_along_axis(p, ids, axis=1)
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


def router_logits(T: int, E: int, seed: int, skew: float = 0.0) -> np.ndarray:
    """fp32 router logits [T, E]: N(0,1) per (token, expert) plus a per-expert N(0, skew) offset, so
    skew > 0 gives the uneven expert loads of a trained router (a few hot experts, some cold)."""
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E))
    if skew:
        lg = lg + skew * rng.standard_normal(E)[None, :]
    return lg.astype(np.float32)


@dataclass
class DecodeCase:
    T: int
    H: int
    I: int
    topk: int
    n_slots: int
    x: torch.Tensor          # [T, H] bf16
    slot_ids: np.ndarray     # [T, topk] int32, -1 = inactive
    weights: np.ndarray      # [T, topk] f32
    w13_q: torch.Tensor      # [S, 2I, H] uint8
    w13_s: torch.Tensor      # [S, 2I/128, H/128] f32
    w2_q: torch.Tensor       # [S, H, I] uint8
    w2_s: torch.Tensor       # [S, H/128, I/128] f32


def decode_slots(T: int, topk: int, n_slots: int, active: int, seed: int, tail: bool = False):
    """Slot ids [T, topk]: `active` distinct slots per token at random positions (or the leading ones
    when tail=True), the others -1; routing weights from `routing` over the slot pool."""
    ids, w = routing(T, n_slots, topk, seed)
    rng = np.random.default_rng(seed + 1)
    slots = ids.copy()
    for t in range(T):
        if tail:
            inactive = np.arange(active, topk)
        else:
            inactive = rng.permutation(topk)[: topk - active]
        slots[t, inactive] = -1
    return slots.astype(np.int32), w


def decode_case(H: int, I: int, topk: int, n_slots: int, active: int, seed: int, T: int = 1,
                device="cpu", tail: bool = False) -> DecodeCase:
    w13_q, w13_s = block_fp8_weights(n_slots, 2 * I, H, seed * 7 + 11, device=device)
    w2_q, w2_s = block_fp8_weights(n_slots, H, I, seed * 7 + 13, device=device)
    x = bf16_normal((T, H), seed * 7 + 17, device=device)
    slots, w = decode_slots(T, topk, n_slots, active, seed * 7 + 19, tail=tail)
    return DecodeCase(T, H, I, topk, n_slots, x, slots, w, w13_q, w13_s, w2_q, w2_s)


def gather_case(k: int, tokens: int, topk: int, seed: int, g: int | None = None):
    """(src_q uint8 [tokens,k], src_s int32-bits [tokens,g], dst2src int32 [tokens*topk])."""
    gen = _gen(seed)
    g = (k + 127) // 128 if g is None else g
    src_q = torch.randint(0, 256, (tokens, k), generator=gen, dtype=torch.int32).to(torch.uint8)
    src_s = torch.randint(-(2 ** 31), 2 ** 31 - 1, (tokens, g), generator=gen, dtype=torch.int64).to(torch.int32)
    dst2src = torch.randint(0, max(tokens, 1), (tokens * topk,), generator=gen, dtype=torch.int32)
    return src_q.numpy(), src_s.numpy(), dst2src.numpy()


@dataclass
class PrefillRoutes:
    T: int
    E: int
    topk: int
    expert_ids: np.ndarray     # [T, topk] int32, distinct per token
    weights: np.ndarray        # [T, topk] f32
    dst2src: np.ndarray        # [R] int32: token of each expert-sorted row
    route_rows: np.ndarray     # [T, topk] int32: sorted row of route (t, j)
    expert_offsets: np.ndarray  # [E+1] int32


def prefill_routes(T: int, E: int, topk: int, seed: int) -> PrefillRoutes:
    """Each token picks `topk` distinct experts uniformly; rows are sorted by (expert, token)."""
    rng = np.random.default_rng(seed)
    keys = rng.random((T, E))
    ids = np.argsort(keys, axis=1, kind="stable")[:, :topk].astype(np.int32)
    w = rng.random((T, topk)).astype(np.float32) + 0.05
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    flat_e = ids.reshape(-1).astype(np.int64)
    flat_t = np.repeat(np.arange(T, dtype=np.int64), topk)
    order = np.lexsort((flat_t, flat_e))          # by expert, then token
    dst2src = flat_t[order].astype(np.int32)
    route_rows = np.empty(T * topk, np.int32)
    route_rows[order] = np.arange(T * topk, dtype=np.int32)
    counts = np.bincount(flat_e, minlength=E)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    return PrefillRoutes(T, E, topk, ids, w, dst2src, route_rows.reshape(T, topk), offsets)


def fp8_rows(rows: int, k: int, seed: int, device="cpu", full_range: bool = False):
    """Activation rows as fp8 codes with 1x128 group scales, drawn directly (no quantizer):
    codes uniform over the finite e4m3 codes with |value| <= 4 (4-bit mantissa grid), or with
    full_range over every finite code (|value| up to 448, subnormals included, as a quantized row's
    codes span), scales log-uniform in [2^-8, 2^-4]."""
    g = _gen(seed, device)
    # finite codes with |v| <= 4: exponent field 0..9 (2^(e-7) <= 4) -> codes 0x00..0x48 and their negatives;
    # full range: 0x00..0x7E (0x7F is NaN)
    mag = torch.randint(0, 0x7F if full_range else 0x49, (rows, k), generator=g, device=device, dtype=torch.int32)
    sign = torch.randint(0, 2, (rows, k), generator=g, device=device, dtype=torch.int32) * 0x80
    q = (mag | sign).to(torch.uint8)
    gk = (k + 127) // 128
    s = torch.exp2(torch.rand((rows, gk), generator=g, device=device) * 4.0 - 8.0).to(torch.float32)
    return q, s


def powers_of_two_case(E: int, N: int, K: int, rows: int, seed: int):
    """Integer-exact block-FP8 operands: codes of the values -4..4 and power-of-two scales, so that
    every product, block sum and scaled sum is exact in fp32.  Returns numpy arrays
    (a_q [rows,K], a_s [rows,K/128], w_q [E,N,K], w_s [E,N/128,K/128])."""
    rng = np.random.default_rng(seed)
    # e4m3 codes of -4..4: 0 -> 0x00, 1 -> 0x38, 2 -> 0x40, 3 -> 0x44, 4 -> 0x48
    pos = np.array([0x00, 0x38, 0x40, 0x44, 0x48], np.uint8)
    def draw(shape):
        v = rng.integers(-4, 5, size=shape)
        c = pos[np.abs(v)]
        return np.where(v < 0, c | 0x80, c).astype(np.uint8)
    a_q = draw((rows, K))
    w_q = draw((E, N, K))
    a_s = np.exp2(rng.integers(-3, 2, size=(rows, (K + 127) // 128))).astype(np.float32)
    w_s = np.exp2(rng.integers(-3, 2, size=(E, (N + 127) // 128, (K + 127) // 128))).astype(np.float32)
    return a_q, a_s, w_q, w_s


def mxfp4_exact_case(E: int, N: int, K: int, rows: int, seed: int):
    """Exact operands for the MXFP4 GEMM (K <= 8192): activation codes of -4..4 with scales in {1/2, 1, 2},
    every E2M1 weight code, E8M0 exponents 126..128.  Each product is a multiple of 2^-3 of magnitude at most
    4*2*6*2 = 96, so every partial sum is a multiple of 2^-3 below 96*8192 < 2^20: 23 significant bits, which
    fp32 holds exactly in any order.  Returns numpy arrays
    (a_q [rows,K], a_s [rows,K/128], w4 [E,N,K/2], w4_s [E,N,K/32])."""
    assert K <= 8192
    rng = np.random.default_rng(seed)
    pos = np.array([0x00, 0x38, 0x40, 0x44, 0x48], np.uint8)
    v = rng.integers(-4, 5, size=(rows, K))
    a_q = np.where(v < 0, pos[np.abs(v)] | 0x80, pos[np.abs(v)]).astype(np.uint8)
    a_s = np.exp2(rng.integers(-1, 2, size=(rows, K // 128))).astype(np.float32)
    w4 = rng.integers(0, 256, size=(E, N, K // 2)).astype(np.uint8)
    w4_s = rng.integers(126, 129, size=(E, N, K // 32)).astype(np.uint8)
    return a_q, a_s, w4, w4_s


def nbytes_expert(H: int, I: int) -> int:
    """Bytes one active decode route streams: W13 + W2 fp8 plus their fp32 block scales."""
    return 2 * I * H + H * I + 4 * (math.ceil(2 * I / 128) * math.ceil(H / 128) + math.ceil(H / 128) * math.ceil(I / 128))
