"""CPU oracle of the routed-expert hot path (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this module.  It builds ``orc.c`` with gcc into
``liborc.so`` and wraps each entry point for numpy arrays.  Nothing here
imports or calls the HIP library, and the HIP library never imports this.

Each function below follows the C function of the same name in ``orc.c``;
the definitions and the passages they come from are documented there.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "orc.c")
_LIB_PATH = os.path.join(_HERE, "liborc.so")

BF16, F32, F16 = 0, 1, 2
MODE_GROUPED, MODE_SLOT = 0, 1

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with plain gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(
        os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "orc.h"))
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-Wno-unused-parameter", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.orc_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_to_f32.restype = ctypes.c_float
        L.orc_f32_to_e4m3.argtypes = [ctypes.c_float]
        L.orc_f32_to_e4m3.restype = ctypes.c_uint8
        for name in ("orc_e4m3_decode_array", "orc_e4m3_encode_array", "orc_bf16_encode_array",
                     "orc_f16_encode_array"):
            getattr(L, name).argtypes = [P, I64, P]
            getattr(L, name).restype = None
        L.orc_quant_groups.argtypes = [P, I32, I64, I64, I64, P, I64, P, I64]
        L.orc_gather_rows_scales.argtypes = [P, I64, P, I64, I64, I64, I64, P, I64, P, I64, P, I64]
        L.orc_block_gemm.argtypes = [P, I64, P, I64, P, I64, I64, P, I64, I64, I64, I64, I64,
                                     I32, P, P, I64, I64, P, I32, I64]
        L.orc_silu_mul_quant.argtypes = [P, I32, I64, I64, I64, P, I64, P, I64]
        L.orc_gated_act_quant.argtypes = [P, I32, I64, I64, I64, I32, P, I64, P, I64]
        L.orc_topk_reduce.argtypes = [P, I32, I64, P, P, P, I64, I64, I64, P, I64]
        L.orc_mxfp4_gemm.argtypes = [P, I64, P, I64, P, I64, I64, P, I64, I64, I64, I64, I64,
                                     I32, P, P, I64, I64, P, I32, I64]
        L.orc_e2m1_to_f32.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_to_f32.restype = ctypes.c_float
        L.orc_e8m0_to_f32.argtypes = [ctypes.c_uint8]
        L.orc_e8m0_to_f32.restype = ctypes.c_float
        L.orc_route_prep.argtypes = [P, I64, I64, I64, I64, P, P, P, P, P]
        L.orc_fused_decode.argtypes = [P, I64, I64, I64, I64, I32, P, P, I64, P, P, P, P, P,
                                       P, P, P, P, P, P]
        for name in ("orc_quant_groups", "orc_gather_rows_scales", "orc_block_gemm",
                     "orc_silu_mul_quant", "orc_gated_act_quant", "orc_topk_reduce", "orc_fused_decode",
                     "orc_mxfp4_gemm"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    a = np.asarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    assert a.flags["C_CONTIGUOUS"]
    return a


def _dt_code(dtype) -> int:
    if dtype == np.float32:
        return F32
    if dtype == np.float16:
        return F16
    if dtype == np.uint16:  # bf16 carried as raw uint16 bits
        return BF16
    raise ValueError(dtype)


def _check(rc):
    if rc != 0:
        raise ValueError("oracle rejected its arguments (status %d)" % rc)


# ---- codecs -------------------------------------------------------------

def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, np.float32)
    lib().orc_e4m3_decode_array(_p(codes), codes.size, _p(out))
    return out


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().orc_e4m3_encode_array(_p(v), v.size, _p(out))
    return out


def bf16_encode(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint16)
    lib().orc_bf16_encode_array(_p(v), v.size, _p(out))
    return out


def f16_encode(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint16)
    lib().orc_f16_encode_array(_p(v), v.size, _p(out))
    return out


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


# ---- O1 ---------------------------------------------------------------------

def quant_groups(x: np.ndarray):
    """x: [rows, n] float32, float16 or bf16-as-uint16 -> (q uint8 [rows,n], s f32 [rows,ceil(n/128)])."""
    x = np.ascontiguousarray(x)
    rows, n = x.shape
    g = (n + 127) // 128
    q = np.empty((rows, n), np.uint8)
    s = np.empty((rows, g), np.float32)
    _check(lib().orc_quant_groups(_p(x), _dt_code(x.dtype), n, rows, n, _p(q), n, _p(s), g))
    return q, s


# ---- O2 ---------------------------------------------------------------------

def gather_rows_scales(src_q: np.ndarray, src_s: np.ndarray, dst2src: np.ndarray, k: int | None = None,
                       g: int | None = None):
    src_q = _c(src_q, np.uint8)
    src_s = np.ascontiguousarray(src_s).view(np.float32)
    dst2src = _c(dst2src, np.int32)
    n_src = src_q.shape[0]
    k = src_q.shape[1] if k is None else k
    g = src_s.shape[1] if g is None else g
    n_dst = dst2src.shape[0]
    dq = np.empty((n_dst, k), np.uint8)
    ds = np.empty((n_dst, g), np.float32)
    _check(lib().orc_gather_rows_scales(_p(src_q), src_q.shape[1], _p(src_s), src_s.shape[1], n_src, k, g,
                                        _p(dst2src), n_dst, _p(dq), k, _p(ds), g))
    return dq, ds


# ---- O3 ---------------------------------------------------------------------

def block_gemm(a_q, a_s, w_q, w_s, *, mode, out_dtype=np.float32, expert_offsets=None, slot_ids=None,
               m_rows=None, a_row_div=1):
    """a_q [Ra, K] u8, a_s [Ra, ceil(K/128)] f32, w_q [E, N, K] u8, w_s [E, ceil(N/128), ceil(K/128)] f32.

    out_dtype: np.float32, np.float16 or np.uint16 (= bf16 bits).  Returns [m_rows, N]."""
    a_q = _c(a_q, np.uint8)
    a_s = _c(a_s, np.float32)
    w_q = _c(w_q, np.uint8)
    w_s = _c(w_s, np.float32)
    E, N, K = w_q.shape
    if mode == MODE_GROUPED:
        expert_offsets = _c(expert_offsets, np.int32)
        m_rows = int(expert_offsets[-1])
    else:
        slot_ids = _c(slot_ids, np.int32)
        m_rows = slot_ids.shape[0] if m_rows is None else m_rows
    out = np.empty((m_rows, N), out_dtype)
    _check(lib().orc_block_gemm(_p(a_q), a_q.shape[1], _p(a_s), a_s.shape[1],
                                _p(w_q), N * K, K, _p(w_s), w_s.shape[1] * w_s.shape[2], w_s.shape[2],
                                E, N, K, mode, _p(expert_offsets), _p(slot_ids), m_rows, a_row_div,
                                _p(out), _dt_code(np.dtype(out_dtype)), N))
    return out


# ---- O4 ---------------------------------------------------------------------

# ---- O8 ---------------------------------------------------------------------

def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """FP4 E2M1 codes (low 4 bits of each entry) -> float32."""
    return np.array([lib().orc_e2m1_to_f32(int(c) & 15) for c in np.asarray(codes).ravel()],
                    np.float32).reshape(np.shape(codes))


def e8m0_decode(codes: np.ndarray) -> np.ndarray:
    return np.array([lib().orc_e8m0_to_f32(int(c)) for c in np.asarray(codes).ravel()],
                    np.float32).reshape(np.shape(codes))


def mxfp4_gemm(a_q, a_s, w4, w4_s, *, mode, out_dtype=np.float32, expert_offsets=None, slot_ids=None,
               m_rows=None, a_row_div=1):
    """a_q [Ra, K] u8, a_s [Ra, K/128] f32, w4 [E, N, K/2] u8 (two E2M1 per byte, even k low),
    w4_s [E, N, K/32] u8 (E8M0).  Returns [m_rows, N] of out_dtype (np.float32, np.float16, np.uint16 = bf16)."""
    a_q, a_s = _c(a_q, np.uint8), _c(a_s, np.float32)
    w4, w4_s = _c(w4, np.uint8), _c(w4_s, np.uint8)
    E, N, K2 = w4.shape
    K = 2 * K2
    if mode == MODE_GROUPED:
        expert_offsets = _c(expert_offsets, np.int32)
        m_rows = int(expert_offsets[-1]) if m_rows is None else m_rows
    else:
        slot_ids = _c(slot_ids, np.int32)
        m_rows = slot_ids.size if m_rows is None else m_rows
    out = np.empty((m_rows, N), out_dtype)
    _check(lib().orc_mxfp4_gemm(_p(a_q), a_q.shape[1], _p(a_s), a_s.shape[1], _p(w4), N * K2, K2, _p(w4_s),
                                N * (K // 32), K // 32, E, N, K, mode, _p(expert_offsets), _p(slot_ids), m_rows,
                                a_row_div, _p(out), _dt_code(out_dtype), N))
    return out


# gated activations of O4 (the five GLU variants; values as in the C header)
ACT_SILU_MUL, ACT_GELU_MUL, ACT_RELU_MUL, ACT_SIGMOID_MUL, ACT_MUL = 1, 2, 3, 4, 5


def gated_act_quant(c1: np.ndarray, act: int):
    """c1: [rows, 2n] (float32, float16 or bf16 bits), gate then up -> (q [rows, n], s [rows, ceil(n/128)])."""
    c1 = np.ascontiguousarray(c1)
    rows, n2 = c1.shape
    n = n2 // 2
    g = (n + 127) // 128
    q = np.empty((rows, n), np.uint8)
    s = np.empty((rows, g), np.float32)
    _check(lib().orc_gated_act_quant(_p(c1), _dt_code(c1.dtype), n2, rows, n, act, _p(q), n, _p(s), g))
    return q, s


def silu_mul_quant(c1: np.ndarray):
    """c1: [rows, 2n] (float32, float16 or bf16 bits) -> (q [rows, n], s [rows, ceil(n/128)])."""
    c1 = np.ascontiguousarray(c1)
    rows, n2 = c1.shape
    n = n2 // 2
    g = (n + 127) // 128
    q = np.empty((rows, n), np.uint8)
    s = np.empty((rows, g), np.float32)
    _check(lib().orc_silu_mul_quant(_p(c1), _dt_code(c1.dtype), n2, rows, n, _p(q), n, _p(s), g))
    return q, s


# ---- O5 ---------------------------------------------------------------------

def topk_reduce(y: np.ndarray, slot_ids: np.ndarray, weights: np.ndarray, route_rows=None):
    """y: [R, H]; slot_ids, weights: [T, topk]; route_rows [T, topk] or None -> bf16 bits [T, H]."""
    y = np.ascontiguousarray(y)
    slot_ids = _c(slot_ids, np.int32)
    weights = _c(weights, np.float32)
    T, topk = slot_ids.shape
    H = y.shape[1]
    rr = None if route_rows is None else _c(route_rows, np.int32)
    out = np.empty((T, H), np.uint16)
    _check(lib().orc_topk_reduce(_p(y), _dt_code(y.dtype), H, _p(slot_ids), _p(rr), _p(weights),
                                 T, topk, H, _p(out), H))
    return out


# ---- O6 ---------------------------------------------------------------------

def fused_decode(x_bf16, slot_ids, weights, w13_q, w13_s, w2_q, w2_s, intermediates=False, act=ACT_SILU_MUL):
    """x_bf16: [T, H] uint16 bits; slot_ids/weights: [T, topk]; W13 [S, 2I, H], W2 [S, H, I].

    Returns out bf16 bits [T, H] (and a dict of intermediates if asked)."""
    x_bf16 = _c(x_bf16, np.uint16)
    slot_ids = _c(slot_ids, np.int32)
    weights = _c(weights, np.float32)
    w13_q, w13_s = _c(w13_q, np.uint8), _c(w13_s, np.float32)
    w2_q, w2_s = _c(w2_q, np.uint8), _c(w2_s, np.float32)
    T, H = x_bf16.shape
    topk = slot_ids.shape[1]
    S, I2, H2 = w13_q.shape
    I = I2 // 2
    assert H2 == H and w2_q.shape == (S, H, I)
    assert w13_s.shape == (S, (2 * I + 127) // 128, (H + 127) // 128)
    assert w2_s.shape == (S, (H + 127) // 128, (I + 127) // 128)
    R = T * topk
    out = np.empty((T, H), np.uint16)
    im = None
    if intermediates:
        im = dict(xq=np.empty((T, H), np.uint8), xs=np.empty((T, (H + 127) // 128), np.float32),
                  c1=np.empty((R, 2 * I), np.float32), aq=np.empty((R, I), np.uint8),
                  as_=np.empty((R, (I + 127) // 128), np.float32), c2=np.empty((R, H), np.float32))
    g = (lambda k: _p(im[k])) if im else (lambda k: None)
    _check(lib().orc_fused_decode(_p(x_bf16), T, H, I, topk, act, _p(slot_ids), _p(weights), S,
                                  _p(w13_q), _p(w13_s), _p(w2_q), _p(w2_s), _p(out),
                                  g("xq"), g("xs"), g("c1"), g("aq"), g("as_"), g("c2")))
    return (out, im) if intermediates else out


def route_prep(logits: np.ndarray, topk: int):
    """O7: top-k routing and the (expert, token)-ordered route maps.
    Returns dict with expert_ids [T,topk] int32, weights [T,topk] f32, dst2src [T*topk], route_rows [T*topk],
    expert_offsets [E+1] (all int32)."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.zeros((T, topk), np.int32)
    w = np.zeros((T, topk), np.float32)
    d2s = np.zeros(T * topk, np.int32)
    rr = np.zeros(T * topk, np.int32)
    offs = np.zeros(E + 1, np.int32)
    rc = lib().orc_route_prep(_p(logits), E, T, E, topk, _p(ids), _p(w), _p(d2s), _p(rr), _p(offs))
    if rc:
        raise ValueError("orc_route_prep: bad arguments")
    return dict(expert_ids=ids, weights=w, dst2src=d2s, route_rows=rr, expert_offsets=offs)
