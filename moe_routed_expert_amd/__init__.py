"""Python binding of libmoe_routed (the MI355X routed-expert hot path).

Argument marshalling only: every function takes torch tensors that live on
the GPU, passes their device pointers, element strides and the current HIP
stream to the C entry point of the same name, and raises on a non-OK status.
No step of the path runs in Python or in torch, and there is no fallback: if
the shared library is missing, importing works but every call raises.

Dtypes: fp8 buffers are torch.uint8 (raw e4m3 codes), scales torch.float32,
slot ids / maps / offsets torch.int32, 16-bit outputs torch.bfloat16 or
torch.float16.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_routed.so")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_WORKSPACE, MOE_ERR_ALIGN, MOE_ERR_HIP = 0, -1, -2, -3, -4, -5, -6
MOE_ERR_SCRATCH = -7
MOE_BF16, MOE_F32, MOE_F16 = 0, 1, 2
MOE_ACT_IDENTITY, MOE_ACT_SILU_MUL, MOE_ACT_GELU_MUL, MOE_ACT_RELU_MUL, MOE_ACT_SIGMOID_MUL, MOE_ACT_MUL = 0, 1, 2, 3, 4, 5
MOE_MODE_GROUPED, MOE_MODE_SLOT = 0, 1
MOE_W_PACKED = -1

EXPORTS = (
    "moe_abi_version", "moe_status_string", "moe_last_hip_error", "moe_gather_rows_scales", "moe_act_quant",
    "moe_pick_block_m", "moe_bf8_grouped_gemm", "moe_topk_reduce", "moe_fused_decode_workspace_size",
    "moe_fused_decode_workspace_layout", "moe_fused_decode_workspace_init", "moe_fused_decode",
    "moe_route_prep_workspace_size", "moe_route_prep", "moe_bf8_grouped_gemm_act_quant",
    "moe_mxfp4_grouped_gemm", "moe_mxfp4_grouped_gemm_act_quant", "moe_fused_decode_noalloc", "moe_pack_weights",
    "moe_grouped_block_m",
)

_lib = None


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        L = lib()
        msg = L.moe_status_string(status).decode()
        if status == MOE_ERR_HIP:
            msg += ": " + L.moe_last_hip_error().decode()
        super().__init__("%s failed with status %d (%s)" % (fn, status, msg))
        self.status = status


def lib():
    """Load libmoe_routed.so (built in-tree by moe_routed_expert_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe_routed.so is not built (run moe_routed_expert_amd/build.py); "
                               "there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        sig = {
            "moe_abi_version": ([], I32),
            "moe_status_string": ([I32], ctypes.c_char_p),
            "moe_last_hip_error": ([], ctypes.c_char_p),
            "moe_gather_rows_scales": ([P, I64, P, I64, I64, I64, I64, P, I64, P, I64, P, I64, P], I32),
            "moe_act_quant": ([P, I32, I64, I64, I64, I32, P, I64, P, I64, P], I32),
            "moe_pick_block_m": ([I64, I64], I32),
            "moe_grouped_block_m": ([I64, I64, I64, I32, I32, I32], I32),
            "moe_bf8_grouped_gemm": ([P, I64, P, I64, P, I64, I64, P, I64, I64, I64, I64, I64, I32, P, P, I64, I64,
                                      ctypes.c_int32, P, I32, I64, P], I32),
            "moe_topk_reduce": ([P, I32, I64, P, P, P, I64, I64, I64, P, I64, P], I32),
            "moe_fused_decode_workspace_size": ([I64, I64, I64, I64], SZ),
            "moe_fused_decode_workspace_layout": ([I64, I64, I64, I64, P], I32),
            "moe_fused_decode_workspace_init": ([P, SZ, I64, I64, I64, I64, P], I32),
            "moe_fused_decode": ([P, I64, I64, I64, I64, I32, P, P, I64, P, P, P, P, P, SZ, P, P], I32),
            "moe_fused_decode_noalloc": ([P, I64, I64, I64, I64, I32, P, P, I64, P, P, P, P, P, P], I32),
            "moe_route_prep_workspace_size": ([I64, I64], SZ),
            "moe_route_prep": ([P, I64, I64, I64, I64, P, P, P, P, P, P, SZ, P], I32),
            "moe_bf8_grouped_gemm_act_quant": ([P, I64, P, I64, P, I64, I64, P, I64, I64, I64, I64, I64, P, I64,
                                                I32, I32, P, I64, P, I64, P], I32),
            "moe_mxfp4_grouped_gemm": ([P, I64, P, I64, P, I64, I64, P, I64, I64, I64, I64, I64, P, I64,
                                        I32, P, I32, I64, P], I32),
            "moe_mxfp4_grouped_gemm_act_quant": ([P, I64, P, I64, P, I64, I64, P, I64, I64, I64, I64, I64, P,
                                                  I64, I32, I32, P, I64, P, I64, P], I32),
            "moe_pack_weights": ([P, I64, I64, I64, I64, I64, I64, P, I64, P], I32),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status)


def _ptr(t):
    if t is None:
        return None
    assert t.is_cuda, "device tensor expected"
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dt(t: torch.Tensor) -> int:
    return {torch.bfloat16: MOE_BF16, torch.float32: MOE_F32, torch.float16: MOE_F16}[t.dtype]


def _rowstride(t: torch.Tensor) -> int:
    assert t.dim() == 2 and t.stride(1) == 1, "row-major 2-D tensor with unit column stride expected"
    return t.stride(0)


# ---------------------------------------------------------------------------

def abi_version() -> int:
    return lib().moe_abi_version()


def pick_block_m(routes: int, experts: int) -> int:
    return lib().moe_pick_block_m(routes, experts)


def grouped_block_m(routes: int, experts: int, K: int, mxfp4: bool = False, packed: bool = False,
                    fused: bool = False) -> int:
    """The M tile the grouped GEMMs take for block_m = 0 (moe_grouped_block_m)."""
    return lib().moe_grouped_block_m(routes, experts, K, int(mxfp4), int(packed), int(fused))


def gather_rows_scales(src_q, src_s, dst2src, dst_q, dst_s, k=None, g=None, stream=None):
    """dst_q[i] = src_q[dst2src[i]] (bytes), dst_s[i] = src_s[dst2src[i]] (32-bit words)."""
    k = src_q.shape[1] if k is None else k
    g = src_s.shape[1] if g is None else g
    _check("moe_gather_rows_scales", lib().moe_gather_rows_scales(
        _ptr(src_q), _rowstride(src_q), _ptr(src_s), _rowstride(src_s), src_q.shape[0], k, g,
        _ptr(dst2src), dst2src.numel(), _ptr(dst_q), _rowstride(dst_q), _ptr(dst_s), _rowstride(dst_s),
        _stream(stream)))


def act_quant(x, out_q, out_s, act=MOE_ACT_IDENTITY, n=None, stream=None):
    """1x128 fp8 quantization of x rows (IDENTITY) or of SiLU(gate)*up (SILU_MUL, x = [gate | up])."""
    n = (x.shape[1] if act == MOE_ACT_IDENTITY else x.shape[1] // 2) if n is None else n
    _check("moe_act_quant", lib().moe_act_quant(
        _ptr(x), _dt(x), _rowstride(x), x.shape[0], n, act, _ptr(out_q), _rowstride(out_q), _ptr(out_s),
        _rowstride(out_s), _stream(stream)))


def pack_weights(w, step_bytes, out=None, stream=None):
    """The packed order of an expert bank (moe_pack_weights): w [E, N, row_bytes] bytes with unit last stride,
    step_bytes 128 for block-FP8 codes (row_bytes = K) or 64 for MXFP4 (row_bytes = K/2).  Returns out (a new
    contiguous [E, N, row_bytes] byte tensor when None), to be passed to the grouped GEMMs with w_packed=True."""
    E, N, RB = w.shape
    assert w.dtype == torch.uint8 and w.stride(2) == 1
    if out is None:
        out = torch.empty((E, N, RB), dtype=torch.uint8, device=w.device)
    assert out.dtype == torch.uint8 and tuple(out.shape) == (E, N, RB) and out.stride(2) == 1 and out.stride(1) == RB
    _check("moe_pack_weights", lib().moe_pack_weights(
        _ptr(w), w.stride(0), w.stride(1), E, N, RB, step_bytes, _ptr(out), out.stride(0), _stream(stream)))
    return out


def _w_strides(w, packed):
    """(expert stride, row stride) of a weight bank argument: MOE_W_PACKED as the row stride of a packed one."""
    if packed:
        assert w.stride(2) == 1 and w.stride(1) == w.shape[2], "a packed bank is contiguous per expert"
        return w.stride(0), MOE_W_PACKED
    return w.stride(0), w.stride(1)


def bf8_grouped_gemm(a_q, a_s, w_q, w_s, out, *, mode, expert_offsets=None, slot_ids=None, m_rows=None,
                     a_row_div=1, block_m=0, w_packed=False, stream=None):
    """Block-FP8 GEMM; w_q [E, N, K] (unit K stride; the packed order of pack_weights when w_packed),
    w_s [E, ceil(N/128), K/128]."""
    E, N, K = w_q.shape
    if m_rows is None:
        m_rows = out.shape[0]
    assert w_q.stride(2) == 1 and w_s.stride(2) == 1
    _check("moe_bf8_grouped_gemm", lib().moe_bf8_grouped_gemm(
        _ptr(a_q), _rowstride(a_q), _ptr(a_s), _rowstride(a_s),
        _ptr(w_q), *_w_strides(w_q, w_packed), _ptr(w_s), w_s.stride(0), w_s.stride(1),
        E, N, K, mode, _ptr(expert_offsets), _ptr(slot_ids), m_rows, a_row_div, block_m,
        _ptr(out), _dt(out), _rowstride(out), _stream(stream)))


def bf8_grouped_gemm_act_quant(a_q, a_s, w13_q, w13_s, expert_offsets, out_q, out_s, m_rows=None, block_m=0,
                               act=1, w_packed=False, stream=None):
    """Prefill gate/up GEMM with act(gate)*up (moe_act 1..5, default SwiGLU) and the 1x128 fp8 requant in
    its epilogue.
    w13_q [E, 2I, K] (gate rows, then up rows), w13_s [E, 2I/128, K/128]; out_q [rows, I] u8, out_s [rows, I/128]."""
    E, N, K = w13_q.shape
    if m_rows is None:
        m_rows = out_q.shape[0]
    assert w13_q.stride(2) == 1 and w13_s.stride(2) == 1
    _check("moe_bf8_grouped_gemm_act_quant", lib().moe_bf8_grouped_gemm_act_quant(
        _ptr(a_q), _rowstride(a_q), _ptr(a_s), _rowstride(a_s),
        _ptr(w13_q), *_w_strides(w13_q, w_packed), _ptr(w13_s), w13_s.stride(0), w13_s.stride(1),
        E, N // 2, K, _ptr(expert_offsets), m_rows, block_m, act, _ptr(out_q), _rowstride(out_q),
        _ptr(out_s), _rowstride(out_s), _stream(stream)))


def _mxfp4_weights(w4, w4_s):
    E, N, K2 = w4.shape
    assert w4.dtype == torch.uint8 and w4_s.dtype == torch.uint8, "MXFP4 weights are byte tensors"
    assert w4.stride(2) == 1 and w4_s.stride(2) == 1 and tuple(w4_s.shape) == (E, N, K2 // 16)
    return E, N, 2 * K2


def mxfp4_grouped_gemm(a_q, a_s, w4, w4_s, expert_offsets, out, m_rows=None, block_m=0, w_packed=False,
                       stream=None):
    """Grouped GEMM with MXFP4 weights: w4 [E, N, K/2] bytes (two E2M1 codes, even k in the low nibble),
    w4_s [E, N, K/32] E8M0 bytes; a_q/a_s/out as bf8_grouped_gemm in grouped mode."""
    E, N, K = _mxfp4_weights(w4, w4_s)
    if m_rows is None:
        m_rows = out.shape[0]
    _check("moe_mxfp4_grouped_gemm", lib().moe_mxfp4_grouped_gemm(
        _ptr(a_q), _rowstride(a_q), _ptr(a_s), _rowstride(a_s),
        _ptr(w4), *_w_strides(w4, w_packed), _ptr(w4_s), w4_s.stride(0), w4_s.stride(1),
        E, N, K, _ptr(expert_offsets), m_rows, block_m, _ptr(out), _dt(out), _rowstride(out), _stream(stream)))


def mxfp4_grouped_gemm_act_quant(a_q, a_s, w4, w4_s, expert_offsets, out_q, out_s, m_rows=None, block_m=0,
                                 act=1, w_packed=False, stream=None):
    """bf8_grouped_gemm_act_quant with MXFP4 gate/up weights w4 [E, 2I, K/2], w4_s [E, 2I, K/32]."""
    E, N, K = _mxfp4_weights(w4, w4_s)
    if m_rows is None:
        m_rows = out_q.shape[0]
    _check("moe_mxfp4_grouped_gemm_act_quant", lib().moe_mxfp4_grouped_gemm_act_quant(
        _ptr(a_q), _rowstride(a_q), _ptr(a_s), _rowstride(a_s),
        _ptr(w4), *_w_strides(w4, w_packed), _ptr(w4_s), w4_s.stride(0), w4_s.stride(1),
        E, N // 2, K, _ptr(expert_offsets), m_rows, block_m, act, _ptr(out_q), _rowstride(out_q),
        _ptr(out_s), _rowstride(out_s), _stream(stream)))


def topk_reduce(y, slot_ids, weights, out, route_rows=None, stream=None):
    """out[t] = bf16(sum over active j of weights[t,j] * y[row(t,j)])."""
    T, topk = slot_ids.shape
    H = out.shape[1]
    _check("moe_topk_reduce", lib().moe_topk_reduce(
        _ptr(y), _dt(y), _rowstride(y), _ptr(slot_ids), _ptr(route_rows), _ptr(weights), T, topk, H,
        _ptr(out), _rowstride(out), _stream(stream)))


def fused_decode_workspace_size(T, H, I, topk) -> int:
    return lib().moe_fused_decode_workspace_size(T, H, I, topk)


def fused_decode_workspace_layout(T, H, I, topk):
    offs = (ctypes.c_int64 * 7)()
    _check("moe_fused_decode_workspace_layout", lib().moe_fused_decode_workspace_layout(T, H, I, topk, offs))
    return dict(zip(("c1", "h", "aq", "as", "c2", "ctl", "total"), list(offs)))


def fused_decode_workspace(T, H, I, topk, device="cuda", stream=None) -> torch.Tensor:
    """Allocates (with torch) and initializes a workspace for moe_fused_decode."""
    size = fused_decode_workspace_size(T, H, I, topk)
    if size == 0:
        raise MoeError("moe_fused_decode_workspace_size", MOE_ERR_SHAPE)
    ws = torch.empty(size, dtype=torch.uint8, device=device)
    _check("moe_fused_decode_workspace_init", lib().moe_fused_decode_workspace_init(
        _ptr(ws), size, T, H, I, topk, _stream(stream)))
    return ws


def fused_decode(x, slot_ids, weights, w13_q, w13_s, w2_q, w2_s, workspace, out, act=1, stream=None):
    """One routed-expert decode step: x [T, H] bf16 -> out [T, H] bf16."""
    T, H = x.shape
    topk = slot_ids.shape[1]
    S = w13_q.shape[0]
    I = w13_q.shape[1] // 2
    for t in (x, slot_ids, weights, w13_q, w13_s, w2_q, w2_s, out):
        assert t.is_contiguous()
    _check("moe_fused_decode", lib().moe_fused_decode(
        _ptr(x), T, H, I, topk, act, _ptr(slot_ids), _ptr(weights), S, _ptr(w13_q), _ptr(w13_s), _ptr(w2_q), _ptr(w2_s),
        _ptr(workspace), workspace.numel(), _ptr(out), _stream(stream)))


def fused_decode_noalloc(x, slot_ids, weights, w13_q, w13_s, w2_q, w2_s, out, act=1, stream=None):
    """fused_decode on the library's fixed device scratch (no workspace, nothing allocated)."""
    T, H = x.shape
    topk = slot_ids.shape[1]
    S = w13_q.shape[0]
    I = w13_q.shape[1] // 2
    for t in (x, slot_ids, weights, w13_q, w13_s, w2_q, w2_s, out):
        assert t.is_contiguous()
    _check("moe_fused_decode_noalloc", lib().moe_fused_decode_noalloc(
        _ptr(x), T, H, I, topk, act, _ptr(slot_ids), _ptr(weights), S, _ptr(w13_q), _ptr(w13_s), _ptr(w2_q),
        _ptr(w2_s), _ptr(out), _stream(stream)))


def route_prep(logits, topk, stream=None):
    """Top-k routing and the (expert, token)-ordered route maps of a prefill step.

    logits: [T, E] float32 on the GPU.  Returns (expert_ids [T,topk] i32, weights [T,topk] f32,
    dst2src [T*topk] i32, route_rows [T*topk] i32, expert_offsets [E+1] i32)."""
    T, E = logits.shape
    dev = logits.device
    ids = torch.empty((T, topk), dtype=torch.int32, device=dev)
    w = torch.empty((T, topk), dtype=torch.float32, device=dev)
    d2s = torch.empty(T * topk, dtype=torch.int32, device=dev)
    rr = torch.empty(T * topk, dtype=torch.int32, device=dev)
    offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
    size = lib().moe_route_prep_workspace_size(T, E)
    if size == 0:
        raise MoeError("moe_route_prep_workspace_size", MOE_ERR_SHAPE)
    ws = torch.empty(size, dtype=torch.uint8, device=dev)
    _check("moe_route_prep", lib().moe_route_prep(
        _ptr(logits), _rowstride(logits), T, E, topk, _ptr(ids) if T else None, _ptr(w) if T else None,
        _ptr(d2s) if T else None, _ptr(rr) if T else None, _ptr(offs), _ptr(ws), size, _stream(stream)))
    return ids, w, d2s, rr, offs
