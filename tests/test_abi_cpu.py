"""CPU-only checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments on the host before any launch."""
import ctypes
import json
import os
import re

import pytest

import moe_routed_expert_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_routed.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("moe_gather_rows_scales", "moe_bf8_grouped_gemm", "moe_act_quant", "moe_topk_reduce",
                 "moe_fused_decode", "moe_pick_block_m", "moe_status_string"):
        assert want in names


def test_library_exports_every_declared_symbol():
    L = m.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(declared_functions()) == set(m.EXPORTS)


def test_abi_version_and_status_strings():
    assert m.abi_version() == 1
    L = m.lib()
    for st in (0, -1, -2, -3, -4, -5, -6, -7):
        assert L.moe_status_string(st).decode() not in ("", "unknown status")
    assert L.moe_status_string(7).decode() == "unknown status"


def test_pick_block_m_follows_density_like_the_page():
    """The page (sm_89) found the best M tile tracks rows per expert (16, 32, 128 at 6, 24, 96 rows,
    tests/golden/tile_picker_density.json).  The picker keeps that rule -- a pure, non-decreasing
    function of rows per expert -- with MI355X's own thresholds from a sweep of every tile: 16 at 6
    rows per expert, 64 at 24 (and 48), 128 at 96, so the ends agree with the page and the middle
    tile is 64 rather than 32."""
    spec = json.load(open(os.path.join(ROOT, "tests", "golden", "tile_picker_density.json")))
    mi355x = {6: 16, 24: 64, 96: 128}
    prev = 0
    for c in spec["cases"]:
        bm = m.pick_block_m(c["routes"], spec["experts"])
        assert bm == mi355x[c["rows_per_expert"]], c
        assert bm >= prev
        prev = bm
    assert [m.pick_block_m(c["routes"], spec["experts"]) for c in spec["cases"]][::2] == \
        [c["block_m"] for c in spec["cases"]][::2]          # the page's two ends
    last = 0
    for r in range(0, 100000, 97):
        bm = m.pick_block_m(r, 256)
        assert bm in (16, 32, 64, 128) and bm >= last
        last = bm
    assert m.pick_block_m(0, 256) == 16 and m.pick_block_m(10, 0) == 16
    assert m.pick_block_m(256 * 48, 256) == 64 and m.pick_block_m(256 * 1000, 256) == 128


P = ctypes.c_void_p
FAKE = P(0x1000)       # never dereferenced: every call below fails validation first


def gemm(**kw):
    a = dict(a_q=FAKE, a_stride=256, a_s=FAKE, a_s_stride=2, w_q=FAKE, w_stride_e=256 * 256, w_stride_n=256,
             w_s=FAKE, w_s_stride_e=4, w_s_stride_n=2, n_experts=4, N=256, K=256, mode=1, expert_offsets=FAKE,
             slot_ids=FAKE, m_rows=8, a_row_div=1, block_m=0, out=FAKE, out_dt=1, out_stride=256, stream=None)
    a.update(kw)
    return m.lib().moe_bf8_grouped_gemm(*a.values())


def test_gemm_argument_checks():
    assert gemm(K=200) == m.MOE_ERR_SHAPE          # K % 128
    assert gemm(N=200) == m.MOE_ERR_SHAPE          # N % 16
    assert gemm(mode=5) == m.MOE_ERR_SHAPE
    assert gemm(out_dt=9) == m.MOE_ERR_DTYPE
    assert gemm(m_rows=0) == m.MOE_OK              # no work, no launch
    assert gemm(out=None) == m.MOE_ERR_NULL
    assert gemm(w_q=None) == m.MOE_ERR_NULL
    assert gemm(slot_ids=None) == m.MOE_ERR_NULL
    assert gemm(a_row_div=0) == m.MOE_ERR_SHAPE
    assert gemm(w_q=P(0x1001)) == m.MOE_ERR_ALIGN
    assert gemm(a_stride=264, w_stride_n=264, w_stride_e=264 * 256) == m.MOE_ERR_ALIGN
    assert gemm(w_stride_n=128) == m.MOE_ERR_SHAPE  # stride < K
    assert gemm(out_stride=100) == m.MOE_ERR_SHAPE
    assert gemm(mode=0, expert_offsets=None) == m.MOE_ERR_NULL
    assert gemm(mode=0, N=144) == m.MOE_ERR_SHAPE  # grouped mode needs N % 128
    assert gemm(mode=0, block_m=48) == m.MOE_ERR_SHAPE
    assert gemm(mode=0, n_experts=0, w_q=None, w_s=None) == m.MOE_ERR_SHAPE
    big_k = dict(K=8320, a_stride=8320, a_s_stride=65, w_stride_n=8320, w_stride_e=8320 * 256, w_s_stride_n=65,
                 w_s_stride_e=2 * 65)
    assert gemm(mode=0, **big_k) == m.MOE_ERR_SHAPE          # grouped mode keeps K/128 <= 64 scales per tile
    assert gemm(mode=0, n_experts=1025, **big_k) == m.MOE_ERR_SHAPE
    # more rows than an int holds: rejected before any row count is narrowed (both modes)
    assert gemm(m_rows=2 ** 31) == m.MOE_ERR_SHAPE
    assert gemm(mode=0, m_rows=2 ** 31 + 5) == m.MOE_ERR_SHAPE
    L = m.lib()
    assert L.moe_bf8_grouped_gemm_act_quant(FAKE, 256, FAKE, 2, FAKE, 256 * 256, 256, FAKE, 4, 2, 4, 128, 256, FAKE,
                                            2 ** 31, 0, 1, FAKE, 128, FAKE, 1, None) == m.MOE_ERR_SHAPE


def test_gather_act_reduce_argument_checks():
    L = m.lib()
    # empty map: OK without launching, even with NULL buffers
    assert L.moe_gather_rows_scales(None, 0, None, 0, 0, 7168, 56, None, 0, None, 0, None, 0, None) == m.MOE_OK
    assert L.moe_gather_rows_scales(FAKE, 16, FAKE, 1, 4, 32, 1, None, 8, FAKE, 32, FAKE, 1, None) == m.MOE_ERR_NULL
    assert L.moe_gather_rows_scales(FAKE, 16, FAKE, 1, 4, 32, 1, FAKE, 8, FAKE, 32, FAKE, 1, None) == m.MOE_ERR_SHAPE
    assert L.moe_gather_rows_scales(FAKE, 32, FAKE, 1, 0, 32, 1, FAKE, 8, FAKE, 32, FAKE, 1, None) == m.MOE_ERR_SHAPE
    assert L.moe_act_quant(FAKE, 7, 256, 4, 256, 0, FAKE, 256, FAKE, 2, None) == m.MOE_ERR_DTYPE
    assert L.moe_act_quant(FAKE, 0, 256, 4, 256, 6, FAKE, 256, FAKE, 2, None) == m.MOE_ERR_SHAPE
    assert L.moe_act_quant(FAKE, 0, 256, 4, 256, 1, FAKE, 256, FAKE, 2, None) == m.MOE_ERR_SHAPE  # SILU needs 2n
    assert L.moe_act_quant(FAKE, 0, 256, 0, 256, 0, None, 256, None, 2, None) == m.MOE_OK
    assert L.moe_act_quant(FAKE, 0, 256, 4, 256, 0, None, 256, FAKE, 2, None) == m.MOE_ERR_NULL
    assert L.moe_topk_reduce(FAKE, 1, 64, FAKE, None, FAKE, 4, 8, 128, FAKE, 128, None) == m.MOE_ERR_SHAPE
    assert L.moe_topk_reduce(FAKE, 5, 128, FAKE, None, FAKE, 4, 8, 128, FAKE, 128, None) == m.MOE_ERR_DTYPE
    assert L.moe_topk_reduce(FAKE, 1, 128, FAKE, None, FAKE, 0, 8, 128, FAKE, 128, None) == m.MOE_OK


def test_fused_decode_workspace_and_checks():
    L = m.lib()
    lay = m.fused_decode_workspace_layout(1, 2048, 768, 8)
    assert lay["c1"] == 0
    assert lay["h"] >= 8 * 1536 * 4 and lay["aq"] >= lay["h"] + 8 * 768 * 4 and lay["as"] >= lay["aq"] + 8 * 768
    assert lay["c2"] >= lay["as"] + 8 * 6 * 4 and lay["ctl"] >= lay["c2"] + 8 * 2048 * 4
    assert lay["total"] == m.fused_decode_workspace_size(1, 2048, 768, 8)
    assert all(v % 256 == 0 for v in lay.values())
    assert m.fused_decode_workspace_size(1, 2000, 768, 8) == 0          # H % 128
    assert m.fused_decode_workspace_size(1, 2 ** 31, 768, 8) == 0       # H beyond 65536
    assert m.fused_decode_workspace_size(1, 2048, 65536 + 128, 8) == 0  # I beyond 65536
    assert m.fused_decode_workspace_size(1, 2048, 768, 0) == 0          # topk >= 1
    size = lay["total"]
    args = [FAKE, 1, 2048, 768, 8, 1, FAKE, FAKE, 64, FAKE, FAKE, FAKE, FAKE, FAKE, size, FAKE, None]
    a = list(args); a[14] = size - 1
    assert L.moe_fused_decode(*a) == m.MOE_ERR_WORKSPACE
    a = list(args); a[13] = P(0x1008)
    assert L.moe_fused_decode(*a) == m.MOE_ERR_ALIGN
    for bad_act in (0, 6):
        a = list(args); a[5] = bad_act
        assert L.moe_fused_decode(*a) == m.MOE_ERR_SHAPE
    a = list(args); a[0] = None
    assert L.moe_fused_decode(*a) == m.MOE_ERR_NULL
    a = list(args); a[2] = 2000
    assert L.moe_fused_decode(*a) == m.MOE_ERR_SHAPE
    a = list(args); a[1] = 0
    assert L.moe_fused_decode(*a) == m.MOE_OK
    assert L.moe_fused_decode_workspace_init(FAKE, size - 1, 1, 2048, 768, 8, None) == m.MOE_ERR_WORKSPACE


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(m, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(m, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        m.lib()


def test_route_prep_workspace_and_checks():
    L = m.lib()
    size = L.moe_route_prep_workspace_size(4096, 256)
    assert size >= (4096 // 16) * 256 * 4 and size % 256 == 0          # a count per (16-token chunk, expert)
    assert L.moe_route_prep_workspace_size(4097, 256) > size
    assert 0 < L.moe_route_prep_workspace_size(0, 256) < size
    assert L.moe_route_prep_workspace_size(10, 0) == 0 and L.moe_route_prep_workspace_size(10, 1025) == 0
    args = [FAKE, 256, 4096, 256, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, size, None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return L.moe_route_prep(*a)

    assert call(a4=0) == m.MOE_ERR_SHAPE              # topk >= 1
    assert call(a4=65) == m.MOE_ERR_SHAPE             # topk <= 64
    assert call(a3=4, a4=5) == m.MOE_ERR_SHAPE        # topk <= E
    assert call(a3=1025) == m.MOE_ERR_SHAPE           # E <= 1024
    assert call(a1=255) == m.MOE_ERR_SHAPE            # logits stride >= E
    assert call(a0=None) == m.MOE_ERR_NULL
    assert call(a7=None) == m.MOE_ERR_NULL
    assert call(a9=None) == m.MOE_ERR_NULL
    assert call(a11=size - 1) == m.MOE_ERR_WORKSPACE
    assert call(a10=P(0x1008)) == m.MOE_ERR_ALIGN


def test_fused_gate_up_act_quant_checks():
    L = m.lib()
    args = dict(a_q=FAKE, a_stride=256, a_s=FAKE, a_s_stride=2, w_q=FAKE, w_stride_e=256 * 256, w_stride_n=256,
                w_s=FAKE, w_s_stride_e=4, w_s_stride_n=2, n_experts=4, I=128, K=256, offsets=FAKE, m_rows=8,
                block_m=0, act=1, q=FAKE, q_stride=128, s=FAKE, s_stride=1, stream=None)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return L.moe_bf8_grouped_gemm_act_quant(*a.values())

    assert call(I=200) == m.MOE_ERR_SHAPE                 # I % 128
    assert call(K=200) == m.MOE_ERR_SHAPE                 # K % 128
    assert call(K=8320, a_stride=8320, w_stride_n=8320, w_stride_e=8320 * 256, a_s_stride=65,
                w_s_stride_n=65, w_s_stride_e=2 * 65) == m.MOE_ERR_SHAPE   # K <= 8192
    assert call(n_experts=0) == m.MOE_ERR_SHAPE
    assert call(n_experts=1025) == m.MOE_ERR_SHAPE
    assert call(block_m=48) == m.MOE_ERR_SHAPE
    assert call(act=0) == m.MOE_ERR_SHAPE                 # a gated activation is required
    assert call(act=6) == m.MOE_ERR_SHAPE
    assert call(m_rows=0, q=None, s=None) == m.MOE_OK   # no work, no launch
    assert call(q=None) == m.MOE_ERR_NULL
    assert call(offsets=None) == m.MOE_ERR_NULL
    assert call(q_stride=100) == m.MOE_ERR_SHAPE
    assert call(w_stride_e=128 * 256) == m.MOE_ERR_SHAPE  # experts overlap: 2I rows of 256 each
    assert call(w_q=P(0x1008)) == m.MOE_ERR_ALIGN


def test_mxfp4_gemm_checks():
    L = m.lib()
    # K = 256: 128 weight bytes and 8 E8M0 bytes per row; N = 256 rows per expert
    args = dict(a_q=FAKE, a_stride=256, a_s=FAKE, a_s_stride=2, w4=FAKE, w4_stride_e=256 * 128, w4_stride_n=128,
                w4s=FAKE, w4s_stride_e=256 * 8, w4s_stride_n=8, n_experts=4, N=256, K=256, offsets=FAKE, m_rows=8,
                block_m=0, out=FAKE, out_dt=m.MOE_BF16, out_stride=256, stream=None)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return L.moe_mxfp4_grouped_gemm(*a.values())

    assert call(out_dt=9) == m.MOE_ERR_DTYPE
    assert call(N=200) == m.MOE_ERR_SHAPE                 # N % 128
    assert call(K=192) == m.MOE_ERR_SHAPE                 # K % 128
    assert call(K=8320, a_stride=8320, w4_stride_n=4160, w4_stride_e=4160 * 256, a_s_stride=65,
                w4s_stride_n=260, w4s_stride_e=260 * 256) == m.MOE_ERR_SHAPE   # K <= 8192
    assert call(n_experts=0) == m.MOE_ERR_SHAPE
    assert call(n_experts=1025) == m.MOE_ERR_SHAPE
    assert call(block_m=48) == m.MOE_ERR_SHAPE
    assert call(m_rows=0, out=None, w4=None) == m.MOE_OK   # no work, no launch
    assert call(out=None) == m.MOE_ERR_NULL
    assert call(w4s=None) == m.MOE_ERR_NULL
    assert call(offsets=None) == m.MOE_ERR_NULL
    assert call(out_stride=100) == m.MOE_ERR_SHAPE
    assert call(w4_stride_n=64) == m.MOE_ERR_SHAPE       # a row holds K/2 bytes
    assert call(w4s_stride_n=4) == m.MOE_ERR_SHAPE       # and K/32 scale bytes
    assert call(w4_stride_e=128 * 128) == m.MOE_ERR_SHAPE  # experts overlap
    assert call(w4s_stride_e=128 * 8) == m.MOE_ERR_SHAPE
    assert call(w4=P(0x1008)) == m.MOE_ERR_ALIGN
    assert call(w4_stride_n=136, w4_stride_e=136 * 256) == m.MOE_ERR_ALIGN
    assert call(w4s=P(0x1002)) == m.MOE_ERR_ALIGN
    assert call(w4s_stride_n=10, w4s_stride_e=10 * 256) == m.MOE_ERR_ALIGN


def test_mxfp4_fused_gate_up_act_quant_checks():
    L = m.lib()
    # I = 128: 2I = 256 W13 rows; K = 256
    args = dict(a_q=FAKE, a_stride=256, a_s=FAKE, a_s_stride=2, w4=FAKE, w4_stride_e=256 * 128, w4_stride_n=128,
                w4s=FAKE, w4s_stride_e=256 * 8, w4s_stride_n=8, n_experts=4, I=128, K=256, offsets=FAKE, m_rows=8,
                block_m=0, act=1, q=FAKE, q_stride=128, s=FAKE, s_stride=1, stream=None)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return L.moe_mxfp4_grouped_gemm_act_quant(*a.values())

    assert call(I=192) == m.MOE_ERR_SHAPE
    assert call(K=192) == m.MOE_ERR_SHAPE
    assert call(n_experts=1025) == m.MOE_ERR_SHAPE
    assert call(act=0) == m.MOE_ERR_SHAPE
    assert call(act=6) == m.MOE_ERR_SHAPE
    assert call(m_rows=0, q=None, s=None) == m.MOE_OK
    assert call(s=None) == m.MOE_ERR_NULL
    assert call(w4=None) == m.MOE_ERR_NULL
    assert call(s_stride=0) == m.MOE_ERR_SHAPE
    assert call(w4_stride_e=128 * 128) == m.MOE_ERR_SHAPE   # 2I rows per expert
    assert call(w4s=P(0x1001)) == m.MOE_ERR_ALIGN


def test_fused_decode_noalloc_checks():
    """The no-workspace decode rejects shapes beyond its fixed 4 MiB scratch and bad arguments on the host,
    before any HIP call."""
    L = m.lib()
    P = ctypes.c_void_p
    f = L.moe_fused_decode_noalloc
    args = lambda T, H, I, topk, act=1: (FAKE, T, H, I, topk, act, FAKE, FAKE, 64, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert m.fused_decode_workspace_size(32, 4096, 1024, 8) > 4 << 20
    assert f(*args(32, 4096, 1024, 8)) == m.MOE_ERR_SCRATCH
    assert m.fused_decode_workspace_size(16, 4096, 1024, 8) <= 4 << 20
    assert f(*args(1, 2048, 700, 8)) == m.MOE_ERR_SHAPE        # I % 128
    assert f(*args(1, 2048, 768, 65)) == m.MOE_ERR_SHAPE       # topk > 64
    assert f(*args(1, 2048, 768, 8, act=0)) == m.MOE_ERR_SHAPE # not a gated activation
    assert f(*args(0, 2048, 768, 8)) == m.MOE_OK               # no tokens: nothing launched


def test_pack_weights_and_packed_bank_checks():
    """moe_pack_weights validates before any launch; the grouped GEMMs take MOE_W_PACKED as a row stride
    in grouped mode only, with a packed bank's expert stride (N * row_bytes)."""
    L = m.lib()

    def pack(**kw):
        a = dict(w=FAKE, w_stride_e=256 * 256, w_stride_n=256, n_experts=4, N=256, row_bytes=256, step_bytes=128,
                 out=P(0x10000000), out_stride_e=256 * 256, stream=None)
        a.update(kw)
        return L.moe_pack_weights(*a.values())

    assert pack(step_bytes=96) == m.MOE_ERR_SHAPE
    assert pack(N=24) == m.MOE_ERR_SHAPE                      # 16-row groups
    assert pack(row_bytes=192) == m.MOE_ERR_SHAPE             # whole K steps
    assert pack(n_experts=-1) == m.MOE_ERR_SHAPE
    assert pack(n_experts=0, w=None, out=None) == m.MOE_OK   # nothing to copy, no launch
    assert pack(w=None) == m.MOE_ERR_NULL
    assert pack(out=None) == m.MOE_ERR_NULL
    assert pack(w_stride_n=128) == m.MOE_ERR_SHAPE            # row stride < row bytes
    assert pack(w_stride_e=128 * 256) == m.MOE_ERR_SHAPE      # source experts overlap
    assert pack(out_stride_e=128 * 256) == m.MOE_ERR_SHAPE    # packed experts overlap
    assert pack(w=P(0x1008)) == m.MOE_ERR_ALIGN
    assert pack(out=P(0x10000008)) == m.MOE_ERR_ALIGN
    assert pack(w_stride_n=264, w_stride_e=264 * 256) == m.MOE_ERR_ALIGN
    assert pack(out=P(0x1000 + 4096)) == m.MOE_ERR_SHAPE      # the two ranges meet
    # packed banks in the GEMMs
    assert gemm(mode=1, w_stride_n=m.MOE_W_PACKED) == m.MOE_ERR_SHAPE    # slot mode: row-major only
    assert gemm(mode=0, w_stride_n=m.MOE_W_PACKED, w_stride_e=255 * 256) == m.MOE_ERR_SHAPE   # < N*K
    assert gemm(mode=0, w_stride_n=m.MOE_W_PACKED, w_stride_e=256 * 256 + 8) == m.MOE_ERR_ALIGN
    assert gemm(mode=0, w_stride_n=-2) == m.MOE_ERR_SHAPE    # other negative strides stay invalid
    fused = dict(a_q=FAKE, a_stride=256, a_s=FAKE, a_s_stride=2, w_q=FAKE, w_stride_e=256 * 256,
                 w_stride_n=m.MOE_W_PACKED, w_s=FAKE, w_s_stride_e=4, w_s_stride_n=2, n_experts=4, I=128, K=256,
                 offsets=FAKE, m_rows=8, block_m=0, act=1, q=FAKE, q_stride=128, s=FAKE, s_stride=1, stream=None)
    a = dict(fused, w_stride_e=200 * 256)
    assert L.moe_bf8_grouped_gemm_act_quant(*a.values()) == m.MOE_ERR_SHAPE
    mx = dict(a_q=FAKE, a_stride=256, a_s=FAKE, a_s_stride=2, w4=FAKE, w4_stride_e=255 * 128,
              w4_stride_n=m.MOE_W_PACKED, w4s=FAKE, w4s_stride_e=256 * 8, w4s_stride_n=8, n_experts=4, N=256, K=256,
              offsets=FAKE, m_rows=8, block_m=0, out=FAKE, out_dt=m.MOE_BF16, out_stride=256, stream=None)
    assert L.moe_mxfp4_grouped_gemm(*mx.values()) == m.MOE_ERR_SHAPE    # < N*K/2


def test_grouped_block_m_refines_the_density_rule():
    """moe_grouped_block_m: the tile the grouped GEMMs take for block_m = 0 (a pure function)."""
    for r in (1, 6, 24, 96, 1000):
        R = 256 * r
        assert m.grouped_block_m(R, 256, 4096) == 128                                      # fp8 row-major
        assert m.grouped_block_m(R, 256, 4096, fused=True) == m.pick_block_m(R, 256)      # fp8 row-major fused
    assert [m.grouped_block_m(256 * r, 256, 4096, packed=True) for r in (8, 9, 64, 65)] == [16, 64, 64, 128]
    assert [m.grouped_block_m(256 * r, 256, 1024, packed=True) for r in (8, 9, 64, 65)] == [16, 128, 128, 128]
    assert [m.grouped_block_m(256 * r, 256, 4096, mxfp4=True) for r in (1, 8, 9, 64, 65)] == [16, 16, 64, 64, 128]
    assert [m.grouped_block_m(256 * r, 256, 4096, mxfp4=True, packed=True) for r in (8, 9, 64, 65)] == [16, 32, 32, 64]
    assert m.grouped_block_m(256 * 96, 256, 2048, mxfp4=True, packed=True) == 128    # <= 16 K steps
    assert m.grouped_block_m(256 * 96, 256, 1024, mxfp4=True, fused=True) == 128
    assert m.grouped_block_m(0, 256, 4096) == 16 and m.grouped_block_m(10, 0, 4096, mxfp4=True) == 16
