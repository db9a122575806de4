/*
 * moe_routed.h -- C ABI of the routed-expert hot path of a block-FP8
 * Mixture-of-Experts layer, for AMD Instinct MI355X (gfx950).
 *
 * Library: libmoe_routed.so (moe_routed_expert_amd/libmoe_routed.so).
 *
 * Number formats used by every entry point:
 *   - fp8 means the OCP e4m3fn byte (bias 7, max 448, 0x7F/0xFF NaN);
 *   - an activation row of K fp8 bytes carries ceil(K/128) fp32 scales, one
 *     per 1x128 group; a weight matrix [N][K] carries one fp32 scale per
 *     128x128 block, laid out [ceil(N/128)][ceil(K/128)];
 *   - the dequantized value is code * scale, and a scale is amax/448.
 *
 * Sources ("page" = one of the descriptions this library is built from):
 *   [inactive]  "perf(moe): skip inactive block-fp8 decode routes", opening
 *               section and Validation: a negative slot id marks an inactive
 *               route; its GEMM output tile is written as zero and nothing
 *               else of it is read; launch shapes stay fixed and the same
 *               captured graph must serve all-active, mixed and all-inactive
 *               steps with inputs changed in place.
 *   [gather]    "[MoE] Gather the cutlass MoE activation and its scales in
 *               one launch", Motivation / Modifications / Accuracy Tests:
 *               one pass over a dst2src map copies the fp8 row bytes and
 *               the row's k//128 fp32 scales; row bases in 64-bit; tails
 *               masked (k = 896 has 7 scale groups); an empty map is a no-op.
 *   [tile]      "perf(dsfp4): pick the grouped-prefill tile from route
 *               density on sm_89", The Hopper assumption / Measurements /
 *               What is not the mechanism / Testing: the prefill kernel's
 *               expert weights are FP4 and dequantizing them bounds it; the
 *               best M tile follows rows per expert (16, 32, 128 at about 6,
 *               24, 96 rows) and BLOCK_K is 128; the picker is a pure
 *               function of route and expert counts.
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     allocates, frees and copies nothing, never synchronizes the stream and
 *     never reads device data on the host, so every call can be captured into
 *     a hipGraph.  `stream` is a hipStream_t (NULL = the null stream).
 *   - Sizes and strides are in ELEMENTS of the buffer they describe (bytes for
 *     fp8 buffers, floats for scale buffers), 64-bit.
 *   - Every output element named in a call is overwritten; outputs never need
 *     to be cleared by the caller.
 *   - Argument checks are host-side and look at scalars and pointers only.
 *     Device contents are not validated: a slot id >= the number of slots or
 *     offsets that disagree with m_rows are undefined behaviour (the gather's
 *     map entries are bounds-checked on the device, see below).
 *   - A call with no work (zero rows) returns MOE_OK without launching.
 *   - Results are deterministic: no floating-point atomics are used.
 */
#ifndef MOE_ROUTED_H
#define MOE_ROUTED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,      /* a required pointer is NULL */
    MOE_ERR_SHAPE = -2,     /* a size, stride, mode or enum is out of range */
    MOE_ERR_DTYPE = -3,     /* unsupported element type for this argument */
    MOE_ERR_WORKSPACE = -4, /* workspace too small */
    MOE_ERR_ALIGN = -5,     /* a pointer or stride breaks the required alignment */
    MOE_ERR_HIP = -6,       /* the HIP runtime rejected the launch */
    MOE_ERR_SCRATCH = -7    /* moe_fused_decode_noalloc: the step needs more than its fixed scratch */
} moe_status;

typedef enum { MOE_BF16 = 0, MOE_F32 = 1, MOE_F16 = 2 } moe_dtype;
/* Gated activations h = act(gate) * up: the five GLU variants (SwiGLU, GEGLU with the exact GELU,
 * ReGLU, GLU, bilinear); IDENTITY quantizes its input as is. */
typedef enum {
    MOE_ACT_IDENTITY = 0,
    MOE_ACT_SILU_MUL = 1,     /* (g / (1 + exp(-g))) * u */
    MOE_ACT_GELU_MUL = 2,     /* (g * (0.5 * (1 + erf(g / sqrt 2)))) * u */
    MOE_ACT_RELU_MUL = 3,     /* (g > 0 ? g : +0) * u */
    MOE_ACT_SIGMOID_MUL = 4,  /* (1 / (1 + exp(-g))) * u */
    MOE_ACT_MUL = 5           /* g * u */
} moe_act;
typedef enum { MOE_MODE_GROUPED = 0, MOE_MODE_SLOT = 1 } moe_gemm_mode;
/* Passed as the weight row stride (w_stride_n, w4_stride_n) of the grouped-mode GEMMs: the weights are
 * in the packed order that moe_pack_weights writes, and the expert stride keeps its meaning. */
#define MOE_W_PACKED (-1)

/* Version of this header the library was built from (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* Human-readable text for a moe_status value (static storage). */
const char* moe_status_string(int status);

/* Text of the last HIP error seen by a launch on the calling host thread (thread-local storage). */
const char* moe_last_hip_error(void);

/*
 * moe_gather_rows_scales  [gather]
 *   for i in [0, n_dst):  src = dst2src[i]
 *     src >= 0: dst_q[i, 0:k] = src_q[src, 0:k]   (bytes, never decoded)
 *               dst_s[i, 0:g] = src_s[src, 0:g]   (raw 32-bit words)
 *     src <  0 or src >= n_src: dst_q[i, 0:k] = 0 and dst_s[i, 0:g] = +0.0
 *       (the page defines in-range entries only; an out-of-range entry is
 *       caught on the device and reads no source row)
 *   src_q  [n_src][src_q_stride] bytes;  src_s [n_src][src_s_stride] fp32
 *   dst_q  [n_dst][dst_q_stride] bytes;  dst_s [n_dst][dst_s_stride] fp32
 *   g is passed explicitly (normally ceil(k/128)); g == 0 reads and writes no
 *   scale word, so src_s and dst_s may then be NULL.  Strides >= widths.
 *   Alignment: none required; 16-byte aligned rows take the vector path.
 *   n_dst == 0 returns MOE_OK with no launch.
 */
int moe_gather_rows_scales(const void* src_q, int64_t src_q_stride,
                           const float* src_s, int64_t src_s_stride,
                           int64_t n_src, int64_t k, int64_t g,
                           const int32_t* dst2src, int64_t n_dst,
                           void* dst_q, int64_t dst_q_stride,
                           float* dst_s, int64_t dst_s_stride,
                           void* stream);

/*
 * moe_act_quant  -- per-row 1x128 fp8 quantization, optionally of a gated activation
 *   act = MOE_ACT_IDENTITY: v = in[r, c] for c in [0, n)
 *   gated acts (moe_act 1..5): in row is [gate(0:n) | up(n:2n)], v = act(gate) * up in fp32, with the
 *   expressions of moe_act ([inactive] Validation lists five activations; the five GLU variants are
 *   taken as them)
 *   per group of 128 columns of v (last group may be shorter):
 *     s = max|v| / 448 (fp32, correctly rounded);  q = (s == 0) ? 0x00 : e4m3_rne(v / s)
 *   in    [rows][in_stride] of in_dt (MOE_BF16, MOE_F16 or MOE_F32)
 *   out_q [rows][q_stride] bytes, out_s [rows][s_stride] fp32 (ceil(n/128) used)
 *   Inputs must be finite.  IDENTITY mode is bit-exact with a correctly
 *   rounded division and round-to-nearest-even e4m3 encoding, and so are
 *   RELU_MUL and MUL (exact fp32 products).  SILU and SIGMOID take the
 *   sigmoid as rcp(1 + exp2(-g * log2 e)) from the hardware exp2 and
 *   reciprocal (each within 1 ulp; 0 once 1 + e^-g exceeds 2^126, i.e. for
 *   g below about -87.3), GELU the device erff, so their values differ from
 *   the fp32 libm expressions of moe_act by a few ulp and a code may differ
 *   by one e4m3 step, rarely.  An all-zero group gives s = +0 and q = 0x00 (a zeroed
 *   inactive-route tile stays zero, [inactive] opening section).
 */
int moe_act_quant(const void* in, int in_dt, int64_t in_stride, int64_t rows, int64_t n, int act,
                  uint8_t* out_q, int64_t q_stride, float* out_s, int64_t s_stride, void* stream);

/*
 * moe_pick_block_m  [tile]
 *   The M tile of the grouped GEMM for `routes` routed rows over `experts`
 *   experts.  As on the page, the tile grows with rows per expert; the
 *   thresholds are MI355X's (a sweep of every tile at 6, 24, 48 and 96 rows
 *   per expert): with r = ceil(routes/experts), r <= 8 gives 16, r <= 64
 *   gives 64, larger r gives 128.  Pure function of its two arguments;
 *   returns 16 when either is <= 0.
 */
int moe_pick_block_m(int64_t routes, int64_t experts);

/*
 * moe_grouped_block_m  [tile]
 *   The M tile the grouped-mode GEMMs take when called with block_m = 0, for
 *   `routes` rows over `experts` experts, K, the weight format (mxfp4 = 0:
 *   block-FP8, 1: MXFP4), the bank layout (packed = 1: MOE_W_PACKED) and the
 *   form (fused = 1: the gate/up + requant entry points).  It refines
 *   moe_pick_block_m with an MI355X sweep of every tile at 48 to 24576 routes
 *   over 256 experts; with r = ceil(routes/experts):
 *     block-FP8 row-major: 128 (plain), moe_pick_block_m (fused);
 *     block-FP8 packed:    r <= 8: 16; r <= 64: 128 if K <= 2048, else 64; 128;
 *     MXFP4:               r <= 8: 16; r <= 64: 32 (packed) or 64; 128, or 64
 *                          for packed banks with K > 2048.
 *   Pure function; 16 when routes or experts is <= 0.
 */
int moe_grouped_block_m(int64_t routes, int64_t experts, int64_t K, int mxfp4, int packed, int fused);

/*
 * moe_bf8_grouped_gemm  -- block-FP8 GEMM for the gate/up and the down projections
 *   ("bf8" = block-FP8 with e4m3 operands.)
 *   out[r, n] = sum_kb ( sum_{k in kb} A[ar, k] * W[e, n, k] ) * a_s[ar, kb] * w_s[e, n/128, kb]
 *   with fp8 products exact; the 128 products of a K block are summed by the fp8 MFMA, which keeps
 *   about 13-14 significant bits of that sum (error below 2^-12 of the block's sum |products|), and
 *   the scaled block sums are accumulated in fp32.
 *   a_q  [*][a_stride] fp8,   a_s [*][a_s_stride] fp32 (K/128 used)
 *   w_q  [n_experts] x [N][K] fp8: element (e,n,k) at e*w_stride_e + n*w_stride_n + k
 *   w_s  fp32: block (e,nb,kb) at e*w_s_stride_e + nb*w_s_stride_n + kb
 *   out  [m_rows][out_stride] of out_dt (MOE_BF16, MOE_F16 or MOE_F32)
 *   mode MOE_MODE_GROUPED (prefill, [tile]): rows sorted by expert; rows
 *        [expert_offsets[e], expert_offsets[e+1]) use expert e and A row r;
 *        expert_offsets is a DEVICE int32 array of n_experts+1 entries with
 *        expert_offsets[0] = 0 and expert_offsets[n_experts] <= m_rows (rows
 *        beyond it are left untouched).  block_m = 0 picks the M tile with
 *        moe_grouped_block_m (moe_pick_block_m's density rule, refined per
 *        weight format and bank layout); 16, 32, 64 or 128 forces it.
 *        The kernel is persistent (one workgroup per resident slot); tiles
 *        come from the device offsets, clamped to [0, m_rows].
 *   mode MOE_MODE_SLOT (decode, [inactive]): row r uses slot slot_ids[r]
 *        (DEVICE int32 [m_rows]) and A row r / a_row_div; a negative slot
 *        writes a +0 output row and reads no A, W or scales of that row.
 *        Meant for decode-sized row counts (every row streams its expert).
 *   Requirements: K % 128 == 0, N % 16 == 0, m_rows <= 2^31 - 1 (every
 *   grouped entry point: MOE_ERR_SHAPE beyond); w_q, a_q and their strides
 *   16-byte aligned (MOE_ERR_ALIGN otherwise).  Grouped mode also needs
 *   N % 128 == 0, 1 <= n_experts <= 1024 and K <= 8192 (a tile keeps all its
 *   K-block scales in LDS); MOE_ERR_SHAPE otherwise.  n_experts == 0 with NULL
 *   w_q/w_s is allowed in slot mode (an empty bank: every slot must be < 0).
 *   Grouped mode also takes a packed bank (moe_pack_weights with step_bytes
 *   128): w_stride_n = MOE_W_PACKED, w_stride_e >= N*K when n_experts > 1.
 */
int moe_bf8_grouped_gemm(const uint8_t* a_q, int64_t a_stride, const float* a_s, int64_t a_s_stride,
                         const uint8_t* w_q, int64_t w_stride_e, int64_t w_stride_n,
                         const float* w_s, int64_t w_s_stride_e, int64_t w_s_stride_n,
                         int64_t n_experts, int64_t N, int64_t K,
                         int mode, const int32_t* expert_offsets, const int32_t* slot_ids,
                         int64_t m_rows, int64_t a_row_div, int32_t block_m,
                         void* out, int out_dt, int64_t out_stride, void* stream);

/*
 * moe_bf8_grouped_gemm_act_quant  -- the prefill gate/up GEMM with the gated
 *   activation and its requant in the epilogue  [tile] [inactive]
 *   The gate/up GEMM of grouped (prefill) mode followed by moe_act_quant with
 *   a gated act (moe_act 1..5), in one launch: with c1 the fp32 GEMM result of
 *   moe_bf8_grouped_gemm (N = 2I, W13 rows 0..I-1 gate, I..2I-1 up), never
 *   stored, h[r, c] = act(g) * u with g = c1[r, c], u = c1[r, I + c] (fp32,
 *   the moe_act expressions), then per 1x128 group s = amax/448 and
 *   q = e4m3(h/s) as in moe_act_quant (q = 0x00, s = +0 when amax = 0).
 *   a_q, a_s, w_q, w_s, expert_offsets, m_rows, block_m: as moe_bf8_grouped_gemm
 *   in MOE_MODE_GROUPED with N = 2I.
 *   out_q [m_rows][q_stride] fp8 (I used), out_s [m_rows][s_stride] fp32 (I/128
 *   used).  The results equal moe_bf8_grouped_gemm with MOE_F32 output followed
 *   by moe_act_quant with the same act on it, bit for bit.
 *   Requirements: I % 128 == 0, K % 128 == 0, K <= 8192, 1 <= n_experts <=
 *   1024, alignment as moe_bf8_grouped_gemm; m_rows == 0 launches nothing.
 *   w_stride_n = MOE_W_PACKED takes a packed bank as moe_bf8_grouped_gemm.
 */
int moe_bf8_grouped_gemm_act_quant(const uint8_t* a_q, int64_t a_stride, const float* a_s, int64_t a_s_stride,
                                   const uint8_t* w_q, int64_t w_stride_e, int64_t w_stride_n,
                                   const float* w_s, int64_t w_s_stride_e, int64_t w_s_stride_n,
                                   int64_t n_experts, int64_t I, int64_t K, const int32_t* expert_offsets,
                                   int64_t m_rows, int32_t block_m, int act, uint8_t* out_q, int64_t q_stride,
                                   float* out_s, int64_t s_stride, void* stream);

/*
 * moe_mxfp4_grouped_gemm  -- the grouped (prefill) GEMM with FP4 expert weights
 *   [tile]: the routed-expert prefill kernel of that page takes FP4 weights and
 *   is limited by dequantizing them.  The page does not fix the FP4 format;
 *   the one taken is OCP MXFP4: E2M1 elements (+-{0, 0.5, 1, 1.5, 2, 3, 4, 6}),
 *   two per byte with K element 2i in the low nibble, and one E8M0 scale byte
 *   (2^(e-127)) per 32 consecutive K elements.
 *   out[r, n] = sum_kb ( sum_{k in kb} A[r, k] * W[e, n, k] * 2^(w4_s[e, n, k/32] - 127) ) * a_s[r, kb]
 *   with products exact, each 128-wide K block (kb) summed by the MFMA as in moe_bf8_grouped_gemm
 *   and the scaled block sums accumulated in fp32.
 *   a_q, a_s: fp8 activations with 1x128 fp32 scales, as moe_bf8_grouped_gemm.
 *   w4   [n_experts] x [N][K/2] bytes: the byte of (e, n, k) is at
 *        e*w4_stride_e + n*w4_stride_n + k/2 (strides in BYTES).
 *   w4_s [n_experts] x [N][K/32] E8M0 bytes: block (e, n, k/32) at
 *        e*w4s_stride_e + n*w4s_stride_n + k/32 (strides in bytes).
 *   expert_offsets, m_rows, block_m, out, out_dt, out_stride: as
 *   moe_bf8_grouped_gemm in MOE_MODE_GROUPED.
 *   Requirements: N % 128 == 0, K % 128 == 0, K <= 8192, 1 <= n_experts <=
 *   1024 (MOE_ERR_SHAPE); a_q, w4 and their strides 16-byte aligned, w4_s and
 *   its strides 4-byte aligned (MOE_ERR_ALIGN).  A scale byte of 255 (NaN in
 *   the format) gives results this library does not define, and so do scaled
 *   products below the fp32 normal range.  m_rows == 0 launches nothing.
 *   w4_stride_n = MOE_W_PACKED takes a packed bank (moe_pack_weights with
 *   step_bytes 64), w4_stride_e >= N*K/2 when n_experts > 1; w4_s unchanged.
 */
int moe_mxfp4_grouped_gemm(const uint8_t* a_q, int64_t a_stride, const float* a_s, int64_t a_s_stride,
                           const uint8_t* w4, int64_t w4_stride_e, int64_t w4_stride_n,
                           const uint8_t* w4_s, int64_t w4s_stride_e, int64_t w4s_stride_n,
                           int64_t n_experts, int64_t N, int64_t K, const int32_t* expert_offsets,
                           int64_t m_rows, int32_t block_m, void* out, int out_dt, int64_t out_stride,
                           void* stream);

/*
 * moe_mxfp4_grouped_gemm_act_quant  -- moe_bf8_grouped_gemm_act_quant with
 *   MXFP4 gate/up weights  [tile] [inactive]
 *   c1 is the fp32 result of moe_mxfp4_grouped_gemm with N = 2I (W13 rows
 *   0..I-1 gate, I..2I-1 up), never stored; the gated activation and its
 *   1x128 requant into out_q / out_s are those of
 *   moe_bf8_grouped_gemm_act_quant.  The results equal moe_mxfp4_grouped_gemm
 *   with MOE_F32 output followed by moe_act_quant with the same act, bit for
 *   bit.  Requirements: I % 128 == 0 and the rest as moe_mxfp4_grouped_gemm.
 */
int moe_mxfp4_grouped_gemm_act_quant(const uint8_t* a_q, int64_t a_stride, const float* a_s, int64_t a_s_stride,
                                     const uint8_t* w4, int64_t w4_stride_e, int64_t w4_stride_n,
                                     const uint8_t* w4_s, int64_t w4s_stride_e, int64_t w4s_stride_n,
                                     int64_t n_experts, int64_t I, int64_t K, const int32_t* expert_offsets,
                                     int64_t m_rows, int32_t block_m, int act, uint8_t* out_q, int64_t q_stride,
                                     float* out_s, int64_t s_stride, void* stream);

/*
 * moe_pack_weights  -- an expert bank in the grouped GEMMs' operand order
 *   Not a step of the pages' method: a one-time copy of static weights into an
 *   order in which every 1 KiB load of the grouped GEMMs reads contiguous bytes
 *   (row-major weights are read as 64 bytes of each of 16 rows 4 KiB or more
 *   apart, which streams about 15 % slower on MI355X).
 *   w     [n_experts] x [N][row_bytes] bytes: byte (e, n, c) at e*w_stride_e + n*w_stride_n + c
 *         (block-FP8: row_bytes = K; MXFP4: row_bytes = K/2 nibble pairs).
 *   step_bytes: bytes of one 128-wide K block of a row: 128 (block-FP8) or 64 (MXFP4).
 *   out   packed bank, expert e at e*out_stride_e.  Within an expert, for each 16-row
 *         group g = n/16 and K step s = c/step_bytes, a block of 16*step_bytes bytes at
 *         (g*(row_bytes/step_bytes) + s)*16*step_bytes holds 16-byte pieces p = 0 ..
 *         step_bytes-1: piece p is row 16g + (p%16), bytes s*step_bytes + 64*(p/64) +
 *         16*((p%64)/16) .. +15.  The scale arrays keep their own layout.
 *   The grouped-mode GEMMs read such a bank when given w_stride_n = MOE_W_PACKED
 *   and the bank's expert stride; their results are those of the row-major bank,
 *   bit for bit.  Slot mode and the fused decode take row-major banks only.
 *   Requirements: N % 16 == 0, step_bytes 64 or 128, row_bytes % step_bytes == 0,
 *   w_stride_n >= row_bytes, w_stride_e >= N*w_stride_n and out_stride_e >=
 *   N*row_bytes when n_experts > 1 (MOE_ERR_SHAPE); w, out and every stride
 *   16-byte aligned (MOE_ERR_ALIGN).  w and out must not overlap.
 */
int moe_pack_weights(const uint8_t* w, int64_t w_stride_e, int64_t w_stride_n, int64_t n_experts, int64_t N,
                     int64_t row_bytes, int64_t step_bytes, uint8_t* out, int64_t out_stride_e, void* stream);

/*
 * moe_topk_reduce  -- routing-weighted sum over each token's top-k routes
 *   out[t, h] = bf16_rne( sum_{j = 0..topk-1, slot_ids[t,j] >= 0} weights[t,j] * y[row(t,j), h] )
 *   summed in fp32 in ascending j from +0; row(t,j) = route_rows[t*topk + j]
 *   (DEVICE int32) or t*topk + j when route_rows is NULL.  The weight of an
 *   inactive route is never read ([inactive] opening section).  A token with
 *   no active route gets +0.0.
 *   y [*][y_stride] of y_dt;  slot_ids, weights [T][topk];  out [T][out_stride] bf16.
 */
int moe_topk_reduce(const void* y, int y_dt, int64_t y_stride,
                    const int32_t* slot_ids, const int32_t* route_rows, const float* weights,
                    int64_t T, int64_t topk, int64_t H, uint16_t* out_bf16, int64_t out_stride,
                    void* stream);

/*
 * Fused decode workspace.  Layout (byte offsets written to offsets[0..6]):
 *   [0] c1   R x 2I           fp32 gate/up output (R = T*topk routes)
 *   [1] h    R x I            fp32 SiLU(gate)*up
 *   [2] aq   R x I            fp8 activation (1x128 requant of h)
 *   [3] as   R x ceil(I/128)  fp32 activation scales
 *   [4] c2   R x H            fp32 down output
 *   [5] ctl  control block: the error word and the hand-off state of the
 *            one-launch step (per-tile call counters, ready words and a
 *            tagged copy of h)
 *   [6] total size in bytes
 * Regions [0]..[4] may hold anything between calls: every call rewrites them
 * completely, and an inactive route's c1/h/aq/as/c2 rows become exact zeros
 * (h is only written when I <= 1024; wider I runs the step as four launches
 * that do not store h).  The control region must be cleared once with
 * moe_fused_decode_workspace_init before the first call and carries state
 * from call to call: a workspace serves one shape (T, H, I, topk), and calls
 * that share it must not overlap in time (e.g. on two streams without an
 * event between them).  Its first 32-bit word is the error word: nonzero
 * after a call means the step's output is not valid (its affected output
 * rows are NaN) and the workspace must be initialized again -- 1: a
 * hand-off wait gave up; 2: the workspace was
 * initialized for another (T, H, I, topk) (init writes the shape into word 1
 * of the control block, and the one-launch step checks it before it waits on
 * any hand-off word).  The library never reads the word on the host; callers
 * that need the check copy it back themselves.  Size 0 / MOE_ERR_SHAPE for
 * shapes moe_fused_decode rejects.
 */
size_t moe_fused_decode_workspace_size(int64_t T, int64_t H, int64_t I, int64_t topk);
int moe_fused_decode_workspace_layout(int64_t T, int64_t H, int64_t I, int64_t topk, int64_t offsets[7]);
int moe_fused_decode_workspace_init(void* workspace, size_t ws_bytes, int64_t T, int64_t H, int64_t I,
                                    int64_t topk, void* stream);

/*
 * moe_route_prep  -- routing prep of a prefill step  [gather] [tile]
 *   The step before the gather: the dst2src map that replicates each token's
 *   activation once per routed expert, and the expert-grouped row order of the
 *   grouped GEMM.
 *   logits   DEVICE fp32 [T][logits_stride] (E used), finite.  A NaN logit
 *   ranks as -inf so every selected id is a valid expert, but the weights of
 *   such a token are then unspecified.
 *   For each token: the topk experts with the largest logits in descending order
 *   (ties: lower expert index), and weights w_j = exp(l_j - l_max) /
 *   sum_{i in top-k} exp(l_i - l_max), i.e. the softmax over all E experts
 *   renormalized over the top-k.
 *   expert_ids [T][topk] int32, weights [T][topk] fp32.
 *   Route maps in (expert, token) order: dst2src [T*topk] int32 (token of each
 *   sorted row), route_rows [T*topk] int32 (row of route t*topk+j, the
 *   route_rows argument of moe_topk_reduce), expert_offsets [E+1] int32 (rows
 *   of expert e are [offsets[e], offsets[e+1]), the grouped GEMM's offsets).
 *   workspace: moe_route_prep_workspace_size(T, E) bytes of DEVICE memory,
 *   16-byte aligned; no initialization needed; scratch between the three
 *   launches of one call, so overlapping calls need their own workspaces.
 *   Deterministic (integer counting only).
 *   Requirements: 1 <= E <= 1024, 1 <= topk <= min(E, 64), T * topk < 2^31.
 *   T == 0 launches one small kernel that writes E + 1 zero offsets (the one
 *   exception to "no work, no launch").
 */
size_t moe_route_prep_workspace_size(int64_t T, int64_t E);
int moe_route_prep(const float* logits, int64_t logits_stride, int64_t T, int64_t E, int64_t topk,
                   int32_t* expert_ids, float* weights, int32_t* dst2src, int32_t* route_rows,
                   int32_t* expert_offsets, void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_fused_decode  -- one decode step of the routed experts  [inactive]
 *   x (T x H bf16) -> 1x128 fp8 quant -> gate/up GEMM per route (slot mode,
 *   A row = token) -> act(gate)*up + 1x128 requant -> down GEMM per route
 *   -> routing-weighted top-k reduce -> out (T x H bf16).  act: a gated
 *   moe_act (1..5), as in moe_act_quant ([inactive] Validation: five
 *   activations).
 *   slot_ids, weights: DEVICE [T][topk]; slot < 0 = inactive route (zero
 *   c1/act/c2 tiles, no reads of its weights, scales or routing weight).
 *   w13_q [n_slots][2I][H] fp8 (gate rows 0..I-1, up rows I..2I-1), contiguous;
 *   w13_s [n_slots][ceil(2I/128)][ceil(H/128)] fp32;  w2_q [n_slots][H][I];
 *   w2_s [n_slots][ceil(H/128)][ceil(I/128)].
 *   Requirements: H % 128 == 0, I % 128 == 0, H and I <= 65536, 1 <= topk <= 64,
 *   T * topk <= 65535; 16-byte aligned weights and workspace, 4-byte aligned x.
 *   Launch shapes depend on (T, H, I, topk) and the device only, so one
 *   captured graph serves any slot/weight/x contents.  For small steps
 *   (H <= 2048, I <= 1024, I/8 even or a multiple of 3) whose workgroups all
 *   fit on the device at once, the step is a single launch in which gate/up
 *   tiles hand h to the down tiles through the workspace's control block;
 *   otherwise it is two launches (I <= 1024) or four (wider I).
 */
int moe_fused_decode(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t I, int64_t topk, int act,
                     const int32_t* slot_ids, const float* weights, int64_t n_slots,
                     const uint8_t* w13_q, const float* w13_s,
                     const uint8_t* w2_q, const float* w2_s,
                     void* workspace, size_t ws_bytes, uint16_t* out_bf16, void* stream);

/*
 * moe_fused_decode_noalloc  -- moe_fused_decode without a caller workspace
 *   For callers that cannot allocate device memory at all: code under hipGraph
 *   capture, tight serving loops, harnesses that forbid allocation.  Arguments
 *   and results are those of moe_fused_decode minus the workspace; the step
 *   runs the same kernels on a fixed device array inside the library
 *   (4 MiB, 256-byte aligned; each GPU the library runs on holds its own copy
 *   until the process ends).  The call allocates and frees nothing.
 *   Limit: steps whose workspace (moe_fused_decode_workspace_size) exceeds
 *   4 MiB return MOE_ERR_SCRATCH without launching; e.g. up to 16 tokens at
 *   H = 4096, I = 1024, top-8.
 *   State: the array keeps the last call's contents.  The first call on a
 *   device, and every call whose (T, H, I, topk) differs from that device's
 *   previous call, first clears the control block with a fill kernel on
 *   `stream`; later calls of the same shape continue its call counters, as
 *   with an initialized workspace.  All calls on one GPU share the array, so
 *   calls that overlap in time on one GPU (two streams, two host threads
 *   without ordering) race and give undefined results.  The device is the
 *   current HIP device.
 *   Errors: as moe_fused_decode, plus MOE_ERR_SCRATCH; if a hand-off wait
 *   ever gives up, that step's affected output rows are NaN.
 */
int moe_fused_decode_noalloc(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t I, int64_t topk, int act,
                             const int32_t* slot_ids, const float* weights, int64_t n_slots,
                             const uint8_t* w13_q, const float* w13_s,
                             const uint8_t* w2_q, const float* w2_s,
                             uint16_t* out_bf16, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_ROUTED_H */
