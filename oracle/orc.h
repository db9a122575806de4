/*
 * CPU oracle for the routed-expert hot path of a block-FP8 MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, obviously-correct
 * restatement of what the hot path computes.  Only the test suite, the
 * package smoke check and the CPU-baseline leg of the benchmark may load it.
 * It shares no source with the HIP library and must never be reached from
 * the product path.
 *
 * Number formats (the block-FP8 scheme the pages work in):
 *   - fp8 is OCP e4m3fn (bias 7, no infinities, 0x7F/0xFF are NaN, max 448);
 *   - activations carry one fp32 scale per 1x128 group of a row
 *     ("[MoE] Gather the cutlass MoE activation and its scales in one
 *     launch", Motivation: k // 128 fp32 scales per row of k fp8 values);
 *   - weights carry one fp32 scale per 128x128 block;
 *   - a scale is amax/448 and the dequantized value is code * scale.
 *
 * Every fp32 operation below is a separately rounded IEEE-754 operation
 * (the file is compiled with -ffp-contract=off and without fast-math).
 *
 * Status codes: 0 = ok, -2 = shape/argument error.
 */
#ifndef MOE_ORACLE_ORC_H
#define MOE_ORACLE_ORC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types for the 16-bit/32-bit float buffers the path materializes */
enum { ORC_BF16 = 0, ORC_F32 = 1, ORC_F16 = 2 };
/* gemm row-to-expert modes */
enum { ORC_MODE_GROUPED = 0, ORC_MODE_SLOT = 1 };

/* ---- scalar codecs (OCP FP8 e4m3fn; IEEE binary16; bfloat16) ---- */
float    orc_e4m3_to_f32(uint8_t code);
uint8_t  orc_f32_to_e4m3(float v);          /* RNE of clamp(v,-448,448); NaN -> 0x7F */
float    orc_bf16_to_f32(uint16_t h);
uint16_t orc_f32_to_bf16(float v);          /* RNE, NaN stays NaN */
float    orc_f16_to_f32(uint16_t h);
uint16_t orc_f32_to_f16(float v);           /* RNE, overflow -> inf */

void orc_e4m3_decode_array(const uint8_t* in, int64_t n, float* out);
void orc_e4m3_encode_array(const float* in, int64_t n, uint8_t* out);
void orc_bf16_encode_array(const float* in, int64_t n, uint16_t* out);
void orc_f16_encode_array(const float* in, int64_t n, uint16_t* out);

/* ---- O1: per-row 1x128 group quantization ----
 * in: rows x n values of type in_dt (row stride in elements).
 * For each group of 128 columns (the last one may be shorter):
 *   a = max |v|, s = a / 448, q = (s == 0) ? 0x00 : e4m3(v / s).
 * q: rows x n bytes (row stride q_stride); s: rows x ceil(n/128) (stride s_stride). */
int orc_quant_groups(const void* in, int in_dt, int64_t in_stride, int64_t rows, int64_t n,
                     uint8_t* q, int64_t q_stride, float* s, int64_t s_stride);

/* ---- O2: gather of byte rows and fp32 scale rows through a dst2src map ----
 * dst_q[i, 0:k] = src_q[map[i], 0:k] and dst_s[i, 0:g] = src_s[map[i], 0:g] as raw
 * bits; map[i] < 0 writes a zero row and zero scales; n_dst == 0 does nothing. */
int orc_gather_rows_scales(const uint8_t* src_q, int64_t src_q_stride,
                           const float* src_s, int64_t src_s_stride,
                           int64_t n_src, int64_t k, int64_t g,
                           const int32_t* dst2src, int64_t n_dst,
                           uint8_t* dst_q, int64_t dst_q_stride,
                           float* dst_s, int64_t dst_s_stride);

/* ---- O3: block-FP8 GEMM  out[r, n] = sum_kb (sum_{k in kb} A*W) * sA[r,kb] * sW[e,n/128,kb] ----
 * A: fp8 rows (stride a_stride bytes), scales a_s (stride a_s_stride floats).
 * W: fp8 [E][N][K] with strides w_stride_e / w_stride_n in bytes, K contiguous.
 * W scales: [E][ceil(N/128)][ceil(K/128)] with strides w_s_stride_e / w_s_stride_n (floats).
 * mode GROUPED: rows [off[e], off[e+1]) use expert e, A row = r; m_rows = off[n_experts].
 * mode SLOT: row r uses slot_ids[r] (negative = inactive: +0 row, nothing read),
 *            A row = r / a_row_div.
 * out: m_rows x N of type out_dt, row stride out_stride (elements). */
int orc_block_gemm(const uint8_t* a_q, int64_t a_stride, const float* a_s, int64_t a_s_stride,
                   const uint8_t* w_q, int64_t w_stride_e, int64_t w_stride_n,
                   const float* w_s, int64_t w_s_stride_e, int64_t w_s_stride_n,
                   int64_t n_experts, int64_t N, int64_t K,
                   int mode, const int32_t* expert_offsets, const int32_t* slot_ids,
                   int64_t m_rows, int64_t a_row_div,
                   void* out, int out_dt, int64_t out_stride);

/* ---- O8: block-FP8 activations x MXFP4 weights ----
 * The FP4 weight variant of O3 ("perf(dsfp4): pick the grouped-prefill tile from route density on
 * sm_89": the routed-expert prefill kernel whose weights are FP4 and whose cost is dequantization).
 * The page does not fix the FP4 format; the reading taken is OCP MXFP4: E2M1 elements (sign, 2
 * exponent bits with bias 1, 1 mantissa bit: +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}), two per byte with K
 * element 2i in the low nibble, and one E8M0 scale (2^(e - 127), e = 255 NaN) per 32 consecutive K
 * elements.  w4 [n_experts] x [N][K/2] bytes (strides in bytes), w4_s [n_experts] x [N][K/32] bytes.
 * Activations and their 1x128 fp32 scales as in O3.  Per 128-K block kb, p = sum over its k in
 * ascending order of dq8(a[k]) * (dq4(w[k]) * 2^(e[k/32] - 127)) (each product exact), then
 * acc = acc + p * a_s[kb].  Modes as in O3.  K % 128 == 0. */
float orc_e2m1_to_f32(uint8_t code);
float orc_e8m0_to_f32(uint8_t e);
int orc_mxfp4_gemm(const uint8_t* a_q, int64_t a_stride, const float* a_s, int64_t a_s_stride,
                   const uint8_t* w4, int64_t w4_stride_e, int64_t w4_stride_n,
                   const uint8_t* w4_s, int64_t w4s_stride_e, int64_t w4s_stride_n,
                   int64_t n_experts, int64_t N, int64_t K,
                   int mode, const int32_t* expert_offsets, const int32_t* slot_ids,
                   int64_t m_rows, int64_t a_row_div,
                   void* out, int out_dt, int64_t out_stride);

/* ---- O4: gated activation + requant ----
 * in: rows x 2n (gate g = columns [0,n), up u = columns [n,2n)) of type in_dt.  h in fp32, then O1
 * on h.  The activations are the five GLU variants ("GLU Variants Improve Transformer", the gated
 * linear units with sigmoid, identity, ReLU, GELU and Swish_1 gates); the pages name "five
 * activations" without listing them:
 *   SILU_MUL    h = (g / (1 + expf(-g))) * u          (SwiGLU)
 *   GELU_MUL    h = (g * (0.5 * (1 + erff(g * 1/sqrt2)))) * u   (GEGLU, exact GELU)
 *   RELU_MUL    h = (g > 0 ? g : +0) * u              (ReGLU)
 *   SIGMOID_MUL h = (1 / (1 + expf(-g))) * u          (GLU)
 *   MUL         h = g * u                             (bilinear) */
enum { ORC_ACT_SILU_MUL = 1, ORC_ACT_GELU_MUL = 2, ORC_ACT_RELU_MUL = 3, ORC_ACT_SIGMOID_MUL = 4, ORC_ACT_MUL = 5 };
int orc_gated_act_quant(const void* in, int in_dt, int64_t in_stride, int64_t rows, int64_t n, int act,
                        uint8_t* q, int64_t q_stride, float* s, int64_t s_stride);
int orc_silu_mul_quant(const void* in, int in_dt, int64_t in_stride, int64_t rows, int64_t n,
                       uint8_t* q, int64_t q_stride, float* s, int64_t s_stride);

/* ---- O5: top-k weighted reduce ----
 * out[t, h] = bf16( sum_{j ascending, slot_ids[t,j] >= 0} w[t,j] * y[row(t,j), h] ), fp32 sum
 * starting at +0; row(t,j) = route_rows[t*topk+j], or t*topk+j when route_rows is NULL.
 * Weights of inactive routes are never read. */
int orc_topk_reduce(const void* y, int y_dt, int64_t y_stride,
                    const int32_t* slot_ids, const int32_t* route_rows, const float* weights,
                    int64_t T, int64_t topk, int64_t H, uint16_t* out_bf16, int64_t out_stride);

/* ---- O6: fused decode = O1(x) -> O3 slot(W13, fp32) -> O4 (act) -> O3 slot(W2, fp32) -> O5 ----
 * x: T x H bf16; slots/weights: T x topk; W13 [n_slots][2I][H], W2 [n_slots][H][I] (contiguous),
 * scales [n_slots][2I/128][H/128] and [n_slots][H/128][I/128] (contiguous).
 * Optional outputs of the intermediates (NULL to skip):
 *   xq [T][H], xs [T][ceil(H/128)], c1 [T*topk][2I] f32, aq [T*topk][I], as [T*topk][ceil(I/128)],
 *   c2 [T*topk][H] f32. */
int orc_fused_decode(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t I, int64_t topk, int act,
                     const int32_t* slot_ids, const float* weights, int64_t n_slots,
                     const uint8_t* w13_q, const float* w13_s,
                     const uint8_t* w2_q, const float* w2_s,
                     uint16_t* out_bf16,
                     uint8_t* xq, float* xs, float* c1, uint8_t* aq, float* as, float* c2);

/* ---- O7: routing prep of a prefill step ----
 * Where the dst2src map of the gather comes from ("[MoE] Gather the cutlass MoE activation and its
 * scales in one launch", Motivation: the activation is replicated once per routed expert through a
 * map of m * topk entries) and the expert-grouped row order of the grouped GEMM ("perf(dsfp4): pick
 * the grouped-prefill tile from route density on sm_89", Measurements: routes per expert).
 * logits: T x E fp32 (row stride logits_stride).  For each token, the topk experts with the largest
 * logits, in descending order (ties: lower expert index; logits must be finite); their weights are
 * the softmax over all E experts renormalized over the top-k, computed here in double from the
 * definition (softmax first, then renormalization) and rounded to fp32.
 * Routes are then listed in (expert, token) order: row r of that list is route (dst2src[r], j) with
 * ids[dst2src[r]][j] the row's expert; route_rows[t*topk + j] is the row of route (t, j), and
 * expert_offsets[e] the first row of expert e (expert_offsets[E] = T*topk). */
int orc_route_prep(const float* logits, int64_t logits_stride, int64_t T, int64_t E, int64_t topk,
                   int32_t* expert_ids, float* weights, int32_t* dst2src, int32_t* route_rows,
                   int32_t* expert_offsets);

#ifdef __cplusplus
}
#endif
#endif
