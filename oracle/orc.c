/*
 * CPU oracle for the routed-expert hot path of a block-FP8 MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the package smoke check
 * and the benchmark's CPU-baseline leg; never by the HIP library or its
 * binding.  Plain C99, single-threaded, compiled with -O2 -ffp-contract=off
 * and no fast-math so that every fp32 operation is one IEEE rounding.
 *
 * Sources of each definition (pages, by title and section):
 *   [P1] "perf(moe): skip inactive block-fp8 decode routes" -- opening
 *        section: a negative slot writes zero to the route's output tile and
 *        reads no activations, weights, scales or routing weights; the
 *        activation still processes the zeroed buffer; Validation: outputs
 *        equal the old clamped-slot (slot 0, weight 0) path exactly.
 *   [P2] "[MoE] Gather the cutlass MoE activation and its scales in one
 *        launch" -- Motivation: the activation is quantized once, rows are
 *        replicated per routed expert through a dst2src map of m*topk
 *        entries, k fp8 values travel with k//128 fp32 scales;
 *        Modifications: rows are copied as bytes, never decoded.
 *   [P4] "perf(dsfp4): pick the grouped-prefill tile from route density on
 *        sm_89" -- grouped prefill: rows sorted by expert, each expert's rows
 *        multiplied by that expert's weights, BLOCK_K of 128 = one block
 *        scale per K step.
 * The block-FP8 arithmetic itself (decode the e4m3 bytes, sum exact fp8
 * products in fp32 inside each 128-wide K block, then scale that partial sum
 * by the activation group scale times the weight block scale and add it to
 * an fp32 accumulator) is the plain definition of a product of two
 * block-scaled operands.
 */
#include "orc.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* codecs                                                             */
/* ------------------------------------------------------------------ */

/* OCP 8-bit floating point, E4M3 ("fn": no infinities, one NaN per sign):
 * exponent bias 7; e == 0 is subnormal m/8 * 2^-6; S.1111.111 is NaN. */
float orc_e4m3_to_f32(uint8_t code) {
    int s = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    float v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexpf((float)m, -9);            /* m/8 * 2^-6 */
    else
        v = ldexpf((float)(8 + m), e - 10);  /* (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

/* Round to nearest, ties to even, after clamping to the finite range. */
uint8_t orc_f32_to_e4m3(float v) {
    uint8_t sign;
    float a, f, m;
    int e, E;
    if (isnan(v)) return 0x7F;
    sign = signbit(v) ? 0x80 : 0x00;
    a = fabsf(v);
    if (a > 448.0f) a = 448.0f;
    if (a < 0.015625f) {                     /* below 2^-6: subnormal grid of 2^-9 */
        m = rintf(ldexpf(a, 9));             /* exact scaling, then RNE; 8 = 2^-6 */
        return (uint8_t)(sign | (uint8_t)m);
    }
    f = frexpf(a, &e);                       /* a = f * 2^e, f in [0.5, 1) */
    m = rintf((2.0f * f - 1.0f) * 8.0f);     /* mantissa field, RNE (exact operands) */
    E = e - 1 + 7;
    if (m == 8.0f) { m = 0.0f; E += 1; }
    return (uint8_t)(sign | (uint8_t)(E << 3) | (uint8_t)m);
}

float orc_bf16_to_f32(uint16_t h) {
    uint32_t x = (uint32_t)h << 16;
    float v;
    memcpy(&v, &x, 4);
    return v;
}

uint16_t orc_f32_to_bf16(float v) {
    uint32_t x;
    memcpy(&x, &v, 4);
    if ((x & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((x >> 16) | 0x0040u);
    x += 0x7FFFu + ((x >> 16) & 1u);
    return (uint16_t)(x >> 16);
}

float orc_f16_to_f32(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
    float v;
    if (e == 31) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexpf((float)m, -24);
    else v = ldexpf((float)(1024 + m), e - 25);
    return s ? -v : v;
}

uint16_t orc_f32_to_f16(float v) {
    uint32_t x, ax, mant, r, rem;
    uint16_t sign;
    memcpy(&x, &v, 4);
    sign = (uint16_t)((x >> 16) & 0x8000u);
    ax = x & 0x7FFFFFFFu;
    if (ax > 0x7F800000u) return (uint16_t)(sign | 0x7E00u);
    if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u);   /* >= 65520 rounds to inf */
    if (ax < 0x38800000u) {                                      /* below 2^-14: subnormal */
        float a;
        memcpy(&a, &ax, 4);
        return (uint16_t)(sign | (uint16_t)rintf(a * 16777216.0f)); /* units of 2^-24 */
    }
    mant = ax & 0x7FFFFFu;
    r = ((((ax >> 23) - 127u + 15u)) << 10) | (mant >> 13);
    rem = mant & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (r & 1u))) r++;
    return (uint16_t)(sign | r);
}

void orc_e4m3_decode_array(const uint8_t* in, int64_t n, float* out) {
    for (int64_t i = 0; i < n; i++) out[i] = orc_e4m3_to_f32(in[i]);
}
void orc_e4m3_encode_array(const float* in, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; i++) out[i] = orc_f32_to_e4m3(in[i]);
}
void orc_bf16_encode_array(const float* in, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; i++) out[i] = orc_f32_to_bf16(in[i]);
}
void orc_f16_encode_array(const float* in, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; i++) out[i] = orc_f32_to_f16(in[i]);
}

/* ------------------------------------------------------------------ */
/* helpers                                                            */
/* ------------------------------------------------------------------ */

static float load_elem(const void* base, int dt, int64_t idx) {
    switch (dt) {
        case ORC_F32: return ((const float*)base)[idx];
        case ORC_BF16: return orc_bf16_to_f32(((const uint16_t*)base)[idx]);
        default: return orc_f16_to_f32(((const uint16_t*)base)[idx]);
    }
}

static void store_elem(void* base, int dt, int64_t idx, float v) {
    switch (dt) {
        case ORC_F32: ((float*)base)[idx] = v; break;
        case ORC_BF16: ((uint16_t*)base)[idx] = orc_f32_to_bf16(v); break;
        default: ((uint16_t*)base)[idx] = orc_f32_to_f16(v); break;
    }
}

static int dt_ok(int dt) { return dt == ORC_F32 || dt == ORC_BF16 || dt == ORC_F16; }

/* One row of 1x128 group quantization on fp32 values. */
static void quant_row(const float* v, int64_t n, uint8_t* q, float* s) {
    for (int64_t g0 = 0, gi = 0; g0 < n; g0 += 128, gi++) {
        int64_t gl = (n - g0 < 128) ? (n - g0) : 128;
        float amax = 0.0f, sc;
        for (int64_t c = 0; c < gl; c++) {
            float a = fabsf(v[g0 + c]);
            if (a > amax) amax = a;
        }
        sc = amax / 448.0f;
        for (int64_t c = 0; c < gl; c++)
            q[g0 + c] = (sc == 0.0f) ? (uint8_t)0x00 : orc_f32_to_e4m3(v[g0 + c] / sc);
        s[gi] = sc;
    }
}

/* ------------------------------------------------------------------ */
/* O1                                                                 */
/* ------------------------------------------------------------------ */

int orc_quant_groups(const void* in, int in_dt, int64_t in_stride, int64_t rows, int64_t n,
                     uint8_t* q, int64_t q_stride, float* s, int64_t s_stride) {
    float* row;
    if (rows < 0 || n < 0 || !dt_ok(in_dt)) return -2;
    if (rows == 0 || n == 0) return 0;
    row = (float*)malloc((size_t)n * sizeof(float));
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t c = 0; c < n; c++) row[c] = load_elem(in, in_dt, r * in_stride + c);
        quant_row(row, n, q + r * q_stride, s + r * s_stride);
    }
    free(row);
    return 0;
}

/* ------------------------------------------------------------------ */
/* O2                                                                 */
/* ------------------------------------------------------------------ */

int orc_gather_rows_scales(const uint8_t* src_q, int64_t src_q_stride,
                           const float* src_s, int64_t src_s_stride,
                           int64_t n_src, int64_t k, int64_t g,
                           const int32_t* dst2src, int64_t n_dst,
                           uint8_t* dst_q, int64_t dst_q_stride,
                           float* dst_s, int64_t dst_s_stride) {
    if (n_dst < 0 || k < 0 || g < 0 || n_src < 0) return -2;
    for (int64_t i = 0; i < n_dst; i++) {
        int64_t src = dst2src[i];
        if (src < 0) {
            memset(dst_q + i * dst_q_stride, 0, (size_t)k);
            memset(dst_s + i * dst_s_stride, 0, (size_t)g * sizeof(float));
            continue;
        }
        if (src >= n_src) return -2;
        memcpy(dst_q + i * dst_q_stride, src_q + src * src_q_stride, (size_t)k);
        memcpy(dst_s + i * dst_s_stride, src_s + src * src_s_stride, (size_t)g * sizeof(float));
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* O3                                                                 */
/* ------------------------------------------------------------------ */

static void gemm_row(const float* lut, const uint8_t* arow, const float* asrow,
                     const uint8_t* w_e, int64_t w_stride_n, const float* ws_e, int64_t w_s_stride_n,
                     int64_t N, int64_t K, void* out, int out_dt, int64_t out_row) {
    int64_t nkb = (K + 127) / 128;
    for (int64_t n = 0; n < N; n++) {
        const uint8_t* wrow = w_e + n * w_stride_n;
        const float* wsrow = ws_e + (n / 128) * w_s_stride_n;
        float acc = 0.0f;
        for (int64_t kb = 0; kb < nkb; kb++) {
            int64_t k0 = kb * 128, k1 = (k0 + 128 < K) ? k0 + 128 : K;
            float p = 0.0f, sc;
            for (int64_t k = k0; k < k1; k++) {
                float prod = lut[arow[k]] * lut[wrow[k]];   /* exact: 4-bit x 4-bit mantissas */
                p = p + prod;
            }
            sc = asrow[kb] * wsrow[kb];
            acc = acc + p * sc;
        }
        store_elem(out, out_dt, out_row + n, acc);
    }
}

int orc_block_gemm(const uint8_t* a_q, int64_t a_stride, const float* a_s, int64_t a_s_stride,
                   const uint8_t* w_q, int64_t w_stride_e, int64_t w_stride_n,
                   const float* w_s, int64_t w_s_stride_e, int64_t w_s_stride_n,
                   int64_t n_experts, int64_t N, int64_t K,
                   int mode, const int32_t* expert_offsets, const int32_t* slot_ids,
                   int64_t m_rows, int64_t a_row_div,
                   void* out, int out_dt, int64_t out_stride) {
    float lut[256];
    if (N < 0 || K < 0 || m_rows < 0 || n_experts < 0 || !dt_ok(out_dt)) return -2;
    for (int c = 0; c < 256; c++) lut[c] = orc_e4m3_to_f32((uint8_t)c);
    if (mode == ORC_MODE_GROUPED) {
        if (expert_offsets[0] != 0 || expert_offsets[n_experts] != m_rows) return -2;
        for (int64_t e = 0; e < n_experts; e++) {
            if (expert_offsets[e + 1] < expert_offsets[e]) return -2;
            for (int64_t r = expert_offsets[e]; r < expert_offsets[e + 1]; r++)
                gemm_row(lut, a_q + r * a_stride, a_s + r * a_s_stride,
                         w_q + e * w_stride_e, w_stride_n, w_s + e * w_s_stride_e, w_s_stride_n,
                         N, K, out, out_dt, r * out_stride);
        }
        return 0;
    }
    if (mode != ORC_MODE_SLOT || a_row_div < 1) return -2;
    for (int64_t r = 0; r < m_rows; r++) {
        int64_t slot = slot_ids[r];
        int64_t ar = r / a_row_div;
        if (slot < 0) {                       /* inactive route: +0 row, nothing read */
            for (int64_t n = 0; n < N; n++) store_elem(out, out_dt, r * out_stride + n, 0.0f);
            continue;
        }
        if (slot >= n_experts) return -2;
        gemm_row(lut, a_q + ar * a_stride, a_s + ar * a_s_stride,
                 w_q + slot * w_stride_e, w_stride_n, w_s + slot * w_s_stride_e, w_s_stride_n,
                 N, K, out, out_dt, r * out_stride);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* O8: block-FP8 activations x MXFP4 weights                          */
/* ------------------------------------------------------------------ */

/* E2M1 element (low 4 bits of code): sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; exponent
 * 0 is subnormal: 0.5 * m. */
float orc_e2m1_to_f32(uint8_t code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    float v = e == 0 ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
    return s ? -v : v;
}

/* E8M0 scale: 2^(e - 127); e = 255 is NaN. */
float orc_e8m0_to_f32(uint8_t e) {
    if (e == 255) return NAN;
    return ldexpf(1.0f, (int)e - 127);
}

static void mx_gemm_row(const float* lut8, const uint8_t* arow, const float* asrow, const uint8_t* w_e,
                        int64_t w_stride_n, const uint8_t* ws_e, int64_t ws_stride_n, int64_t N, int64_t K,
                        void* out, int out_dt, int64_t out_row) {
    int64_t nkb = K / 128;
    for (int64_t n = 0; n < N; n++) {
        const uint8_t* wrow = w_e + n * w_stride_n;
        const uint8_t* wsrow = ws_e + n * ws_stride_n;
        float acc = 0.0f;
        for (int64_t kb = 0; kb < nkb; kb++) {
            float p = 0.0f;
            for (int64_t k = kb * 128; k < kb * 128 + 128; k++) {
                uint8_t byte = wrow[k / 2];
                float w = orc_e2m1_to_f32(k % 2 == 0 ? (uint8_t)(byte & 15) : (uint8_t)(byte >> 4));
                float ws = w * orc_e8m0_to_f32(wsrow[k / 32]);        /* exact: power-of-two scaling */
                float prod = lut8[arow[k]] * ws;                        /* exact: 4 x 2 significant bits */
                p = p + prod;
            }
            acc = acc + p * asrow[kb];
        }
        store_elem(out, out_dt, out_row + n, acc);
    }
}

int orc_mxfp4_gemm(const uint8_t* a_q, int64_t a_stride, const float* a_s, int64_t a_s_stride,
                   const uint8_t* w4, int64_t w4_stride_e, int64_t w4_stride_n,
                   const uint8_t* w4_s, int64_t w4s_stride_e, int64_t w4s_stride_n,
                   int64_t n_experts, int64_t N, int64_t K,
                   int mode, const int32_t* expert_offsets, const int32_t* slot_ids,
                   int64_t m_rows, int64_t a_row_div,
                   void* out, int out_dt, int64_t out_stride) {
    float lut8[256];
    if (N < 0 || K < 0 || K % 128 || m_rows < 0 || n_experts < 0 || !dt_ok(out_dt)) return -2;
    for (int c = 0; c < 256; c++) lut8[c] = orc_e4m3_to_f32((uint8_t)c);
    if (mode == ORC_MODE_GROUPED) {
        if (expert_offsets[0] != 0 || expert_offsets[n_experts] != m_rows) return -2;
        for (int64_t e = 0; e < n_experts; e++) {
            if (expert_offsets[e + 1] < expert_offsets[e]) return -2;
            for (int64_t r = expert_offsets[e]; r < expert_offsets[e + 1]; r++)
                mx_gemm_row(lut8, a_q + r * a_stride, a_s + r * a_s_stride, w4 + e * w4_stride_e, w4_stride_n,
                            w4_s + e * w4s_stride_e, w4s_stride_n, N, K, out, out_dt, r * out_stride);
        }
        return 0;
    }
    if (mode != ORC_MODE_SLOT || a_row_div < 1) return -2;
    for (int64_t r = 0; r < m_rows; r++) {
        int64_t slot = slot_ids[r];
        int64_t ar = r / a_row_div;
        if (slot < 0) {
            for (int64_t n = 0; n < N; n++) store_elem(out, out_dt, r * out_stride + n, 0.0f);
            continue;
        }
        if (slot >= n_experts) return -2;
        mx_gemm_row(lut8, a_q + ar * a_stride, a_s + ar * a_s_stride, w4 + slot * w4_stride_e, w4_stride_n,
                    w4_s + slot * w4s_stride_e, w4s_stride_n, N, K, out, out_dt, r * out_stride);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* O4                                                                 */
/* ------------------------------------------------------------------ */

/* The gated activations, each one fp32 expression in this order of operations: the five GLU variants
 * (GLU, bilinear, ReGLU, GEGLU, SwiGLU of "GLU Variants Improve Transformer"), gate g and up u. */
static float gated_act(int act, float g, float u) {
    switch (act) {
        case ORC_ACT_SILU_MUL: {        /* Swish_1(g) * u = g * sigmoid(g) * u */
            float den = 1.0f + expf(-g);
            return (g / den) * u;
        }
        case ORC_ACT_GELU_MUL: {        /* GELU(g) * u = g * Phi(g) * u, Phi via erf */
            float phi = 0.5f * (1.0f + erff(g * 0.70710678118654752f));
            return (g * phi) * u;
        }
        case ORC_ACT_RELU_MUL:          /* max(g, 0) * u, with +0 for g <= 0 */
            return (g > 0.0f ? g : 0.0f) * u;
        case ORC_ACT_SIGMOID_MUL: {     /* sigmoid(g) * u */
            float den = 1.0f + expf(-g);
            return (1.0f / den) * u;
        }
        default:                        /* ORC_ACT_MUL: g * u */
            return g * u;
    }
}

int orc_gated_act_quant(const void* in, int in_dt, int64_t in_stride, int64_t rows, int64_t n, int act,
                        uint8_t* q, int64_t q_stride, float* s, int64_t s_stride) {
    float* h;
    if (rows < 0 || n < 0 || !dt_ok(in_dt) || act < ORC_ACT_SILU_MUL || act > ORC_ACT_MUL) return -2;
    if (rows == 0 || n == 0) return 0;
    h = (float*)malloc((size_t)n * sizeof(float));
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t c = 0; c < n; c++) {
            float g = load_elem(in, in_dt, r * in_stride + c);
            float u = load_elem(in, in_dt, r * in_stride + n + c);
            h[c] = gated_act(act, g, u);
        }
        quant_row(h, n, q + r * q_stride, s + r * s_stride);
    }
    free(h);
    return 0;
}

int orc_silu_mul_quant(const void* in, int in_dt, int64_t in_stride, int64_t rows, int64_t n,
                       uint8_t* q, int64_t q_stride, float* s, int64_t s_stride) {
    return orc_gated_act_quant(in, in_dt, in_stride, rows, n, ORC_ACT_SILU_MUL, q, q_stride, s, s_stride);
}

/* ------------------------------------------------------------------ */
/* O5                                                                 */
/* ------------------------------------------------------------------ */

int orc_topk_reduce(const void* y, int y_dt, int64_t y_stride,
                    const int32_t* slot_ids, const int32_t* route_rows, const float* weights,
                    int64_t T, int64_t topk, int64_t H, uint16_t* out_bf16, int64_t out_stride) {
    if (T < 0 || topk < 0 || H < 0 || !dt_ok(y_dt)) return -2;
    for (int64_t t = 0; t < T; t++) {
        for (int64_t hh = 0; hh < H; hh++) {
            float acc = 0.0f;
            for (int64_t j = 0; j < topk; j++) {
                int64_t rt = t * topk + j;
                int64_t row;
                float term;
                if (slot_ids[rt] < 0) continue;   /* inactive: weight not read */
                row = route_rows ? route_rows[rt] : rt;
                term = weights[rt] * load_elem(y, y_dt, row * y_stride + hh);
                acc = acc + term;
            }
            out_bf16[t * out_stride + hh] = orc_f32_to_bf16(acc);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* O6                                                                 */
/* ------------------------------------------------------------------ */

int orc_fused_decode(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t I, int64_t topk, int act,
                     const int32_t* slot_ids, const float* weights, int64_t n_slots,
                     const uint8_t* w13_q, const float* w13_s,
                     const uint8_t* w2_q, const float* w2_s,
                     uint16_t* out_bf16,
                     uint8_t* xq, float* xs, float* c1, uint8_t* aq, float* as, float* c2) {
    int64_t R = T * topk;
    int64_t gH = (H + 127) / 128, gI = (I + 127) / 128, g2I = (2 * I + 127) / 128;
    int own_xq = !xq, own_xs = !xs, own_c1 = !c1, own_aq = !aq, own_as = !as, own_c2 = !c2;
    int rc;
    if (T < 0 || H <= 0 || I <= 0 || topk < 0 || n_slots < 0) return -2;
    if (own_xq) xq = (uint8_t*)malloc((size_t)(T * H + 1));
    if (own_xs) xs = (float*)malloc((size_t)(T * gH + 1) * sizeof(float));
    if (own_c1) c1 = (float*)malloc((size_t)(R * 2 * I + 1) * sizeof(float));
    if (own_aq) aq = (uint8_t*)malloc((size_t)(R * I + 1));
    if (own_as) as = (float*)malloc((size_t)(R * gI + 1) * sizeof(float));
    if (own_c2) c2 = (float*)malloc((size_t)(R * H + 1) * sizeof(float));

    rc = orc_quant_groups(x_bf16, ORC_BF16, H, T, H, xq, H, xs, gH);
    if (!rc) rc = orc_block_gemm(xq, H, xs, gH, w13_q, 2 * I * H, H, w13_s, g2I * gH, gH,
                                 n_slots, 2 * I, H, ORC_MODE_SLOT, NULL, slot_ids, R, topk,
                                 c1, ORC_F32, 2 * I);
    if (!rc) rc = orc_gated_act_quant(c1, ORC_F32, 2 * I, R, I, act, aq, I, as, gI);
    if (!rc) rc = orc_block_gemm(aq, I, as, gI, w2_q, H * I, I, w2_s, gH * gI, gI,
                                 n_slots, H, I, ORC_MODE_SLOT, NULL, slot_ids, R, 1,
                                 c2, ORC_F32, H);
    if (!rc) rc = orc_topk_reduce(c2, ORC_F32, H, slot_ids, NULL, weights, T, topk, H, out_bf16, H);

    if (own_xq) free(xq);
    if (own_xs) free(xs);
    if (own_c1) free(c1);
    if (own_aq) free(aq);
    if (own_as) free(as);
    if (own_c2) free(c2);
    return rc;
}

/* O7: routing prep.  Selection repeats "take the largest remaining logit" topk times (strictly larger
 * wins, so equal logits go to the lower index); the weights follow the definition: softmax over all
 * E experts in double, then division by the selected probabilities' sum.  The counting sort walks
 * experts in ascending order and, for each, tokens in ascending order. */
int orc_route_prep(const float* logits, int64_t logits_stride, int64_t T, int64_t E, int64_t topk,
                   int32_t* expert_ids, float* weights, int32_t* dst2src, int32_t* route_rows,
                   int32_t* expert_offsets) {
    int64_t t, e, j, row;
    double* p;
    unsigned char* taken;
    if (T < 0 || E <= 0 || topk < 1 || topk > E || logits_stride < E) return -2;
    p = (double*)malloc((size_t)E * sizeof(double));
    taken = (unsigned char*)malloc((size_t)E);
    for (t = 0; t < T; t++) {
        const float* l = logits + t * logits_stride;
        double mx = l[0], sum = 0.0, sel = 0.0;
        for (e = 1; e < E; e++)
            if (l[e] > mx) mx = l[e];
        for (e = 0; e < E; e++) {
            p[e] = exp((double)l[e] - mx);
            sum += p[e];
        }
        for (e = 0; e < E; e++) {
            p[e] /= sum;
            taken[e] = 0;
        }
        for (j = 0; j < topk; j++) {
            int64_t best = -1;
            for (e = 0; e < E; e++)
                if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
            taken[best] = 1;
            expert_ids[t * topk + j] = (int32_t)best;
            sel += p[best];
        }
        for (j = 0; j < topk; j++) weights[t * topk + j] = (float)(p[expert_ids[t * topk + j]] / sel);
    }
    row = 0;
    for (e = 0; e < E; e++) {
        expert_offsets[e] = (int32_t)row;
        for (t = 0; t < T; t++)
            for (j = 0; j < topk; j++)
                if (expert_ids[t * topk + j] == e) {
                    dst2src[row] = (int32_t)t;
                    route_rows[t * topk + j] = (int32_t)row;
                    row++;
                }
    }
    expert_offsets[E] = (int32_t)row;
    free(p);
    free(taken);
    return 0;
}
