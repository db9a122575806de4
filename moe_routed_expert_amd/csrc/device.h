// Device-side helpers shared by the gfx950 kernels of libmoe_routed.
//
// fp8 here is the OCP e4m3fn byte.  gfx950's v_cvt_pk_fp8_f32 rounds to
// nearest-even but turns magnitudes above 464 into NaN, so every encode
// clamps to +-448 first; with finite inputs that gives round-to-nearest-even
// with saturation.  v_cvt_pk_f32_fp8 decodes exactly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float clamp448(float v) {
    return __builtin_fminf(__builtin_fmaxf(v, -448.0f), 448.0f);
}

// Four fp32 values -> four e4m3 bytes packed little-endian into one word.
__device__ __forceinline__ uint32_t enc4_e4m3(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ uint32_t enc2_e4m3(float a, float b) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false) & 0xFFFFu;
}

// The e4m3 codes of RN(v[i] / s), four per word (little-endian), for N values (N % 4 == 0) sharing the scale
// s = RN(amax / 448) > 0 of a group whose largest magnitude is amax (so |v[i]| <= amax; v finite).  The
// quotients take the steps of the correctly rounded fp32 division: the reciprocal (v_rcp_f32) refined once,
// q = v * y, then two corrections q -= (s * q - v) * y, the residual exact in an fma; what the division adds
// to them is a range scaling and a fix-up of special cases, which s in [2^-90, 2^90] never needs for a
// quotient of magnitude 2^-10 or more.  Smaller quotients may differ in their last bits, but all of them have
// the code of a signed zero, and the residual's sign convention keeps the sign of a zero v.  There s is
// normal, so |q| <= 448 (1 + 2^-23), which the conversion rounds to 448 without a clamp.  Checked on the
// device against the division: every pair of bf16 values, 4.3e9 random fp32 pairs and 9.1e9 quotients on
// and next to e4m3 midpoints, with no code that differs.  Any other s takes the division itself and the
// clamped conversion (a wave-uniform branch in practice).  5 operations and one conversion per two values.
template <int N>
__device__ __forceinline__ void e4m3_codes(const float (&v)[N], float s, uint32_t (&w)[N / 4]) {
    static_assert(N % 4 == 0, "four codes per word");
    if (s >= 0x1p-90f && s <= 0x1p90f) {
        const float y0 = __builtin_amdgcn_rcpf(s);
        const float y = __builtin_fmaf(__builtin_fmaf(-s, y0, 1.0f), y0, y0);
        float q[N];
#pragma unroll
        for (int i = 0; i < N; i++) {
            const float q0 = v[i] * y;
            const float q1 = __builtin_fmaf(-__builtin_fmaf(s, q0, -v[i]), y, q0);
            q[i] = __builtin_fmaf(-__builtin_fmaf(s, q1, -v[i]), y, q1);
        }
#pragma unroll
        for (int k = 0; k < N / 4; k++) {
            const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * k], q[4 * k + 1], 0, false);
            w[k] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[4 * k + 2], q[4 * k + 3], lo, true);
        }
    } else {
#pragma unroll
        for (int k = 0; k < N / 4; k++)
            w[k] = enc4_e4m3(v[4 * k] / s, v[4 * k + 1] / s, v[4 * k + 2] / s, v[4 * k + 3] / s);
    }
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
    uint32_t x = __float_as_uint(v);
    if ((x & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((x >> 16) | 0x40u);
    x += 0x7FFFu + ((x >> 16) & 1u);
    return (uint16_t)(x >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16(float v) {
    _Float16 h = (_Float16)v;
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// Element types of 16/32-bit float buffers (values of moe_dtype).
enum : int { kBF16 = 0, kF32 = 1, kF16 = 2 };

template <int DT>
__device__ __forceinline__ float load_as_f32(const void* p, int64_t i) {
    if constexpr (DT == kF32) return ((const float*)p)[i];
    else if constexpr (DT == kBF16) return bf16_to_f32(((const uint16_t*)p)[i]);
    else return f16_to_f32(((const uint16_t*)p)[i]);
}

template <int DT>
__device__ __forceinline__ void store_from_f32(void* p, int64_t i, float v) {
    if constexpr (DT == kF32) ((float*)p)[i] = v;
    else if constexpr (DT == kBF16) ((uint16_t*)p)[i] = f32_to_bf16(v);
    else ((uint16_t*)p)[i] = f32_to_f16(v);
}

// sigmoid(g) = 1 / (1 + e^-g) from the hardware exp2 (v_exp_f32) of -g*log2(e) and the hardware reciprocal
// (v_rcp_f32), each within an ulp: 4 instructions instead of a libm-accurate expf and a correctly rounded
// division (about 22).  Limits: g = +inf gives 1, g = -inf and g below about -88.7 give 0 (e^-g overflows, as
// in fp32 libm); between -88.7 and -87.3 the true value is below the fp32 normal range and the reciprocal
// returns 0.
__device__ __forceinline__ float fast_sigmoid(float g) {
    const float t = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
    return __builtin_amdgcn_rcpf(1.0f + t);
}

// Gated activation of gate g and up u in fp32 (moe_act values 1..5: SwiGLU, GEGLU with the exact GELU,
// ReGLU, GLU, bilinear -- the five GLU variants), one expression each in a fixed order of operations.
// ACT is a compile-time constant here, so a loop over elements carries no per-element switch.
template <int ACT>
__device__ __forceinline__ float gated_act_t(float g, float u) {
    if constexpr (ACT == 1) return (g * fast_sigmoid(g)) * u;
    else if constexpr (ACT == 2) return (g * (0.5f * (1.0f + erff(g * 0.70710678118654752f)))) * u;
    else if constexpr (ACT == 3) return (g > 0.0f ? g : 0.0f) * u;
    else if constexpr (ACT == 4) return fast_sigmoid(g) * u;
    else return g * u;
}

// The same with the activation chosen at run time (one wave-uniform switch per element).
__device__ __forceinline__ float gated_act(int act, float g, float u) {
    switch (act) {
        case 1: return gated_act_t<1>(g, u);
        case 2: return gated_act_t<2>(g, u);
        case 3: return gated_act_t<3>(g, u);
        case 4: return gated_act_t<4>(g, u);
        default: return gated_act_t<5>(g, u);
    }
}

// Four consecutive elements i..i+3 from fp32 in one store; p + i must be aligned to 4 elements.
template <int DT>
__device__ __forceinline__ void store4_from_f32(void* p, int64_t i, v4f v) {
    if constexpr (DT == kF32) {
        *reinterpret_cast<v4f*>((float*)p + i) = v;
    } else {
        uint16_t h[4];
#pragma unroll
        for (int k = 0; k < 4; k++) h[k] = DT == kBF16 ? f32_to_bf16(v[k]) : f32_to_f16(v[k]);
        uint2 w;
        w.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
        w.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
        *reinterpret_cast<uint2*>((uint16_t*)p + i) = w;
    }
}

// Max over aligned groups of 2^LOG lanes (butterfly; every lane gets the group max).
template <int LOG>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
    for (int m = 1; m < (1 << LOG); m <<= 1) v = __builtin_fmaxf(v, __shfl_xor(v, m, kWave));
    return v;
}

// DPP lane moves (gfx9 encodings): quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror,
// row_mirror, row_bcast:15, row_bcast:31.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float old, float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                                  __builtin_bit_cast(int, v), CTRL, ROW_MASK,
                                                                  0xF, false));
}

// Max over each aligned group of 8 lanes, returned in every lane of the group (register-only DPP moves).
__device__ __forceinline__ float group8_max(float v) {
    v = __builtin_fmaxf(v, dpp_f32<0xB1>(v, v));    // quad_perm [1,0,3,2]
    v = __builtin_fmaxf(v, dpp_f32<0x4E>(v, v));    // quad_perm [2,3,0,1]
    v = __builtin_fmaxf(v, dpp_f32<0x141>(v, v));   // row_half_mirror: lane i <- 7-i within 8
    return v;
}

// Max over each row of 16 lanes, returned in every lane of the row (register-only DPP moves).
__device__ __forceinline__ float row16_max(float v) {
    v = group8_max(v);
    v = __builtin_fmaxf(v, dpp_f32<0x140>(v, v));   // row_mirror: lane i <- 15-i within 16
    return v;
}

// Max over the whole wave as a wave-uniform value: row maxima, then row_bcast:15 /
// row_bcast:31 carry them into lane 63, which is read back as a scalar.
__device__ __forceinline__ float wave_max(float v) {
    v = row16_max(v);
    v = __builtin_fmaxf(v, dpp_f32<0x142, 0xA>(v, v));   // rows 1,3 take lane 15 of rows 0,2
    v = __builtin_fmaxf(v, dpp_f32<0x143, 0xC>(v, v));   // rows 2,3 take lane 31
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// 16x16x128 fp8 x fp8 -> fp32 MFMA (e4m3 operands, no block exponent scaling).
// Operand layout (checked on gfx950): lane l holds row (A) / column (B) l%16 and
// 32 K values for K-quarter l/16; both operands use the same K order, so any
// fixed assignment of 32 K positions per K-quarter works as long as A and B
// agree.  Result: lane l, element i = C[4*(l/16)+i][l%16].
__device__ __forceinline__ v4f mfma16x16x128_e4m3(const v8i& a, const v8i& b, const v4f& c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 16x16x128 MFMA with an MXFP4 row operand and an fp8 (e4m3) column operand (layout checked on gfx950):
// the fp4 operand's lane l holds row l%16 and the 32 consecutive K elements 32*(l/16) .. +31 as 16 bytes
// in the low four dwords of w, K element 2i in the low nibble; the fp8 operand is laid out as in
// mfma16x16x128_e4m3.  Scales are E8M0 bytes (low byte of the word): the scale of K block b for row x
// comes from lane 16b + x, which is the lane that holds that block, so each lane passes its own block's
// scale; the column operand's scale is 2^0.
__device__ __forceinline__ v4f mfma16x16x128_fp4_e4m3(const v4i& w, uint32_t w_scale, const v8i& a, const v4f& c) {
    const v8i w8 = {w[0], w[1], w[2], w[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w8, a, c, 4, 0, 0, (int)w_scale, 0, 127);
}

// Orders this wave's LDS accesses before/after the call (compiler and memory
// model, wavefront scope).  Valid only for data written and read by one wave.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Reads two 32-bit words through the scalar data cache with one wait; each pointer must be the same in
// every lane (the values are wave-uniform).  For the few small words a wave needs before its first
// large vector loads: a scalar read does not wait behind the vector loads the CU already has in
// flight, which under a full weight stream take microseconds to drain.
__device__ __forceinline__ void scalar_read2(const void* p, const void* q, uint32_t& a, uint32_t& b) {
    asm volatile("s_load_dword %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
                 : "=&s"(a), "=&s"(b)
                 : "s"(p), "s"(q)
                 : "memory");
}

// As scalar_read2, for three words.
__device__ __forceinline__ void scalar_read3(const void* p, const void* q, const void* r, uint32_t& a, uint32_t& b,
                                             uint32_t& c) {
    asm volatile("s_load_dword %0, %3, 0x0\n\ts_load_dword %1, %4, 0x0\n\ts_load_dword %2, %5, 0x0\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&s"(a), "=&s"(b), "=&s"(c)
                 : "s"(p), "s"(q), "s"(r)
                 : "memory");
}

}  // namespace moe
