// Per-row 1x128 fp8 quantization, optionally of a gated activation act(gate)*up.
//
// IDENTITY mode quantizes an activation once before it is replicated per
// routed expert ("[MoE] Gather the cutlass MoE activation and its scales in
// one launch", Motivation).  The gated modes (SwiGLU and the other four GLU
// variants) are the activation between the two GEMMs; they also run over the
// zeroed tiles of inactive routes, which they map
// to zero codes and zero scales ("perf(moe): skip inactive block-fp8 decode
// routes", opening section).
//
// MI355X design: one wavefront per (row, 512 columns); each lane owns 8
// consecutive columns, 16 lanes form one 128-column group, and the group amax
// is four DPP row moves inside the wave, so no LDS and no barrier is needed.
// The 8 codes of a lane leave as one 8-byte store.  The scale is amax/448 with
// the correctly rounded fp32 division and each code is v/s rounded to nearest
// even (clamped to +-448), matching the definition bit for bit in IDENTITY mode.
#include "device.h"
#include "host.h"

namespace moe {
namespace {

constexpr int kColsPerLane = 8;
constexpr int kColsPerWave = kWave * kColsPerLane;   // 512 = 4 groups

template <int DT, bool GATED, bool VEC>
__global__ void __launch_bounds__(256)
act_quant_kernel(const void* __restrict__ in, int64_t in_stride, int64_t rows, int64_t n, int act,
                 uint8_t* __restrict__ out_q, int64_t q_stride, float* __restrict__ out_s, int64_t s_stride) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t segs = ceil_div(n, kColsPerWave);
    const int64_t gw = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int64_t row = gw / segs;
    if (row >= rows) return;
    const int64_t c0 = (gw % segs) * kColsPerWave + (int64_t)lane * kColsPerLane;
    const int64_t base = row * in_stride;
    const int64_t ncols = n;   // width of v
    float v[kColsPerLane];
    const bool full = c0 + kColsPerLane <= ncols;
    if (VEC && full) {
        // 16-byte loads: 8 bf16/f16 values, or 2 x 4 f32 values
        if constexpr (DT == kF32) {
            const float4* p = reinterpret_cast<const float4*>((const float*)in + base + c0);
            float4 a = p[0], b = p[1];
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
            if constexpr (GATED) {
                const float4* pu = reinterpret_cast<const float4*>((const float*)in + base + n + c0);
                float4 ua = pu[0], ub = pu[1];
                float u[8] = {ua.x, ua.y, ua.z, ua.w, ub.x, ub.y, ub.z, ub.w};
#pragma unroll
                for (int i = 0; i < 8; i++) v[i] = gated_act(act, v[i], u[i]);
            }
        } else {
            uint4 a = *reinterpret_cast<const uint4*>((const uint16_t*)in + base + c0);
            uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                v[2 * i] = DT == kBF16 ? bf16_to_f32((uint16_t)(w[i] & 0xFFFF)) : f16_to_f32((uint16_t)(w[i] & 0xFFFF));
                v[2 * i + 1] = DT == kBF16 ? bf16_to_f32((uint16_t)(w[i] >> 16)) : f16_to_f32((uint16_t)(w[i] >> 16));
            }
            if constexpr (GATED) {
                uint4 b = *reinterpret_cast<const uint4*>((const uint16_t*)in + base + n + c0);
                uint32_t x[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    float u0 = DT == kBF16 ? bf16_to_f32((uint16_t)(x[i] & 0xFFFF)) : f16_to_f32((uint16_t)(x[i] & 0xFFFF));
                    float u1 = DT == kBF16 ? bf16_to_f32((uint16_t)(x[i] >> 16)) : f16_to_f32((uint16_t)(x[i] >> 16));
                    v[2 * i] = gated_act(act, v[2 * i], u0);
                    v[2 * i + 1] = gated_act(act, v[2 * i + 1], u1);
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kColsPerLane; i++) {
            const int64_t c = c0 + i;
            float x = 0.0f;
            if (c < ncols) {
                x = load_as_f32<DT>(in, base + c);
                if constexpr (GATED) {
                    float u = load_as_f32<DT>(in, base + n + c);
                    x = gated_act(act, x, u);
                }
            }
            v[i] = x;
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kColsPerLane; i++) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
    amax = row16_max(amax);                    // 16 lanes = one 128-column group
    const float s = amax / 448.0f;
    uint32_t lo = 0, hi = 0;
    if (s != 0.0f) {
        lo = enc4_e4m3(v[0] / s, v[1] / s, v[2] / s, v[3] / s);
        hi = enc4_e4m3(v[4] / s, v[5] / s, v[6] / s, v[7] / s);
    }
    if (c0 < ncols) {
        uint8_t* q = out_q + row * q_stride + c0;
        if (full && (reinterpret_cast<uintptr_t>(q) & 7u) == 0) {
            *reinterpret_cast<uint2*>(q) = make_uint2(lo, hi);
        } else {
            for (int i = 0; i < kColsPerLane && c0 + i < ncols; i++)
                q[i] = (uint8_t)(((i < 4 ? lo : hi) >> (8 * (i & 3))) & 0xFF);
        }
        if ((lane & 15) == 0) out_s[row * s_stride + c0 / 128] = s;
    }
}

template <int DT, bool GATED>
void launch_act(bool vec, dim3 grid, hipStream_t st, const void* in, int64_t in_stride, int64_t rows, int64_t n,
                int act, uint8_t* q, int64_t qs, float* s, int64_t ss) {
    if (vec)
        hipLaunchKernelGGL((act_quant_kernel<DT, GATED, true>), grid, dim3(256), 0, st, in, in_stride, rows, n, act,
                           q, qs, s, ss);
    else
        hipLaunchKernelGGL((act_quant_kernel<DT, GATED, false>), grid, dim3(256), 0, st, in, in_stride, rows, n, act,
                           q, qs, s, ss);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_act_quant(const void* in, int in_dt, int64_t in_stride, int64_t rows, int64_t n, int act,
                             uint8_t* out_q, int64_t q_stride, float* out_s, int64_t s_stride, void* stream) {
    if (rows < 0 || n < 0) return MOE_ERR_SHAPE;
    if (!dtype_ok(in_dt)) return MOE_ERR_DTYPE;
    if (act < MOE_ACT_IDENTITY || act > MOE_ACT_MUL) return MOE_ERR_SHAPE;
    if (rows == 0 || n == 0) return MOE_OK;
    if (!in || !out_q || !out_s) return MOE_ERR_NULL;
    const int64_t width = act != MOE_ACT_IDENTITY ? 2 * n : n;
    if (in_stride < width || q_stride < n || s_stride < ceil_div(n, 128)) return MOE_ERR_SHAPE;
    const int64_t esz = in_dt == MOE_F32 ? 4 : 2;
    // vector loads need every lane's 8 elements 16-byte aligned: base, stride and the up offset
    const bool vec = aligned16(in) && (in_stride * esz) % 16 == 0 && (n * esz) % 16 == 0;
    const int64_t waves = rows * ceil_div(n, kColsPerWave);
    const int64_t blocks = ceil_div(waves, 4);
    if (blocks > 0x7FFFFFFF) return MOE_ERR_SHAPE;
    dim3 grid((unsigned)blocks);
    auto st = as_stream(stream);
    if (act == MOE_ACT_IDENTITY) {
        if (in_dt == MOE_F32) launch_act<kF32, false>(vec, grid, st, in, in_stride, rows, n, act, out_q, q_stride, out_s, s_stride);
        else if (in_dt == MOE_BF16) launch_act<kBF16, false>(vec, grid, st, in, in_stride, rows, n, act, out_q, q_stride, out_s, s_stride);
        else launch_act<kF16, false>(vec, grid, st, in, in_stride, rows, n, act, out_q, q_stride, out_s, s_stride);
    } else {
        if (in_dt == MOE_F32) launch_act<kF32, true>(vec, grid, st, in, in_stride, rows, n, act, out_q, q_stride, out_s, s_stride);
        else if (in_dt == MOE_BF16) launch_act<kBF16, true>(vec, grid, st, in, in_stride, rows, n, act, out_q, q_stride, out_s, s_stride);
        else launch_act<kF16, true>(vec, grid, st, in, in_stride, rows, n, act, out_q, q_stride, out_s, s_stride);
    }
    return launch_status();
}
