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
// MI355X design: one wavefront per (row, 1024 columns), from a 2D grid (column
// groups x rows, rows taken in strides beyond 65535) so no index needs an
// integer division.  Each lane owns 16 consecutive columns: the per-group
// scale, refined reciprocal and amax and the addressing (a wave-uniform row
// base plus a 32-bit lane offset) are shared by 16 codes.  Waves that took 2, 4 or 8 rows with all their
// loads in flight at once, or that requested the next row while quantizing the
// current one (fewer, longer-lived workgroups), ran slower, not faster: the
// kernel is bound by how many waves have loads in flight (it runs at 83-89 %
// of a plain copy of its traffic).  The gated modes take the activation as a
// template parameter of the segment loop, chosen by one switch per wave, and
// the sigmoid from the hardware exp2 and reciprocal (fast_sigmoid): with libm's
// expf and a division per element the SiLU requant was bound by VALU issue.
// 8 lanes form one 128-column group, and the group amax is three DPP moves inside the wave,
// so no LDS and no barrier is needed.  The 16 codes of a lane leave as one
// 16-byte store.  The scale is amax/448 with
// the correctly rounded fp32 division and each code is that of v/s rounded to
// nearest even (clamped to +-448), matching the definition bit for bit in
// IDENTITY mode; the quotients take the correctly rounded division's own steps
// without its range scaling (e4m3_codes: 5 operations each, no branch per
// column), which give the same codes.
#include "device.h"
#include "host.h"

namespace moe {
namespace {

constexpr int kColsPerLane = 16;
constexpr int kColsPerWave = kWave * kColsPerLane;   // 1024 = 8 groups


// One lane's 16-byte input words for its 16 columns of one row (four words for f32), and those of
// the matching up columns when the activation is gated.
template <int DT>
struct RawCols {
    static constexpr int W = DT == kF32 ? 4 : 2;
    uint4 g[W];
    uint4 u[W];
};

// rowp: the row's first input byte (wave-uniform); off: this lane's byte offset of column c0
template <int DT, bool GATED>
__device__ __forceinline__ RawCols<DT> load_cols(const char* __restrict__ rowp, uint32_t off, int64_t up_bytes) {
    RawCols<DT> r;
    const uint4* pg = reinterpret_cast<const uint4*>(rowp + off);
#pragma unroll
    for (int i = 0; i < RawCols<DT>::W; i++) r.g[i] = pg[i];
    if constexpr (GATED) {
        const uint4* pu = reinterpret_cast<const uint4*>(rowp + up_bytes + off);
#pragma unroll
        for (int i = 0; i < RawCols<DT>::W; i++) r.u[i] = pu[i];
    }
    return r;
}

template <int DT>
__device__ __forceinline__ void unpack_cols(const uint4 (&w)[RawCols<DT>::W], float (&v)[kColsPerLane]) {
#pragma unroll
    for (int k = 0; k < RawCols<DT>::W; k++) {
        const uint32_t x[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
        if constexpr (DT == kF32) {
#pragma unroll
            for (int i = 0; i < 4; i++) v[4 * k + i] = __uint_as_float(x[i]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                v[8 * k + 2 * i] = DT == kBF16 ? bf16_to_f32((uint16_t)(x[i] & 0xFFFF)) : f16_to_f32((uint16_t)(x[i] & 0xFFFF));
                v[8 * k + 2 * i + 1] = DT == kBF16 ? bf16_to_f32((uint16_t)(x[i] >> 16)) : f16_to_f32((uint16_t)(x[i] >> 16));
            }
        }
    }
}

// The 16 codes (as four words) and the group scale of this lane's columns v; the 8 lanes of a
// 128-column group share the scale.
__device__ __forceinline__ void quant_cols(const float (&v)[kColsPerLane], uint32_t (&w)[4], float& s) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kColsPerLane; i++) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
    amax = group8_max(amax);                   // 8 lanes = one 128-column group
    s = amax / 448.0f;
#pragma unroll
    for (int k = 0; k < 4; k++) w[k] = 0u;
    // the codes of RN(v / s) (e4m3_codes), no branch per column
    if (s != 0.0f) e4m3_codes(v, s, w);
}

// A segment of 1024 columns that lies inside the row, with 16-byte aligned loads: no per-column bounds;
// the row bases are wave-uniform and each lane adds its own 32-bit offset.
template <int DT, int ACT>
__device__ __forceinline__ void act_quant_segment(const void* __restrict__ in, int64_t in_stride, int64_t rows,
                                                  int64_t n, int64_t seg, int lane,
                                                  uint8_t* __restrict__ out_q, int64_t q_stride,
                                                  float* __restrict__ out_s, int64_t s_stride) {
    constexpr int64_t esz = DT == kF32 ? 4 : 2;
    const uint32_t lane_off = (uint32_t)(lane * kColsPerLane * esz);
    const uint32_t q_off = (uint32_t)(lane * kColsPerLane);
    for (int64_t row = blockIdx.y; row < rows; row += gridDim.y) {
        const char* rowp = (const char*)in + (row * in_stride + seg * kColsPerWave) * esz;
        const RawCols<DT> raw = load_cols<DT, ACT != 0>(rowp, lane_off, n * esz);
        float v[kColsPerLane];
        unpack_cols<DT>(raw.g, v);
        if constexpr (ACT != 0) {
            float u[kColsPerLane];
            unpack_cols<DT>(raw.u, u);
#pragma unroll
            for (int i = 0; i < kColsPerLane; i++) v[i] = gated_act_t<ACT>(v[i], u[i]);
        }
        uint32_t w[4];
        float s;
        quant_cols(v, w, s);
        uint8_t* q = out_q + row * q_stride + seg * kColsPerWave + q_off;
        if ((reinterpret_cast<uintptr_t>(q) & 15u) == 0) {
            *reinterpret_cast<uint4*>(q) = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
#pragma unroll
            for (int i = 0; i < kColsPerLane; i++) q[i] = (uint8_t)((w[i >> 2] >> (8 * (i & 3))) & 0xFF);
        }
        if ((lane & 7) == 0) out_s[row * s_stride + seg * (kColsPerWave / 128) + (lane >> 3)] = s;
    }
}

// Any segment: per-column bounds and element loads (the last, partial segment of a row, or inputs whose
// rows or up offset are not 16-byte aligned).  This lane owns columns [c0, c0 + 16).
template <int DT, bool GATED>
__device__ __forceinline__ void act_quant_segment_any(const void* __restrict__ in, int64_t in_stride, int64_t rows,
                                                      int64_t n, int act, int64_t c0, int lane,
                                                      uint8_t* __restrict__ out_q, int64_t q_stride,
                                                      float* __restrict__ out_s, int64_t s_stride) {
    for (int64_t row = blockIdx.y; row < rows; row += gridDim.y) {
        const int64_t base = row * in_stride;
        float v[kColsPerLane];
#pragma unroll
        for (int i = 0; i < kColsPerLane; i++) {
            const int64_t c = c0 + i;
            float x = 0.0f;
            if (c < n) {
                x = load_as_f32<DT>(in, base + c);
                if constexpr (GATED) {
                    float u = load_as_f32<DT>(in, base + n + c);
                    x = gated_act(act, x, u);
                }
            }
            v[i] = x;
        }
        uint32_t w[4];
        float s;
        quant_cols(v, w, s);
        if (c0 < n) {
            uint8_t* q = out_q + row * q_stride + c0;
            for (int i = 0; i < kColsPerLane && c0 + i < n; i++) q[i] = (uint8_t)((w[i >> 2] >> (8 * (i & 3))) & 0xFF);
            if ((lane & 7) == 0) out_s[row * s_stride + c0 / 128] = s;
        }
    }
}

template <int DT, bool GATED, bool VEC>
__global__ void __launch_bounds__(256)
act_quant_kernel(const void* __restrict__ in, int64_t in_stride, int64_t rows, int64_t n, int act,
                 uint8_t* __restrict__ out_q, int64_t q_stride, float* __restrict__ out_s, int64_t s_stride) {
    const int lane = threadIdx.x & (kWave - 1);
    // grid: x = groups of blockDim.x/64 segments of 1024 columns, y = rows (taken in strides beyond the
    // grid), so no index needs an integer division; the segment is wave-uniform
    const int64_t seg = (int64_t)blockIdx.x * (blockDim.x / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (seg * kColsPerWave >= n) return;
    if (VEC && (seg + 1) * kColsPerWave <= n) {
        // one wave-uniform switch on the activation, outside the row and column loops
        if constexpr (!GATED) {
            act_quant_segment<DT, 0>(in, in_stride, rows, n, seg, lane, out_q, q_stride, out_s, s_stride);
        } else {
            switch (act) {
                case 1: act_quant_segment<DT, 1>(in, in_stride, rows, n, seg, lane, out_q, q_stride, out_s, s_stride); break;
                case 2: act_quant_segment<DT, 2>(in, in_stride, rows, n, seg, lane, out_q, q_stride, out_s, s_stride); break;
                case 3: act_quant_segment<DT, 3>(in, in_stride, rows, n, seg, lane, out_q, q_stride, out_s, s_stride); break;
                case 4: act_quant_segment<DT, 4>(in, in_stride, rows, n, seg, lane, out_q, q_stride, out_s, s_stride); break;
                default: act_quant_segment<DT, 5>(in, in_stride, rows, n, seg, lane, out_q, q_stride, out_s, s_stride); break;
            }
        }
    } else
        act_quant_segment_any<DT, GATED>(in, in_stride, rows, n, act, seg * kColsPerWave + (int64_t)lane * kColsPerLane,
                                         lane, out_q, q_stride, out_s, s_stride);
}

template <int DT, bool GATED>
void launch_act(bool vec, dim3 grid, dim3 block, hipStream_t st, const void* in, int64_t in_stride, int64_t rows,
                int64_t n, int act, uint8_t* q, int64_t qs, float* s, int64_t ss) {
    if (vec)
        hipLaunchKernelGGL((act_quant_kernel<DT, GATED, true>), grid, block, 0, st, in, in_stride, rows, n, act,
                           q, qs, s, ss);
    else
        hipLaunchKernelGGL((act_quant_kernel<DT, GATED, false>), grid, block, 0, st, in, in_stride, rows, n, act,
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
    // vector loads need every lane's 16 elements 16-byte aligned: base, stride and the up offset
    const bool vec = aligned16(in) && (in_stride * esz) % 16 == 0 && (n * esz) % 16 == 0;
    const int64_t segs = ceil_div(n, kColsPerWave);                   // 1024-column segments per row
    const int64_t wpb = segs < 4 ? segs : 4;                            // waves per workgroup
    const int64_t col_blocks = ceil_div(segs, wpb);
    const int64_t row_blocks = rows;
    if (col_blocks > 0x7FFFFFFF) return MOE_ERR_SHAPE;
    dim3 grid((unsigned)col_blocks, (unsigned)(row_blocks < 65535 ? row_blocks : 65535)), block((unsigned)(wpb * kWave));
    auto st = as_stream(stream);
    if (act == MOE_ACT_IDENTITY) {
        if (in_dt == MOE_F32) launch_act<kF32, false>(vec, grid, block, st, in, in_stride, rows, n, act, out_q, q_stride, out_s, s_stride);
        else if (in_dt == MOE_BF16) launch_act<kBF16, false>(vec, grid, block, st, in, in_stride, rows, n, act, out_q, q_stride, out_s, s_stride);
        else launch_act<kF16, false>(vec, grid, block, st, in, in_stride, rows, n, act, out_q, q_stride, out_s, s_stride);
    } else {
        if (in_dt == MOE_F32) launch_act<kF32, true>(vec, grid, block, st, in, in_stride, rows, n, act, out_q, q_stride, out_s, s_stride);
        else if (in_dt == MOE_BF16) launch_act<kBF16, true>(vec, grid, block, st, in, in_stride, rows, n, act, out_q, q_stride, out_s, s_stride);
        else launch_act<kF16, true>(vec, grid, block, st, in, in_stride, rows, n, act, out_q, q_stride, out_s, s_stride);
    }
    return launch_status();
}
