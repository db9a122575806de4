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
// MI355X design: one wavefront per (row, 512 columns), from a 2D grid (column
// groups x rows, rows taken in strides beyond 65535) so no index needs an
// integer division.  The kernel is bound by its vector ALU work (about 150
// instructions per wavefront), not by HBM: waves that take 2, 4 or 8 rows with
// all their loads in flight at once ran slower, not faster.  Each lane owns 8
// consecutive columns, 16 lanes form one 128-column group, and the group amax
// is four DPP row moves inside the wave, so no LDS and no barrier is needed.
// The 8 codes of a lane leave as one 8-byte store.  The scale is amax/448 with
// the correctly rounded fp32 division and each code is that of v/s rounded to
// nearest even (clamped to +-448), matching the definition bit for bit in
// IDENTITY mode; the quotient is v * (1/s) except near a code boundary, where
// it is the exact division (e4m3_quot), so one division per lane replaces eight.
#include "device.h"
#include "host.h"

namespace moe {
namespace {

constexpr int kColsPerLane = 8;
constexpr int kColsPerWave = kWave * kColsPerLane;   // 512 = 4 groups

constexpr int kRowsPerWave = 1;                      // rows per wavefront (loads of all issued together)

// One lane's 16-byte input words for its 8 columns of one row (two words for f32), and those of the
// matching up columns when the activation is gated.
template <int DT>
struct RawCols {
    uint4 g[DT == kF32 ? 2 : 1];
    uint4 u[DT == kF32 ? 2 : 1];
};

template <int DT, bool GATED>
__device__ __forceinline__ RawCols<DT> load_cols(const void* __restrict__ in, int64_t base, int64_t n, int64_t c0) {
    RawCols<DT> r;
    const int64_t ge = DT == kF32 ? 4 : 2;      // element size
    const uint4* pg = reinterpret_cast<const uint4*>((const char*)in + (base + c0) * ge);
    r.g[0] = pg[0];
    if constexpr (DT == kF32) r.g[1] = pg[1];
    if constexpr (GATED) {
        const uint4* pu = reinterpret_cast<const uint4*>((const char*)in + (base + n + c0) * ge);
        r.u[0] = pu[0];
        if constexpr (DT == kF32) r.u[1] = pu[1];
    }
    return r;
}

template <int DT>
__device__ __forceinline__ void unpack_cols(const uint4 (&w)[DT == kF32 ? 2 : 1], float (&v)[8]) {
    if constexpr (DT == kF32) {
        const uint32_t x[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = __uint_as_float(x[i]);
    } else {
        const uint32_t x[4] = {w[0].x, w[0].y, w[0].z, w[0].w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            v[2 * i] = DT == kBF16 ? bf16_to_f32((uint16_t)(x[i] & 0xFFFF)) : f16_to_f32((uint16_t)(x[i] & 0xFFFF));
            v[2 * i + 1] = DT == kBF16 ? bf16_to_f32((uint16_t)(x[i] >> 16)) : f16_to_f32((uint16_t)(x[i] >> 16));
        }
    }
}

// One wavefront's 512 columns [c0 - 8*lane, +512) of one row; this lane owns columns [c0, c0 + 8).
template <int DT, bool GATED, bool VEC>
__device__ __forceinline__ void act_quant_row(const void* __restrict__ in, int64_t base, int64_t row, int64_t n, int act,
                                              int64_t c0, int lane, const RawCols<DT>& raw, uint8_t* __restrict__ out_q,
                                              int64_t q_stride, float* __restrict__ out_s, int64_t s_stride) {
    const int64_t ncols = n;   // width of v
    float v[kColsPerLane];
    const bool full = c0 + kColsPerLane <= ncols;
    if (VEC && full) {
        unpack_cols<DT>(raw.g, v);
        if constexpr (GATED) {
            float u[8];
            unpack_cols<DT>(raw.u, u);
#pragma unroll
            for (int i = 0; i < 8; i++) v[i] = gated_act(act, v[i], u[i]);
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
        const float r = 1.0f / s;
        lo = enc4_e4m3(e4m3_quot(v[0], s, r), e4m3_quot(v[1], s, r), e4m3_quot(v[2], s, r), e4m3_quot(v[3], s, r));
        hi = enc4_e4m3(e4m3_quot(v[4], s, r), e4m3_quot(v[5], s, r), e4m3_quot(v[6], s, r), e4m3_quot(v[7], s, r));
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

template <int DT, bool GATED, bool VEC>
__global__ void __launch_bounds__(256)
act_quant_kernel(const void* __restrict__ in, int64_t in_stride, int64_t rows, int64_t n, int act,
                 uint8_t* __restrict__ out_q, int64_t q_stride, float* __restrict__ out_s, int64_t s_stride) {
    const int lane = threadIdx.x & (kWave - 1);
    // grid: x = groups of blockDim.x/64 segments of 512 columns, y = groups of kRowsPerWave rows (taken
    // in strides beyond the grid), so no index needs an integer division
    const int64_t seg = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int64_t c0 = seg * kColsPerWave + (int64_t)lane * kColsPerLane;
    if (seg * kColsPerWave >= n) return;
    const bool full = c0 + kColsPerLane <= n;
    for (int64_t r0 = (int64_t)blockIdx.y * kRowsPerWave; r0 < rows; r0 += (int64_t)gridDim.y * kRowsPerWave) {
        RawCols<DT> raw[kRowsPerWave];
        if (VEC && full) {
            // every row's loads go out before the first is used (rows past the end re-read the last)
#pragma unroll
            for (int u = 0; u < kRowsPerWave; u++) {
                const int64_t row = r0 + u < rows ? r0 + u : rows - 1;
                raw[u] = load_cols<DT, GATED>(in, row * in_stride, n, c0);
            }
        }
#pragma unroll
        for (int u = 0; u < kRowsPerWave; u++)
            if (r0 + u < rows)
                act_quant_row<DT, GATED, VEC>(in, (r0 + u) * in_stride, r0 + u, n, act, c0, lane, raw[u], out_q, q_stride,
                                              out_s, s_stride);
    }
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
    // vector loads need every lane's 8 elements 16-byte aligned: base, stride and the up offset
    const bool vec = aligned16(in) && (in_stride * esz) % 16 == 0 && (n * esz) % 16 == 0;
    const int64_t segs = ceil_div(n, kColsPerWave);                   // 512-column segments per row
    const int64_t wpb = segs < 4 ? segs : 4;                            // waves per workgroup
    const int64_t col_blocks = ceil_div(segs, wpb);
    const int64_t row_blocks = ceil_div(rows, kRowsPerWave);
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
