// Block-FP8 GEMM in slot mode: one output row per route, each route streaming
// its own expert ("perf(moe): skip inactive block-fp8 decode routes", opening
// section: the shared decode kernel serves both gate/up and down; a negative
// slot writes zero to the route's output tile and returns before reading
// activations, expert weights, scales or routing weights).
//
// MI355X design.  At decode sizes every weight byte is used once, so the
// kernel is an HBM stream.  A workgroup owns one route and 16 output rows; its
// four waves split K (128-wide blocks) and each wave keeps UNROLL blocks of
// loads in flight: per block a lane fetches 2x16 B of weights and the matching
// 2x16 B of the activation row.  The fp8 bytes go straight into one
// 16x16x128 e4m3 MFMA per block -- no decode to fp32 on the VALU -- with the
// activation row broadcast over the 16 MFMA rows, and the block partial is
// scaled by a_s[kb] * w_s[n/128][kb] into an fp32 accumulator (one FMA per
// block).  Split-K partials are combined in LDS in wave order, so results are
// deterministic.  A 16-row tile never straddles a 128-row scale block, so the
// weight scale is one scalar load per block.
//
// The gate/up variant takes the bf16 token row instead of an fp8 row and
// quantizes each 128-column group in the prologue of the block that needs it
// (wave amax, amax/448, v/s rounded to e4m3), so the decode step needs no
// separate quantization launch.
#include "device.h"
#include "host.h"

namespace moe {

constexpr int kTileN = 16;
constexpr int kKSplit = 4;      // waves per workgroup, splitting K
constexpr int kUnroll = 4;      // K blocks in flight per wave

// Per-lane K offsets inside a 128-wide block: two 16-byte chunks, quarter q = lane/16
// takes [16q, 16q+16) and [64+16q, 64+16q+16).  A and B fragments use the same map.
__device__ __forceinline__ v8i make_frag(uint4 lo, uint4 hi) {
    v8i f;
    f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
    f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
    return f;
}

// Quantize one 128-column group of a bf16 row held across the wave (2 values per
// lane: columns 2*lane, 2*lane+1) into the LDS slot `dst` (128 bytes); returns the scale.
__device__ __forceinline__ float quant_group_bf16_to_lds(const uint16_t* __restrict__ xrow, int lane,
                                                         uint8_t* dst) {
    const uint32_t pair = reinterpret_cast<const uint32_t*>(xrow)[lane];
    const float v0 = bf16_to_f32((uint16_t)(pair & 0xFFFF));
    const float v1 = bf16_to_f32((uint16_t)(pair >> 16));
    float amax = __builtin_fmaxf(__builtin_fabsf(v0), __builtin_fabsf(v1));
    amax = wave_max(amax);
    const float s = amax / 448.0f;
    const uint32_t codes = s != 0.0f ? enc2_e4m3(v0 / s, v1 / s) : 0u;
    reinterpret_cast<uint16_t*>(dst)[lane] = (uint16_t)codes;
    return s;
}

template <int OUT_DT, bool XBF16>
__global__ void __launch_bounds__(kWave * kKSplit)
slot_gemv_kernel(const void* __restrict__ a_ptr, int64_t a_stride, const float* __restrict__ a_s,
                 int64_t a_s_stride, const uint8_t* __restrict__ w_q, int64_t w_stride_e, int64_t w_stride_n,
                 const float* __restrict__ w_s, int64_t w_s_stride_e, int64_t w_s_stride_n, int64_t K,
                 const int32_t* __restrict__ slot_ids, int64_t a_row_div, void* __restrict__ out,
                 int64_t out_stride) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t r = blockIdx.y;
    const int64_t n0 = (int64_t)blockIdx.x * kTileN;
    const int slot = slot_ids[r];
    if (slot < 0) {   // inactive route: zero tile, nothing else read
        if (threadIdx.x < kTileN) store_from_f32<OUT_DT>(out, r * out_stride + n0 + threadIdx.x, 0.0f);
        return;
    }
    const int nkb = (int)(K / 128);
    const int kb_begin = wave * nkb / kKSplit;
    const int kb_end = (wave + 1) * nkb / kKSplit;
    const int q16 = (lane / 16) * 16;
    const int64_t ar = r / a_row_div;
    const uint8_t* wrow = w_q + (int64_t)slot * w_stride_e + (n0 + (lane & 15)) * w_stride_n + q16;
    const float* wsrow = w_s + (int64_t)slot * w_s_stride_e + (n0 / 128) * w_s_stride_n;

    __shared__ float red[kKSplit][kTileN];
    __shared__ __attribute__((aligned(16))) uint8_t xq[XBF16 ? kKSplit : 1][kUnroll][128];

    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int kb = kb_begin; kb < kb_end; kb += kUnroll) {
        uint4 b_lo[kUnroll], b_hi[kUnroll], a_lo[kUnroll], a_hi[kUnroll];
        float sa[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            if (kb + u < kb_end) {
                const uint8_t* wp = wrow + (int64_t)(kb + u) * 128;
                b_lo[u] = *reinterpret_cast<const uint4*>(wp);
                b_hi[u] = *reinterpret_cast<const uint4*>(wp + 64);
            }
        }
        if constexpr (XBF16) {
            const uint16_t* xrow = (const uint16_t*)a_ptr + ar * a_stride;
#pragma unroll
            for (int u = 0; u < kUnroll; u++)
                if (kb + u < kb_end) sa[u] = quant_group_bf16_to_lds(xrow + (int64_t)(kb + u) * 128, lane, xq[wave][u]);
            // each wave reads back only its own LDS rows, and one wave's LDS operations
            // execute in order, so a wave-scope fence (no s_barrier) orders the exchange
            wave_lds_fence();
#pragma unroll
            for (int u = 0; u < kUnroll; u++) {
                if (kb + u < kb_end) {
                    a_lo[u] = *reinterpret_cast<const uint4*>(&xq[wave][u][q16]);
                    a_hi[u] = *reinterpret_cast<const uint4*>(&xq[wave][u][64 + q16]);
                }
            }
        } else {
            const uint8_t* arow = (const uint8_t*)a_ptr + ar * a_stride + q16;
            const float* asrow = a_s + ar * a_s_stride;
#pragma unroll
            for (int u = 0; u < kUnroll; u++) {
                if (kb + u < kb_end) {
                    a_lo[u] = *reinterpret_cast<const uint4*>(arow + (int64_t)(kb + u) * 128);
                    a_hi[u] = *reinterpret_cast<const uint4*>(arow + (int64_t)(kb + u) * 128 + 64);
                    sa[u] = asrow[kb + u];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            if (kb + u < kb_end) {
                const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
                const v4f p = mfma16x16x128_e4m3(make_frag(a_lo[u], a_hi[u]), make_frag(b_lo[u], b_hi[u]), zero);
                const float sc = sa[u] * wsrow[kb + u];
                acc += p * sc;
            }
        }
        if constexpr (XBF16) wave_lds_fence();   // LDS slots are rewritten next round
    }
    if (lane < kTileN) red[wave][lane] = acc[0];   // row 0 of the MFMA tile: C[0][lane]
    __syncthreads();
    if (wave == 0 && lane < kTileN) {
        float t = red[0][lane];
#pragma unroll
        for (int w = 1; w < kKSplit; w++) t += red[w][lane];
        store_from_f32<OUT_DT>(out, r * out_stride + n0 + lane, t);
    }
}

template <int OUT_DT, bool XBF16>
static void launch_slot_gemv(hipStream_t st, int64_t rows, int64_t N, const void* a, int64_t a_stride,
                             const float* a_s, int64_t a_s_stride, const uint8_t* w_q, int64_t w_stride_e,
                             int64_t w_stride_n, const float* w_s, int64_t w_s_stride_e, int64_t w_s_stride_n,
                             int64_t K, const int32_t* slots, int64_t a_row_div, void* out, int64_t out_stride) {
    dim3 grid((unsigned)(N / kTileN), (unsigned)rows);
    hipLaunchKernelGGL((slot_gemv_kernel<OUT_DT, XBF16>), grid, dim3(kWave * kKSplit), 0, st, a, a_stride, a_s,
                       a_s_stride, w_q, w_stride_e, w_stride_n, w_s, w_s_stride_e, w_s_stride_n, K, slots,
                       a_row_div, out, out_stride);
}

// Slot-mode launch used by moe_bf8_grouped_gemm (fp8 A) and by the fused decode (bf16 A).
int slot_gemm_launch(hipStream_t st, bool a_is_bf16, const void* a, int64_t a_stride, const float* a_s,
                     int64_t a_s_stride, const uint8_t* w_q, int64_t w_stride_e, int64_t w_stride_n,
                     const float* w_s, int64_t w_s_stride_e, int64_t w_s_stride_n, int64_t N, int64_t K,
                     const int32_t* slots, int64_t rows, int64_t a_row_div, void* out, int out_dt,
                     int64_t out_stride) {
    if (rows > 65535 || N / kTileN > 0x7FFFFFFF) return MOE_ERR_SHAPE;
    if (a_is_bf16) {
        launch_slot_gemv<kF32, true>(st, rows, N, a, a_stride, a_s, a_s_stride, w_q, w_stride_e, w_stride_n, w_s,
                                     w_s_stride_e, w_s_stride_n, K, slots, a_row_div, out, out_stride);
    } else if (out_dt == MOE_F32) {
        launch_slot_gemv<kF32, false>(st, rows, N, a, a_stride, a_s, a_s_stride, w_q, w_stride_e, w_stride_n, w_s,
                                      w_s_stride_e, w_s_stride_n, K, slots, a_row_div, out, out_stride);
    } else if (out_dt == MOE_BF16) {
        launch_slot_gemv<kBF16, false>(st, rows, N, a, a_stride, a_s, a_s_stride, w_q, w_stride_e, w_stride_n, w_s,
                                       w_s_stride_e, w_s_stride_n, K, slots, a_row_div, out, out_stride);
    } else {
        launch_slot_gemv<kF16, false>(st, rows, N, a, a_stride, a_s, a_s_stride, w_q, w_stride_e, w_stride_n, w_s,
                                      w_s_stride_e, w_s_stride_n, K, slots, a_row_div, out, out_stride);
    }
    return launch_status();
}

}  // namespace moe
