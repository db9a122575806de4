// Routing-weighted reduce of each token's top-k route outputs ("perf(moe):
// skip inactive block-fp8 decode routes", opening section: the reduction reads
// the route buffers, and a negative slot's routing weight is never read).
//
// MI355X design: HBM-bound elementwise pass.  A thread owns consecutive hidden
// columns of one token (8 with 16-byte loads and stores when the rows allow it,
// else 4), walks the top-k routes in ascending order with an fp32 accumulator
// (the order is fixed, so results are deterministic), and writes its bf16
// values with one store.  Slot ids and routing weights of the token are
// wave-uniform loads.
#include "device.h"
#include "host.h"

namespace moe {
namespace {

constexpr int kRoutesPerPass = 8;
__device__ const float kZeroWeight = 0.0f;

// Eight columns h0..h0+7 of row `row` as fp32 with 16-byte loads (rows 16-byte aligned, H % 8 == 0).
template <int DT>
__device__ __forceinline__ void load8_as_f32(const void* y, int64_t off, float* v) {
    if constexpr (DT == kF32) {
        const float4 a = reinterpret_cast<const float4*>((const float*)y + off)[0];
        const float4 b = reinterpret_cast<const float4*>((const float*)y + off)[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        const uint4 r = *reinterpret_cast<const uint4*>((const uint16_t*)y + off);
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint16_t lo = (uint16_t)(w[i] & 0xFFFF), hi = (uint16_t)(w[i] >> 16);
            v[2 * i] = DT == kBF16 ? bf16_to_f32(lo) : f16_to_f32(lo);
            v[2 * i + 1] = DT == kBF16 ? bf16_to_f32(hi) : f16_to_f32(hi);
        }
    }
}

// VEC: 8 columns per thread with 16-byte loads and stores (H, strides and bases allow it); else 4.
template <int DT, bool VEC>
__global__ void __launch_bounds__(256)
topk_reduce_kernel(const void* __restrict__ y, int64_t y_stride, const int32_t* __restrict__ slot_ids,
                   const int32_t* __restrict__ route_rows, const float* __restrict__ weights, int64_t T,
                   int64_t topk, int64_t H, uint16_t* __restrict__ out, int64_t out_stride) {
    constexpr int CPT = VEC ? 8 : 4;             // columns per thread
    const int64_t chunks = ceil_div(H, CPT);
    const int64_t t = blockIdx.y;
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T || c >= chunks) return;
    const int64_t h0 = c * CPT;
    // columns of this thread, clamped into the row (the clamped tail values are never stored)
    int64_t col[CPT];
#pragma unroll
    for (int i = 0; i < CPT; i++) col[i] = h0 + i < H ? h0 + i : H - 1;
    float acc[CPT];
#pragma unroll
    for (int i = 0; i < CPT; i++) acc[i] = 0.0f;
    for (int64_t j0 = 0; j0 < topk; j0 += kRoutesPerPass) {
        // one pass issues the loads of up to 8 routes back to back with no per-route branch; an
        // inactive route reads its routing weight from a constant zero instead of the weights
        // array, and its y values are dropped by a select
        int32_t sl[kRoutesPerPass];
        int64_t rt[kRoutesPerPass];
#pragma unroll
        for (int u = 0; u < kRoutesPerPass; u++) {
            rt[u] = t * topk + (j0 + u < topk ? j0 + u : topk - 1);
            sl[u] = slot_ids[rt[u]];
        }
        float w[kRoutesPerPass], v[kRoutesPerPass][CPT];
        bool on[kRoutesPerPass];
#pragma unroll
        for (int u = 0; u < kRoutesPerPass; u++) {
            on[u] = j0 + u < topk && sl[u] >= 0;
            w[u] = *(on[u] ? weights + rt[u] : &kZeroWeight);
            const int64_t rr = route_rows ? (int64_t)route_rows[rt[u]] : rt[u];
            const int64_t row = on[u] ? rr : 0;
            if constexpr (VEC) {
                load8_as_f32<DT>(y, row * y_stride + h0, v[u]);
            } else {
#pragma unroll
                for (int i = 0; i < CPT; i++) v[u][i] = load_as_f32<DT>(y, row * y_stride + col[i]);
            }
        }
#pragma unroll
        for (int u = 0; u < kRoutesPerPass; u++)
#pragma unroll
            for (int i = 0; i < CPT; i++) acc[i] = on[u] ? acc[i] + w[u] * v[u][i] : acc[i];
    }
    uint16_t* o = out + t * out_stride + h0;
    if constexpr (VEC) {
        uint32_t p[4];
#pragma unroll
        for (int i = 0; i < 4; i++)
            p[i] = (uint32_t)f32_to_bf16(acc[2 * i]) | ((uint32_t)f32_to_bf16(acc[2 * i + 1]) << 16);
        *reinterpret_cast<uint4*>(o) = make_uint4(p[0], p[1], p[2], p[3]);
    } else if (h0 + 4 <= H && (reinterpret_cast<uintptr_t>(o) & 7u) == 0) {
        const uint32_t lo = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
        *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
    } else {
        for (int i = 0; i < 4 && h0 + i < H; i++) o[i] = f32_to_bf16(acc[i]);
    }
}

template <int DT>
void launch_reduce(hipStream_t st, bool vec, const void* y, int64_t y_stride, const int32_t* slot_ids,
                   const int32_t* route_rows, const float* weights, int64_t T, int64_t topk, int64_t H,
                   uint16_t* out, int64_t out_stride) {
    const int64_t chunks = ceil_div(H, vec ? 8 : 4);
    dim3 grid((unsigned)ceil_div(chunks, 256), (unsigned)T);
    if (vec)
        hipLaunchKernelGGL((topk_reduce_kernel<DT, true>), grid, dim3(256), 0, st, y, y_stride, slot_ids, route_rows,
                           weights, T, topk, H, out, out_stride);
    else
        hipLaunchKernelGGL((topk_reduce_kernel<DT, false>), grid, dim3(256), 0, st, y, y_stride, slot_ids,
                           route_rows, weights, T, topk, H, out, out_stride);
}

}  // namespace

int topk_reduce_launch(hipStream_t st, const void* y, int y_dt, int64_t y_stride, const int32_t* slot_ids,
                       const int32_t* route_rows, const float* weights, int64_t T, int64_t topk, int64_t H,
                       uint16_t* out, int64_t out_stride) {
    // 16-byte rows of y and out: every thread's 8 columns are one aligned vector
    const bool vec = H % 8 == 0 && y_stride % 8 == 0 && out_stride % 8 == 0 && aligned16(y) && aligned16(out);
    if (y_dt == MOE_F32)
        launch_reduce<kF32>(st, vec, y, y_stride, slot_ids, route_rows, weights, T, topk, H, out, out_stride);
    else if (y_dt == MOE_BF16)
        launch_reduce<kBF16>(st, vec, y, y_stride, slot_ids, route_rows, weights, T, topk, H, out, out_stride);
    else
        launch_reduce<kF16>(st, vec, y, y_stride, slot_ids, route_rows, weights, T, topk, H, out, out_stride);
    return launch_status();
}

}  // namespace moe

using namespace moe;

extern "C" int moe_topk_reduce(const void* y, int y_dt, int64_t y_stride, const int32_t* slot_ids,
                               const int32_t* route_rows, const float* weights, int64_t T, int64_t topk,
                               int64_t H, uint16_t* out_bf16, int64_t out_stride, void* stream) {
    if (T < 0 || topk < 0 || H < 0) return MOE_ERR_SHAPE;
    if (!dtype_ok(y_dt)) return MOE_ERR_DTYPE;
    if (T == 0 || H == 0) return MOE_OK;
    if (!out_bf16 || (topk > 0 && (!slot_ids || !weights || !y))) return MOE_ERR_NULL;
    if (out_stride < H || (topk > 0 && y_stride < H)) return MOE_ERR_SHAPE;
    if (T > 65535) return MOE_ERR_SHAPE;
    return topk_reduce_launch(as_stream(stream), y, y_dt, y_stride, slot_ids, route_rows, weights, T, topk, H,
                              out_bf16, out_stride);
}
