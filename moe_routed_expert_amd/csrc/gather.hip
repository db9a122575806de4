// One-pass gather of fp8 activation rows and their fp32 group scales through a
// dst2src map ("[MoE] Gather the cutlass MoE activation and its scales in one
// launch", Modifications: one walk of the map writes both tensors; rows are
// moved as bytes; 64-bit row bases; masked tails).
//
// MI355X design: one wavefront per destination row.  The row bytes move as
// 16-byte vectors, up to eight per lane in flight before the first store, so a
// 7168-byte row is 7 loads per lane; the row's scale words ride in the same
// wave (lanes 0..g-1) with its first chunk, so there is no second launch and
// no second walk of the map.  Stores are non-temporal.  Rows or strides that
// are not 16-byte aligned fall back to a byte loop.
#include "device.h"
#include "host.h"

namespace moe {
namespace {

constexpr int kRowsPerBlock = 4;   // 4 waves, one row each
constexpr int kVecInFlight = 8;    // 16-byte loads per lane issued before the first store

// Destination rows are written once and read by a later kernel, so they are
// stored non-temporally (they stream past the caches instead of evicting the
// source rows, which repeat across the map).
__device__ __forceinline__ void nt_store(v4i* p, v4i v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void nt_store(uint32_t* p, uint32_t v) { __builtin_nontemporal_store(v, p); }

template <bool VEC>
__global__ void __launch_bounds__(64 * kRowsPerBlock)
gather_rows_scales_kernel(const uint8_t* __restrict__ src_q, int64_t src_q_stride,
                          const uint32_t* __restrict__ src_s, int64_t src_s_stride,
                          int64_t k, int64_t g, const int32_t* __restrict__ dst2src, int64_t n_dst,
                          uint8_t* __restrict__ dst_q, int64_t dst_q_stride,
                          uint32_t* __restrict__ dst_s, int64_t dst_s_stride) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    if (row >= n_dst) return;
    const int64_t src = dst2src[row];
    uint8_t* dq = dst_q + row * dst_q_stride;   // int64 row base
    uint32_t* ds = dst_s + row * dst_s_stride;
    if (src < 0) {
        if constexpr (VEC) {
            const v4i z = {0, 0, 0, 0};
            for (int64_t c = lane; c < k / 16; c += kWave) nt_store(reinterpret_cast<v4i*>(dq) + c, z);
        } else {
            for (int64_t c = lane; c < k; c += kWave) dq[c] = 0;
        }
        for (int64_t c = lane; c < g; c += kWave) nt_store(ds + c, 0u);
        return;
    }
    const uint8_t* sq = src_q + src * src_q_stride;
    const uint32_t* ss = src_s + src * src_s_stride;
    if constexpr (VEC) {
        const int64_t nvec = k / 16;
        const v4i* s4 = reinterpret_cast<const v4i*>(sq);
        v4i* d4 = reinterpret_cast<v4i*>(dq);
        for (int64_t base = 0; base < nvec; base += kWave * kVecInFlight) {
            v4i buf[kVecInFlight];
            const bool sv = base == 0 && lane < g;      // the row's scales ride with its first chunk
            const uint32_t sw = ss[sv ? lane : 0];
            // unconditional loads (indices clamped to the row) so all of them issue back to back
#pragma unroll
            for (int i = 0; i < kVecInFlight; i++) {
                const int64_t c = base + i * kWave + lane;
                buf[i] = s4[c < nvec ? c : nvec - 1];
            }
#pragma unroll
            for (int i = 0; i < kVecInFlight; i++) {
                const int64_t c = base + i * kWave + lane;
                if (c < nvec) nt_store(d4 + c, buf[i]);
            }
            if (sv) nt_store(ds + lane, sw);
        }
        // scale words beyond the first 64 (and all of them for an empty row)
        for (int64_t c = lane + (nvec > 0 ? kWave : 0); c < g; c += kWave) nt_store(ds + c, ss[c]);
    } else {
        for (int64_t c = lane; c < k; c += kWave) dq[c] = sq[c];
        for (int64_t c = lane; c < g; c += kWave) nt_store(ds + c, ss[c]);
    }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_gather_rows_scales(const void* src_q, int64_t src_q_stride,
                                      const float* src_s, int64_t src_s_stride,
                                      int64_t n_src, int64_t k, int64_t g,
                                      const int32_t* dst2src, int64_t n_dst,
                                      void* dst_q, int64_t dst_q_stride,
                                      float* dst_s, int64_t dst_s_stride,
                                      void* stream) {
    if (n_dst < 0 || k < 0 || g < 0 || n_src < 0) return MOE_ERR_SHAPE;
    if (n_dst == 0) return MOE_OK;                        // empty map: nothing launched
    if (!dst2src) return MOE_ERR_NULL;
    if ((k > 0 && (!src_q || !dst_q)) || (g > 0 && (!src_s || !dst_s))) return MOE_ERR_NULL;
    if (n_src == 0) return MOE_ERR_SHAPE;                 // a non-empty map needs sources
    if (src_q_stride < k || dst_q_stride < k || src_s_stride < g || dst_s_stride < g) return MOE_ERR_SHAPE;
    const bool vec = k % 16 == 0 && src_q_stride % 16 == 0 && dst_q_stride % 16 == 0 &&
                     aligned16(src_q) && aligned16(dst_q);
    const int64_t blocks = ceil_div(n_dst, kRowsPerBlock);
    if (blocks > 0x7FFFFFFF) return MOE_ERR_SHAPE;
    dim3 grid((unsigned)blocks), block(64 * kRowsPerBlock);
    auto s = as_stream(stream);
    if (vec)
        hipLaunchKernelGGL(gather_rows_scales_kernel<true>, grid, block, 0, s,
                           (const uint8_t*)src_q, src_q_stride, (const uint32_t*)src_s, src_s_stride, k, g,
                           dst2src, n_dst, (uint8_t*)dst_q, dst_q_stride, (uint32_t*)dst_s, dst_s_stride);
    else
        hipLaunchKernelGGL(gather_rows_scales_kernel<false>, grid, block, 0, s,
                           (const uint8_t*)src_q, src_q_stride, (const uint32_t*)src_s, src_s_stride, k, g,
                           dst2src, n_dst, (uint8_t*)dst_q, dst_q_stride, (uint32_t*)dst_s, dst_s_stride);
    return launch_status();
}
