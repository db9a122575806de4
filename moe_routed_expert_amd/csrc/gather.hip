// One-pass gather of fp8 activation rows and their fp32 group scales through a
// dst2src map ("[MoE] Gather the cutlass MoE activation and its scales in one
// launch", Modifications: one walk of the map writes both tensors; rows are
// moved as bytes; 64-bit row bases; masked tails).
//
// MI355X design: one wavefront per destination row.  The row bytes move as
// 16-byte vectors, eight per lane in flight before the first store, so a
// 7168-byte row is 7 loads per lane; the row's scale words ride in the same
// wave (lanes 0..g-1), so there is no second launch and no second walk of the
// map.  Rows or strides that are not 16-byte aligned fall back to a byte loop.
#include "device.h"
#include "host.h"

namespace moe {
namespace {

constexpr int kRowsPerBlock = 4;   // 4 waves, one row each
constexpr int kVecInFlight = 8;

template <bool VEC>
__global__ void __launch_bounds__(256)
gather_rows_scales_kernel(const uint8_t* __restrict__ src_q, int64_t src_q_stride,
                          const uint32_t* __restrict__ src_s, int64_t src_s_stride,
                          int64_t k, int64_t g, const int32_t* __restrict__ dst2src, int64_t n_dst,
                          uint8_t* __restrict__ dst_q, int64_t dst_q_stride,
                          uint32_t* __restrict__ dst_s, int64_t dst_s_stride) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = threadIdx.x / kWave;
    for (int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + wave; row < n_dst;
         row += (int64_t)gridDim.x * kRowsPerBlock) {
        const int64_t src = dst2src[row];
        uint8_t* dq = dst_q + row * dst_q_stride;   // int64 row base
        uint32_t* ds = dst_s + row * dst_s_stride;
        if (src < 0) {
            if constexpr (VEC) {
                const uint4 z = make_uint4(0, 0, 0, 0);
                for (int64_t c = lane; c < k / 16; c += kWave) reinterpret_cast<uint4*>(dq)[c] = z;
            } else {
                for (int64_t c = lane; c < k; c += kWave) dq[c] = 0;
            }
            for (int64_t c = lane; c < g; c += kWave) ds[c] = 0u;
            continue;
        }
        const uint8_t* sq = src_q + src * src_q_stride;
        const uint32_t* ss = src_s + src * src_s_stride;
        // scales first: one word per lane, issued before the row stream
        uint32_t sw[2];
        bool sv[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            int64_t c = lane + i * kWave;
            sv[i] = c < g;
            if (sv[i]) sw[i] = ss[c];
        }
        if constexpr (VEC) {
            const int64_t nvec = k / 16;
            const uint4* s4 = reinterpret_cast<const uint4*>(sq);
            uint4* d4 = reinterpret_cast<uint4*>(dq);
            for (int64_t base = 0; base < nvec; base += kWave * kVecInFlight) {
                uint4 buf[kVecInFlight];
#pragma unroll
                for (int i = 0; i < kVecInFlight; i++) {
                    int64_t c = base + i * kWave + lane;
                    if (c < nvec) buf[i] = s4[c];
                }
#pragma unroll
                for (int i = 0; i < kVecInFlight; i++) {
                    int64_t c = base + i * kWave + lane;
                    if (c < nvec) d4[c] = buf[i];
                }
            }
        } else {
            for (int64_t c = lane; c < k; c += kWave) dq[c] = sq[c];
        }
#pragma unroll
        for (int i = 0; i < 2; i++)
            if (sv[i]) ds[lane + i * kWave] = sw[i];
        for (int64_t c = lane + 2 * kWave; c < g; c += kWave) ds[c] = ss[c];
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
    int64_t blocks = ceil_div(n_dst, kRowsPerBlock);
    if (blocks > 65536) blocks = 65536;
    dim3 grid((unsigned)blocks), block(256);
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
