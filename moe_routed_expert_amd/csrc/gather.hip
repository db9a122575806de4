// One-pass gather of fp8 activation rows and their fp32 group scales through a
// dst2src map ("[MoE] Gather the cutlass MoE activation and its scales in one
// launch", Modifications: one walk of the map writes both tensors; rows are
// moved as bytes; 64-bit row bases; masked tails).
//
// MI355X design: one wavefront per destination row.  The row bytes move as
// 16-byte vectors, up to eight per lane in flight before the first store, so a
// 7168-byte row is 7 loads per lane; the row's scale words ride in the same
// wave (lanes 0..g-1) with its first chunk, so there is no second launch and
// no second walk of the map.  Stores are non-temporal.
//
// A source row usually appears several times in the map (once per routed
// expert of its token).  Each of the 8 XCDs has its own L2, so copies of one
// source row gathered on different XCDs fetch it once per XCD (about 5x the
// distinct source bytes for 1024 tokens x top-8).  From 1024 destination rows
// on, the map is walked in chunks of 8 destination rows by 8 workgroups per
// chunk, one per XCD (workgroups go to XCDs round-robin by index), and
// workgroup x copies only the rows whose source index is x mod 8: every copy of
// a source row is made on one XCD.  A negative entry (a zero row) goes by its
// destination index instead.  Shorter maps keep one wavefront per row on its
// own: there, spreading rows over more CUs beats the saved fetches.  Rows or
// strides that are not 16-byte aligned fall back to a byte loop.  Map entries
// outside [0, n_src) write a zero row, so no entry reads outside the sources.
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

constexpr int kXcds = 8;          // XCDs of the chip; workgroup i runs on XCD i mod 8
constexpr int kChunk = 8;         // destination rows per map chunk (at most 64: one map word per lane)
constexpr int kXWaves = 4;        // waves of an XCD-aware workgroup
constexpr int64_t kXcdMinRows = 1024;   // maps from this length on take the XCD-aware kernel

// Copies one row (k bytes as 16-byte vectors, k % 16 == 0) and its g scale words.
__device__ __forceinline__ void copy_row_vec(const uint8_t* __restrict__ sq, const uint32_t* __restrict__ ss,
                                             uint8_t* __restrict__ dq, uint32_t* __restrict__ ds,
                                             int64_t k, int64_t g, int lane) {
    const int64_t nvec = k / 16;
    const v4i* s4 = reinterpret_cast<const v4i*>(sq);
    v4i* d4 = reinterpret_cast<v4i*>(dq);
    for (int64_t base = 0; base < nvec; base += kWave * kVecInFlight) {
        v4i buf[kVecInFlight];
        const bool sv = base == 0 && lane < g;      // the row's scales ride with its first chunk
        uint32_t sw = 0;
        if (sv) sw = ss[lane];                      // (g == 0: no scale word is read at all)
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
}

__device__ __forceinline__ void zero_row_vec(uint8_t* __restrict__ dq, uint32_t* __restrict__ ds,
                                             int64_t k, int64_t g, int lane) {
    const v4i z = {0, 0, 0, 0};
    for (int64_t c = lane; c < k / 16; c += kWave) nt_store(reinterpret_cast<v4i*>(dq) + c, z);
    for (int64_t c = lane; c < g; c += kWave) nt_store(ds + c, 0u);
}

// 16-byte path: grid = 8 workgroups per 64-row chunk of the map.
__global__ void __launch_bounds__(64 * kXWaves)
gather_rows_scales_xcd_kernel(const uint8_t* __restrict__ src_q, int64_t src_q_stride,
                              const uint32_t* __restrict__ src_s, int64_t src_s_stride,
                              int64_t n_src, int64_t k, int64_t g, const int32_t* __restrict__ dst2src, int64_t n_dst,
                              uint8_t* __restrict__ dst_q, int64_t dst_q_stride,
                              uint32_t* __restrict__ dst_s, int64_t dst_s_stride) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int xcd = blockIdx.x % kXcds;
    const int64_t row_base = (int64_t)(blockIdx.x / kXcds) * kChunk;
    const int64_t my_row = row_base + lane;
    const bool in_map = lane < kChunk && my_row < n_dst;
    int32_t my_src = in_map ? dst2src[my_row] : -1;
    if (my_src >= n_src) my_src = -1;               // out of range: a zero row, like a negative entry
    const int home = my_src >= 0 ? my_src % kXcds : (int)(my_row % kXcds);
    const bool mine = in_map && home == xcd;
    const uint64_t mask = __ballot(mine);
    const int count = __popcll(mask);
    const int rank = __popcll(mask & ((1ull << lane) - 1));
    // the workgroup's rows in map order, dealt round-robin to its waves
    for (int r = wave; r < count; r += kXWaves) {
        const int l = __ffsll((unsigned long long)__ballot(mine && rank == r)) - 1;
        const int64_t row = row_base + l;
        const int32_t src = __builtin_amdgcn_readlane(my_src, l);
        uint8_t* dq = dst_q + row * dst_q_stride;   // int64 row bases
        uint32_t* ds = dst_s + row * dst_s_stride;
        if (src < 0)
            zero_row_vec(dq, ds, k, g, lane);
        else
            copy_row_vec(src_q + src * src_q_stride, src_s + src * src_s_stride, dq, ds, k, g, lane);
    }
}

// One wavefront per destination row: maps shorter than kXcdMinRows (VEC), and
// rows or strides that are not 16-byte aligned (byte loop).
template <bool VEC>
__global__ void __launch_bounds__(64 * kRowsPerBlock)
gather_rows_scales_kernel(const uint8_t* __restrict__ src_q, int64_t src_q_stride,
                          const uint32_t* __restrict__ src_s, int64_t src_s_stride,
                          int64_t n_src, int64_t k, int64_t g, const int32_t* __restrict__ dst2src, int64_t n_dst,
                          uint8_t* __restrict__ dst_q, int64_t dst_q_stride,
                          uint32_t* __restrict__ dst_s, int64_t dst_s_stride) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
    if (row >= n_dst) return;
    int64_t src = dst2src[row];
    if (src >= n_src) src = -1;                     // out of range: a zero row, like a negative entry
    uint8_t* dq = dst_q + row * dst_q_stride;   // int64 row base
    uint32_t* ds = dst_s + row * dst_s_stride;
    if constexpr (VEC) {
        if (src < 0)
            zero_row_vec(dq, ds, k, g, lane);
        else
            copy_row_vec(src_q + src * src_q_stride, src_s + src * src_s_stride, dq, ds, k, g, lane);
    } else {
        if (src < 0) {
            for (int64_t c = lane; c < k; c += kWave) dq[c] = 0;
            for (int64_t c = lane; c < g; c += kWave) nt_store(ds + c, 0u);
            return;
        }
        const uint8_t* sq = src_q + src * src_q_stride;
        const uint32_t* ss = src_s + src * src_s_stride;
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
    auto s = as_stream(stream);
    if (vec && n_dst >= kXcdMinRows) {
        const int64_t blocks = ceil_div(n_dst, kChunk) * kXcds;
        if (blocks > 0x7FFFFFFF) return MOE_ERR_SHAPE;
        hipLaunchKernelGGL(gather_rows_scales_xcd_kernel, dim3((unsigned)blocks), dim3(64 * kXWaves), 0, s,
                           (const uint8_t*)src_q, src_q_stride, (const uint32_t*)src_s, src_s_stride, n_src, k, g,
                           dst2src, n_dst, (uint8_t*)dst_q, dst_q_stride, (uint32_t*)dst_s, dst_s_stride);
        return launch_status();
    }
    const int64_t blocks = ceil_div(n_dst, kRowsPerBlock);
    if (blocks > 0x7FFFFFFF) return MOE_ERR_SHAPE;
    auto kern = vec ? gather_rows_scales_kernel<true> : gather_rows_scales_kernel<false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * kRowsPerBlock), 0, s,
                       (const uint8_t*)src_q, src_q_stride, (const uint32_t*)src_s, src_s_stride, n_src, k, g,
                       dst2src, n_dst, (uint8_t*)dst_q, dst_q_stride, (uint32_t*)dst_s, dst_s_stride);
    return launch_status();
}
