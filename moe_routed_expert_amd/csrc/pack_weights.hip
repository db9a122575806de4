// Expert banks in the grouped GEMMs' operand order (moe_pack_weights).
//
// Not a step of the pages' method: a one-time copy of static weights.  A grouped
// GEMM wave reads, per 128-wide K block, 32 bytes of each of its 16 weight rows
// per lane (as two 16-byte pieces).  In a row-major bank one 1 KiB load then
// touches 64 bytes of 16 rows that lie a row (K or K/2 bytes) apart, and a bank
// streams at about 5.4 TB/s on MI355X; read 1 KiB at a time from contiguous
// bytes it streams at about 6.3 TB/s.  The packed order stores, per expert, per
// 16-row group and per K block, the group's block as the pieces in the order the
// 64 lanes load them, so every load of the GEMM reads contiguous bytes.
//
// One thread per 16-byte piece of the packed bank, so the writes are contiguous;
// the reads gather 16-byte pieces of the row-major bank.
#include "device.h"
#include "host.h"

namespace moe {
namespace {

__global__ void __launch_bounds__(256)
pack_weights_kernel(const uint8_t* __restrict__ w, int64_t w_stride_e, int64_t w_stride_n, int64_t row_bytes,
                    int64_t step, uint8_t* __restrict__ out, int64_t out_stride_e, int64_t pieces_per_expert,
                    int64_t total) {
    const int64_t nsteps = row_bytes / step;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e = i / pieces_per_expert, r = i - e * pieces_per_expert;
        // piece p of block (g, s): a block holds `step` pieces (16 rows x step bytes)
        const int64_t blk = r / step, p = r - blk * step;
        const int64_t g = blk / nsteps, s = blk - g * nsteps;
        const int64_t row = 16 * g + (p & 15);
        const int64_t col = s * step + 64 * (p >> 6) + 16 * ((p & 63) >> 4);
        const uint4 v = *reinterpret_cast<const uint4*>(w + e * w_stride_e + row * w_stride_n + col);
        *reinterpret_cast<uint4*>(out + e * out_stride_e + 16 * r) = v;
    }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_pack_weights(const uint8_t* w, int64_t w_stride_e, int64_t w_stride_n, int64_t n_experts, int64_t N,
                                int64_t row_bytes, int64_t step_bytes, uint8_t* out, int64_t out_stride_e,
                                void* stream) {
    if (n_experts < 0 || N < 0 || row_bytes < 0) return MOE_ERR_SHAPE;
    if (step_bytes != 64 && step_bytes != 128) return MOE_ERR_SHAPE;
    if (N % 16 || row_bytes % step_bytes) return MOE_ERR_SHAPE;
    if (n_experts == 0 || N == 0 || row_bytes == 0) return MOE_OK;
    if (!w || !out) return MOE_ERR_NULL;
    if (w_stride_n < row_bytes) return MOE_ERR_SHAPE;
    if (n_experts > 1 && (w_stride_e < N * w_stride_n || out_stride_e < N * row_bytes)) return MOE_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(out) || w_stride_n % 16 || w_stride_e % 16 || out_stride_e % 16)
        return MOE_ERR_ALIGN;
    // the two byte ranges must not meet (the copy reads and writes in no fixed order)
    const uint64_t w0 = reinterpret_cast<uintptr_t>(w), o0 = reinterpret_cast<uintptr_t>(out);
    const uint64_t w1 = w0 + (uint64_t)((n_experts - 1) * w_stride_e + (N - 1) * w_stride_n + row_bytes);
    const uint64_t o1 = o0 + (uint64_t)((n_experts - 1) * out_stride_e + N * row_bytes);
    if (w0 < o1 && o0 < w1) return MOE_ERR_SHAPE;
    const int64_t per_expert = N * row_bytes / 16;
    const int64_t total = per_expert * n_experts;
    const int64_t blocks = ceil_div(total, 256);
    hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)(blocks < 16384 ? blocks : 16384)), dim3(256), 0,
                       as_stream(stream), w, w_stride_e, w_stride_n, row_bytes, step_bytes, out, out_stride_e,
                       per_expert, total);
    return launch_status();
}
