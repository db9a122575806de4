// Block-FP8 grouped GEMM for prefill: rows sorted by expert, each expert's rows
// times that expert's weights ("perf(dsfp4): pick the grouped-prefill tile
// from route density on sm_89": the M tile follows rows per expert and
// BLOCK_K is 128, one block-scale pair per K step).
//
// MI355X design.
//  * Tile BM x 128 x 128 (BM in {16, 32, 64, 128}); 4 waves, each owning 32 of
//    the 128 output columns for all BM rows.  BN = 128 keeps every tile inside
//    one 128x128 weight-scale block, so the weight scale is one scalar per K step.
//  * Weights are the dominant HBM stream and each weight byte of a tile is used
//    by one wave only, so they go global -> registers directly in MFMA operand
//    order (no LDS round trip), one K step ahead of the MFMAs.
//  * The A tile (BM rows x 128 bytes per K step) is shared by the 4 waves: it is
//    staged through a double-buffered LDS tile stored in fragment order (each
//    lane's 32 bytes contiguous), so the MFMA operand reads are conflict-free.
//  * Per K step: p = A*W with a fresh 16x16x128 e4m3 MFMA, then
//    acc += p * (a_s[row][kb] * w_s[kb]) in fp32.
//  * Work map: M tiles are (expert, 0..ceil(rows_e/BM)-1); the grid is an upper
//    bound (ceil(m_rows/BM) + E tiles) fixed by scalars, and each workgroup finds
//    its (expert, m0) from the device offsets with a block scan, so the launch
//    can be captured.  Workgroup ids are remapped so that consecutive tiles of
//    one M tile land on the same XCD (the dispatcher deals workgroups to the 8
//    XCDs round-robin), keeping the A tile in that XCD's L2.
#include "device.h"
#include "host.h"

namespace moe {

constexpr int kGBN = 128;
constexpr int kGThreads = 256;
constexpr int kXcds = 8;
constexpr int kMaxExpertsScan = 4 * kGThreads;   // experts handled by the in-kernel scan

// Exclusive block scan of one int per thread (256 threads).
__device__ __forceinline__ int block_exclusive_scan(int v, int* lds4, int& total) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    int x = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int y = __shfl_up(x, d, kWave);
        if (lane >= d) x += y;
    }
    if (lane == kWave - 1) lds4[wave] = x;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; w++) base += lds4[w];
    total = lds4[0] + lds4[1] + lds4[2] + lds4[3];
    return base + x - v;
}

template <int BM, int OUT_DT>
__global__ void __launch_bounds__(kGThreads)
grouped_gemm_kernel(const uint8_t* __restrict__ a_q, int64_t a_stride, const float* __restrict__ a_s,
                    int64_t a_s_stride, const uint8_t* __restrict__ w_q, int64_t w_stride_e, int64_t w_stride_n,
                    const float* __restrict__ w_s, int64_t w_s_stride_e, int64_t w_s_stride_n, int n_experts,
                    int64_t K, const int32_t* __restrict__ offsets, int n_tiles_n, int grid_per_xcd,
                    void* __restrict__ out, int64_t out_stride) {
    constexpr int MS = BM / 16;                 // 16-row MFMA sub-tiles
    constexpr int A_CHUNKS = BM * 8;            // 16-byte chunks of one A K-step
    constexpr int A_PER_THREAD = (A_CHUNKS + kGThreads - 1) / kGThreads;
    __shared__ __attribute__((aligned(32))) uint8_t a_lds[2][BM * 128];
    __shared__ float sa_lds[2][BM];
    __shared__ int scan_lds[4];
    __shared__ int tile_info[3];                // expert, row begin, row end

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    // XCD-aware remap of the linear workgroup id
    const int bid = blockIdx.x;
    const int logical = (bid % kXcds) * grid_per_xcd + bid / kXcds;
    const int m_tile = logical / n_tiles_n, n_tile = logical % n_tiles_n;

    // ---- find (expert, m0) for this M tile from the device offsets ----
    int local = 0, my_tiles[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int e = threadIdx.x * 4 + i;
        int t = 0;
        if (e < n_experts) t = (offsets[e + 1] - offsets[e] + BM - 1) / BM;
        my_tiles[i] = t;
        local += t;
    }
    int total;
    int before = block_exclusive_scan(local, scan_lds, total);
    if (threadIdx.x == 0) tile_info[0] = -1;
    __syncthreads();
    if (m_tile >= before && m_tile < before + local) {
        int acc_t = before;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            if (m_tile >= acc_t && m_tile < acc_t + my_tiles[i]) {
                const int e = threadIdx.x * 4 + i;
                tile_info[0] = e;
                tile_info[1] = offsets[e] + (m_tile - acc_t) * BM;
                tile_info[2] = offsets[e + 1];
            }
            acc_t += my_tiles[i];
        }
    }
    __syncthreads();
    const int expert = tile_info[0];
    if (expert < 0) return;                     // beyond the live tiles: nothing to do
    const int row0 = tile_info[1], row_end = tile_info[2];

    const int nkb = (int)(K / 128);
    const int64_t n0 = (int64_t)n_tile * kGBN;
    const int q16 = (lane / 16) * 16;
    // weight fragment pointers: wave owns columns n0 + 32*wave + [0, 32), two 16-column sub-tiles
    const uint8_t* wp0 = w_q + (int64_t)expert * w_stride_e + (n0 + wave * 32 + (lane & 15)) * w_stride_n + q16;
    const uint8_t* wp1 = wp0 + 16 * w_stride_n;
    const float* wsrow = w_s + (int64_t)expert * w_s_stride_e + (n0 / 128) * w_s_stride_n;

    // A staging: chunk c of the BM x 128 K-step -> row c/8, byte 16*(c%8); stored in fragment order
    int64_t a_src[A_PER_THREAD];
    int a_dst[A_PER_THREAD];
#pragma unroll
    for (int j = 0; j < A_PER_THREAD; j++) {
        const int c = threadIdx.x + j * kGThreads;
        const int rr = c / 8, ch = c % 8;
        int row = row0 + rr;
        if (row >= row_end) row = row_end - 1;     // padding rows: any valid row, outputs dropped
        a_src[j] = (int64_t)row * a_stride + ch * 16;
        // fragment order: sub-tile rr/16, lane (rr%16) + 16*(ch%4), half ch/4
        a_dst[j] = (rr / 16) * 2048 + ((rr % 16) + 16 * (ch % 4)) * 32 + (ch / 4) * 16;
    }
    int sa_row = row0 + (int)threadIdx.x;
    if (sa_row >= row_end) sa_row = row_end - 1;

    uint4 a_reg[A_PER_THREAD];
    float sa_reg = 0.0f;
    auto load_a = [&](int kb) {
#pragma unroll
        for (int j = 0; j < A_PER_THREAD; j++)
            if (threadIdx.x + j * kGThreads < A_CHUNKS)
                a_reg[j] = *reinterpret_cast<const uint4*>(a_q + a_src[j] + (int64_t)kb * 128);
        if (threadIdx.x < BM) sa_reg = a_s[(int64_t)sa_row * a_s_stride + kb];
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int j = 0; j < A_PER_THREAD; j++)
            if (threadIdx.x + j * kGThreads < A_CHUNKS)
                *reinterpret_cast<uint4*>(&a_lds[buf][a_dst[j]]) = a_reg[j];
        if (threadIdx.x < BM) sa_lds[buf][threadIdx.x] = sa_reg;
    };
    uint4 w_cur[4], w_nxt[4];
    auto load_w = [&](int kb, uint4* w) {
        const int64_t o = (int64_t)kb * 128;
        w[0] = *reinterpret_cast<const uint4*>(wp0 + o);
        w[1] = *reinterpret_cast<const uint4*>(wp0 + o + 64);
        w[2] = *reinterpret_cast<const uint4*>(wp1 + o);
        w[3] = *reinterpret_cast<const uint4*>(wp1 + o + 64);
    };

    v4f acc[MS][2];
#pragma unroll
    for (int m = 0; m < MS; m++) acc[m][0] = acc[m][1] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    load_w(0, w_cur);
    load_a(0);
    store_a(0);
    __syncthreads();
    for (int kb = 0; kb < nkb; kb++) {
        const int buf = kb & 1;
        const bool more = kb + 1 < nkb;
        if (more) {
            load_w(kb + 1, w_nxt);
            load_a(kb + 1);
        }
        const float sw = wsrow[kb];
        const v8i b0 = {(int)w_cur[0].x, (int)w_cur[0].y, (int)w_cur[0].z, (int)w_cur[0].w,
                        (int)w_cur[1].x, (int)w_cur[1].y, (int)w_cur[1].z, (int)w_cur[1].w};
        const v8i b1 = {(int)w_cur[2].x, (int)w_cur[2].y, (int)w_cur[2].z, (int)w_cur[2].w,
                        (int)w_cur[3].x, (int)w_cur[3].y, (int)w_cur[3].z, (int)w_cur[3].w};
#pragma unroll
        for (int m = 0; m < MS; m++) {
            const v8i a = *reinterpret_cast<const v8i*>(&a_lds[buf][m * 2048 + lane * 32]);
            const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
            const v4f p0 = mfma16x16x128_e4m3(a, b0, zero);
            const v4f p1 = mfma16x16x128_e4m3(a, b1, zero);
            const int rb = m * 16 + 4 * (lane / 16);
            v4f sc;
            sc[0] = sa_lds[buf][rb + 0] * sw;
            sc[1] = sa_lds[buf][rb + 1] * sw;
            sc[2] = sa_lds[buf][rb + 2] * sw;
            sc[3] = sa_lds[buf][rb + 3] * sw;
            acc[m][0] += p0 * sc;
            acc[m][1] += p1 * sc;
        }
        if (more) {
            store_a(buf ^ 1);
#pragma unroll
            for (int i = 0; i < 4; i++) w_cur[i] = w_nxt[i];
        }
        __syncthreads();
    }
    // ---- epilogue: lane holds rows m*16 + 4*(lane/16) + i, column lane%16 of each sub-tile ----
#pragma unroll
    for (int m = 0; m < MS; m++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int row = row0 + m * 16 + 4 * (lane / 16) + i;
            if (row < row_end) {
                const int64_t o = (int64_t)row * out_stride + n0 + wave * 32 + (lane & 15);
                store_from_f32<OUT_DT>(out, o, acc[m][0][i]);
                store_from_f32<OUT_DT>(out, o + 16, acc[m][1][i]);
            }
        }
    }
}

template <int BM>
static void launch_grouped_bm(hipStream_t st, int out_dt, dim3 grid, const uint8_t* a_q, int64_t a_stride,
                              const float* a_s, int64_t a_s_stride, const uint8_t* w_q, int64_t w_stride_e,
                              int64_t w_stride_n, const float* w_s, int64_t w_s_stride_e, int64_t w_s_stride_n,
                              int E, int64_t K, const int32_t* offsets, int n_tiles_n, int per_xcd, void* out,
                              int64_t out_stride) {
#define MOE_GG_ARGS a_q, a_stride, a_s, a_s_stride, w_q, w_stride_e, w_stride_n, w_s, w_s_stride_e, w_s_stride_n, \
                    E, K, offsets, n_tiles_n, per_xcd, out, out_stride
    if (out_dt == MOE_F32)
        hipLaunchKernelGGL((grouped_gemm_kernel<BM, kF32>), grid, dim3(kGThreads), 0, st, MOE_GG_ARGS);
    else if (out_dt == MOE_BF16)
        hipLaunchKernelGGL((grouped_gemm_kernel<BM, kBF16>), grid, dim3(kGThreads), 0, st, MOE_GG_ARGS);
    else
        hipLaunchKernelGGL((grouped_gemm_kernel<BM, kF16>), grid, dim3(kGThreads), 0, st, MOE_GG_ARGS);
#undef MOE_GG_ARGS
}

int grouped_gemm_launch(hipStream_t st, int block_m, const uint8_t* a_q, int64_t a_stride, const float* a_s,
                        int64_t a_s_stride, const uint8_t* w_q, int64_t w_stride_e, int64_t w_stride_n,
                        const float* w_s, int64_t w_s_stride_e, int64_t w_s_stride_n, int64_t E, int64_t N,
                        int64_t K, const int32_t* offsets, int64_t m_rows, void* out, int out_dt,
                        int64_t out_stride) {
    if (E > kMaxExpertsScan || N % kGBN != 0) return MOE_ERR_SHAPE;
    const int64_t n_tiles_n = N / kGBN;
    const int64_t m_tiles = ceil_div(m_rows, block_m) + E;   // upper bound over any split of the rows
    int64_t total = n_tiles_n * m_tiles;
    total = ceil_div(total, kXcds) * kXcds;
    if (total > 0x7FFFFFFF) return MOE_ERR_SHAPE;
    const int per_xcd = (int)(total / kXcds);
    dim3 grid((unsigned)total);
    switch (block_m) {
        case 16: launch_grouped_bm<16>(st, out_dt, grid, a_q, a_stride, a_s, a_s_stride, w_q, w_stride_e, w_stride_n, w_s, w_s_stride_e, w_s_stride_n, (int)E, K, offsets, (int)n_tiles_n, per_xcd, out, out_stride); break;
        case 32: launch_grouped_bm<32>(st, out_dt, grid, a_q, a_stride, a_s, a_s_stride, w_q, w_stride_e, w_stride_n, w_s, w_s_stride_e, w_s_stride_n, (int)E, K, offsets, (int)n_tiles_n, per_xcd, out, out_stride); break;
        case 64: launch_grouped_bm<64>(st, out_dt, grid, a_q, a_stride, a_s, a_s_stride, w_q, w_stride_e, w_stride_n, w_s, w_s_stride_e, w_s_stride_n, (int)E, K, offsets, (int)n_tiles_n, per_xcd, out, out_stride); break;
        case 128: launch_grouped_bm<128>(st, out_dt, grid, a_q, a_stride, a_s, a_s_stride, w_q, w_stride_e, w_stride_n, w_s, w_s_stride_e, w_s_stride_n, (int)E, K, offsets, (int)n_tiles_n, per_xcd, out, out_stride); break;
        default: return MOE_ERR_SHAPE;
    }
    return launch_status();
}

}  // namespace moe
