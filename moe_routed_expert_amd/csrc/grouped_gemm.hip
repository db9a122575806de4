// Block-FP8 grouped GEMM for prefill: rows sorted by expert, each expert's rows
// times that expert's weights ("perf(dsfp4): pick the grouped-prefill tile
// from route density on sm_89": the M tile follows rows per expert and
// BLOCK_K is 128, one block-scale pair per K step).
//
// MI355X design.
//  * Tile BM x 256 x 128 with 8 waves; each wave owns 32 output columns for
//    all BM rows, so a wave's columns sit inside one 128x128 weight-scale block
//    and the weight scale is one scalar per K step.  A last tile may hold only
//    128 columns (N % 256 == 128); its upper four waves then idle.
//  * Weights are the dominant HBM stream and each weight byte of a tile is used
//    by one wave only, so they go global -> registers directly in MFMA operand
//    order (no LDS round trip), through a ring of S K steps (S-1 in flight while
//    one is multiplied), sized so each CU keeps enough bytes in flight to
//    cover HBM latency.
//  * The A tile (BM rows x 128 bytes per K step) is shared by the 8 waves: it
//    is staged through a double-buffered LDS tile stored in fragment order
//    (each lane's 32 bytes contiguous), so the MFMA operand reads are
//    conflict-free.  Registers are kept low enough for two resident
//    workgroups per CU at BM <= 64, which hides more latency than deeper
//    per-wave prefetch (measured).
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

constexpr int kXcds = 8;
constexpr int kMaxExpertsScan = 1024;            // experts handled by the in-kernel scan

// Tile configuration per M tile: 8 waves and a 256-column tile (each wave 32
// columns), which halves how often the A tile is re-read compared with a
// 128-column tile; the weight ring depth shrinks as the M tile grows.
template <int BM> struct GgCfg {
    static constexpr int WAVES = 8;
    static constexpr int BN = 32 * WAVES;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int S = BM >= 128 ? 2 : (BM >= 64 ? 3 : 4);   // weight ring depth (K steps)
};

// Exclusive scan of one int per thread over a block of WAVES waves.
template <int WAVES>
__device__ __forceinline__ int block_exclusive_scan(int v, int* ldsw) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    int x = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int y = __shfl_up(x, d, kWave);
        if (lane >= d) x += y;
    }
    if (lane == kWave - 1) ldsw[wave] = x;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; w++) base += ldsw[w];
    return base + x - v;
}

template <int BM, int OUT_DT>
__global__ void __launch_bounds__(GgCfg<BM>::THREADS)
grouped_gemm_kernel(const uint8_t* __restrict__ a_q, int64_t a_stride, const float* __restrict__ a_s,
                    int64_t a_s_stride, const uint8_t* __restrict__ w_q, int64_t w_stride_e, int64_t w_stride_n,
                    const float* __restrict__ w_s, int64_t w_s_stride_e, int64_t w_s_stride_n, int n_experts,
                    int64_t N, int64_t K, const int32_t* __restrict__ offsets, int n_tiles_n, int grid_per_xcd,
                    void* __restrict__ out, int64_t out_stride) {
    using C = GgCfg<BM>;
    constexpr int MS = BM / 16;                 // 16-row MFMA sub-tiles
    constexpr int S = C::S;                     // W ring depth
    constexpr int NT = C::THREADS;
    constexpr int A_CHUNKS = BM * 8;            // 16-byte chunks of one A K-step
    constexpr int A_PER_THREAD = (A_CHUNKS + NT - 1) / NT;
    constexpr int E_PER_THREAD = kMaxExpertsScan / NT;
    __shared__ __attribute__((aligned(32))) uint8_t a_lds[2][BM * 128];
    __shared__ float sa_lds[2][BM];
    __shared__ int scan_lds[C::WAVES];
    __shared__ int tile_info[3];                // expert, row begin, row end

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    // XCD-aware remap of the linear workgroup id
    const int bid = blockIdx.x;
    const int logical = (bid % kXcds) * grid_per_xcd + bid / kXcds;
    const int m_tile = logical / n_tiles_n, n_tile = logical % n_tiles_n;

    // ---- find (expert, m0) for this M tile from the device offsets ----
    int local = 0, my_tiles[E_PER_THREAD];
#pragma unroll
    for (int i = 0; i < E_PER_THREAD; i++) {
        const int e = threadIdx.x * E_PER_THREAD + i;
        int t = 0;
        if (e < n_experts) t = (offsets[e + 1] - offsets[e] + BM - 1) / BM;
        my_tiles[i] = t;
        local += t;
    }
    int before = block_exclusive_scan<C::WAVES>(local, scan_lds);
    if (threadIdx.x == 0) tile_info[0] = -1;
    __syncthreads();
    if (m_tile >= before && m_tile < before + local) {
        int acc_t = before;
#pragma unroll
        for (int i = 0; i < E_PER_THREAD; i++) {
            if (m_tile >= acc_t && m_tile < acc_t + my_tiles[i]) {
                const int e = threadIdx.x * E_PER_THREAD + i;
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
    const int64_t n0 = (int64_t)n_tile * C::BN;
    const bool cols = n0 + wave * 32 < N;      // a last 256-column tile may hold only 128 columns
    const int q16 = (lane / 16) * 16;
    // weight fragment pointers: wave owns columns n0 + 32*wave + [0, 32), two 16-column sub-tiles
    const uint8_t* wp0 = w_q + (int64_t)expert * w_stride_e + (n0 + wave * 32 + (lane & 15)) * w_stride_n + q16;
    const uint8_t* wp1 = wp0 + 16 * w_stride_n;
    const float* wsrow = w_s + (int64_t)expert * w_s_stride_e + ((n0 + wave * 32) / 128) * w_s_stride_n;

    // A staging: chunk c of the BM x 128 K-step -> row c/8, byte 16*(c%8); stored in fragment order
    int64_t a_src[A_PER_THREAD];
    int a_dst[A_PER_THREAD];
#pragma unroll
    for (int j = 0; j < A_PER_THREAD; j++) {
        const int c = threadIdx.x + j * NT;
        const int rr = c / 8, ch = c % 8;
        int row = row0 + rr;
        if (row >= row_end) row = row_end - 1;     // padding rows: any valid row, outputs dropped
        a_src[j] = (int64_t)row * a_stride + ch * 16;
        // fragment order: sub-tile rr/16, lane (rr%16) + 16*(ch%4), half ch/4
        a_dst[j] = (rr / 16) * 2048 + ((rr % 16) + 16 * (ch % 4)) * 32 + (ch / 4) * 16;
    }
    int sa_row = row0 + (int)threadIdx.x;
    if (sa_row >= row_end) sa_row = row_end - 1;

    v4i a_reg[A_PER_THREAD];
    float sa_reg = 0.0f;
    auto load_a = [&](int kb) {
#pragma unroll
        for (int j = 0; j < A_PER_THREAD; j++)
            if (threadIdx.x + j * NT < A_CHUNKS)
                a_reg[j] = *reinterpret_cast<const v4i*>(a_q + a_src[j] + (int64_t)kb * 128);
        if (threadIdx.x < BM) sa_reg = a_s[(int64_t)sa_row * a_s_stride + kb];
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int j = 0; j < A_PER_THREAD; j++)
            if (threadIdx.x + j * NT < A_CHUNKS)
                *reinterpret_cast<v4i*>(&a_lds[buf][a_dst[j]]) = a_reg[j];
        if (threadIdx.x < BM) sa_lds[buf][threadIdx.x] = sa_reg;
    };
    // W ring: slot s holds K step kb with kb % S == s, 4 x 16 bytes per lane
    v4i w_ring[S][4];
    auto load_w = [&](int kb, v4i* w) {
        if (!cols) return;
        const int64_t o = (int64_t)kb * 128;
        w[0] = *reinterpret_cast<const v4i*>(wp0 + o);
        w[1] = *reinterpret_cast<const v4i*>(wp0 + o + 64);
        w[2] = *reinterpret_cast<const v4i*>(wp1 + o);
        w[3] = *reinterpret_cast<const v4i*>(wp1 + o + 64);
    };

    v4f acc[MS][2];
#pragma unroll
    for (int m = 0; m < MS; m++) acc[m][0] = acc[m][1] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // prologue: A step 0 into LDS, A step 1 in registers, W steps 0..S-2 in flight
    load_a(0);
#pragma unroll
    for (int s = 0; s < S - 1; s++)
        if (s < nkb) load_w(s, w_ring[s]);
    store_a(0);
    if (nkb > 1) load_a(1);
    __syncthreads();
    for (int kb0 = 0; kb0 < nkb; kb0 += S) {
#pragma unroll
        for (int s = 0; s < S; s++) {
            const int kb = kb0 + s;
            if (kb < nkb) {
                // keep S-1 weight steps in flight: issue step kb+S-1 into the slot freed last step
                if (kb + S - 1 < nkb) load_w(kb + S - 1, w_ring[(s + S - 1) % S]);
                const int buf = kb & 1;
                if (cols) {
                const float sw = wsrow[kb];
                const v8i b0 = __builtin_shufflevector(w_ring[s][0], w_ring[s][1], 0, 1, 2, 3, 4, 5, 6, 7);
                const v8i b1 = __builtin_shufflevector(w_ring[s][2], w_ring[s][3], 0, 1, 2, 3, 4, 5, 6, 7);
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
                }
                if (kb + 1 < nkb) {
                    store_a(buf ^ 1);                 // A step kb+1 (loaded one step ago)
                    if (kb + 2 < nkb) load_a(kb + 2);
                }
                __syncthreads();
            }
        }
    }
    // ---- epilogue: lane holds rows m*16 + 4*(lane/16) + i, column lane%16 of each sub-tile ----
#pragma unroll
    for (int m = 0; m < MS; m++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int row = row0 + m * 16 + 4 * (lane / 16) + i;
            if (cols && row < row_end) {
                const int64_t o = (int64_t)row * out_stride + n0 + wave * 32 + (lane & 15);
                store_from_f32<OUT_DT>(out, o, acc[m][0][i]);
                store_from_f32<OUT_DT>(out, o + 16, acc[m][1][i]);
            }
        }
    }
}

template <int BM>
static int launch_grouped_bm(hipStream_t st, int out_dt, const uint8_t* a_q, int64_t a_stride, const float* a_s,
                             int64_t a_s_stride, const uint8_t* w_q, int64_t w_stride_e, int64_t w_stride_n,
                             const float* w_s, int64_t w_s_stride_e, int64_t w_s_stride_n, int64_t E, int64_t N,
                             int64_t K, const int32_t* offsets, int64_t m_rows, void* out, int64_t out_stride) {
    using C = GgCfg<BM>;
    if (N % 128 != 0) return MOE_ERR_SHAPE;
    const int64_t n_tiles_n = ceil_div(N, C::BN);
    const int64_t m_tiles = ceil_div(m_rows, BM) + E;   // upper bound over any split of the rows
    int64_t total = ceil_div(n_tiles_n * m_tiles, kXcds) * kXcds;
    if (total > 0x7FFFFFFF) return MOE_ERR_SHAPE;
    const int per_xcd = (int)(total / kXcds);
    dim3 grid((unsigned)total), block(C::THREADS);
#define MOE_GG_ARGS a_q, a_stride, a_s, a_s_stride, w_q, w_stride_e, w_stride_n, w_s, w_s_stride_e, w_s_stride_n, \
                    (int)E, N, K, offsets, (int)n_tiles_n, per_xcd, out, out_stride
    if (out_dt == MOE_F32)
        hipLaunchKernelGGL((grouped_gemm_kernel<BM, kF32>), grid, block, 0, st, MOE_GG_ARGS);
    else if (out_dt == MOE_BF16)
        hipLaunchKernelGGL((grouped_gemm_kernel<BM, kBF16>), grid, block, 0, st, MOE_GG_ARGS);
    else
        hipLaunchKernelGGL((grouped_gemm_kernel<BM, kF16>), grid, block, 0, st, MOE_GG_ARGS);
#undef MOE_GG_ARGS
    return launch_status();
}

int grouped_gemm_launch(hipStream_t st, int block_m, const uint8_t* a_q, int64_t a_stride, const float* a_s,
                        int64_t a_s_stride, const uint8_t* w_q, int64_t w_stride_e, int64_t w_stride_n,
                        const float* w_s, int64_t w_s_stride_e, int64_t w_s_stride_n, int64_t E, int64_t N,
                        int64_t K, const int32_t* offsets, int64_t m_rows, void* out, int out_dt,
                        int64_t out_stride) {
    if (E > kMaxExpertsScan) return MOE_ERR_SHAPE;
#define MOE_GG_CALL(bm) launch_grouped_bm<bm>(st, out_dt, a_q, a_stride, a_s, a_s_stride, w_q, w_stride_e, w_stride_n, \
                                             w_s, w_s_stride_e, w_s_stride_n, E, N, K, offsets, m_rows, out, out_stride)
    switch (block_m) {
        case 16: return MOE_GG_CALL(16);
        case 32: return MOE_GG_CALL(32);
        case 64: return MOE_GG_CALL(64);
        case 128: return MOE_GG_CALL(128);
        default: return MOE_ERR_SHAPE;
    }
#undef MOE_GG_CALL
}

}  // namespace moe
