// Block-FP8 grouped GEMM for prefill: rows sorted by expert, each expert's rows
// times that expert's weights ("perf(dsfp4): pick the grouped-prefill tile
// from route density on sm_89": the M tile follows rows per expert and
// BLOCK_K is 128, one block-scale pair per K step).
//
// MI355X design.
//  * Tile BM x 256 x 128 with 8 waves of 32 columns (BM <= 64) or 16 waves of
//    16 columns (BM = 128); each wave owns its columns for all BM rows, so a
//    wave's columns sit inside one 128x128 weight-scale block and the weight
//    scale is one scalar per K step.  A last tile may hold only 128 columns
//    (N % 256 == 128); its upper half of the waves then idles.
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
//    acc += p * (a_s[row][kb] * w_s[kb]) in fp32.  All scales of the tile are
//    staged in LDS before the loop, and the loop issues no load behind a
//    branch: vector loads retire in order, so a late small load or a load the
//    compiler cannot count would make a step wait for every load in flight.
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
constexpr int kGgMaxKb = 64;                     // K/128 blocks whose scales a tile keeps in LDS (K <= 8192)

// Tile configuration per M tile, always 256 columns (which halves how often the A
// tile is re-read compared with a 128-column tile).  Up to 64 rows: 8 waves of
// two 16-column MFMA tiles each, with a weight ring that shrinks as the M tile
// grows.  128 rows (an expert's whole row range at high route density, so each
// weight byte enters the CUs once): 16 waves of one 16-column tile each, which
// keeps the accumulators and a 4-step weight ring under 128 registers.
template <int BM> struct GgCfg {
    static constexpr int WAVES = BM >= 128 ? 16 : 8;
    static constexpr int TPW = BM >= 128 ? 1 : 2;                   // 16-column MFMA tiles per wave
    static constexpr int BN = 16 * TPW * WAVES;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int S = BM >= 128 ? 4 : (BM >= 64 ? 3 : 4);   // weight ring depth (K steps)
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
__global__ void __launch_bounds__(GgCfg<BM>::THREADS, BM >= 128 ? 1 : 2)
grouped_gemm_kernel(const uint8_t* __restrict__ a_q, int64_t a_stride, const float* __restrict__ a_s,
                    int64_t a_s_stride, const uint8_t* __restrict__ w_q, int64_t w_stride_e, int64_t w_stride_n,
                    const float* __restrict__ w_s, int64_t w_s_stride_e, int64_t w_s_stride_n, int n_experts,
                    int64_t N, int64_t K, const int32_t* __restrict__ offsets, int n_tiles_n, int grid_per_xcd,
                    void* __restrict__ out, int64_t out_stride) {
    using C = GgCfg<BM>;
    constexpr int TPW = C::TPW;
    constexpr int CPW = 16 * TPW;               // columns per wave
    constexpr int MS = BM / 16;                 // 16-row MFMA sub-tiles
    constexpr int S = C::S;                     // W ring depth
    constexpr int NT = C::THREADS;
    constexpr int A_CHUNKS = BM * 8;            // 16-byte chunks of one A K-step
    constexpr int A_PER_THREAD = (A_CHUNKS + NT - 1) / NT;
    constexpr int E_PER_THREAD = kMaxExpertsScan / NT;
    __shared__ __attribute__((aligned(32))) uint8_t a_lds[2][BM * 128];
    __shared__ __attribute__((aligned(16))) float sa_lds[kGgMaxKb][BM];   // A scales of the tile, [kb][row]
    __shared__ float ws_lds[2][kGgMaxKb];                                  // weight scales, [block][kb]
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
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const bool cols = n0 + wv * CPW < N;        // a last 256-column tile may hold only 128 columns
    const int q16 = (lane / 16) * 16;
    // weight fragment pointers: wave owns columns n0 + CPW*wave + [0, CPW), TPW 16-column sub-tiles.
    // The idle waves of a 128-column last tile read valid columns (their results are dropped), so
    // the loop has no branch around its loads.
    const int64_t wcol = cols ? n0 + wv * CPW : n0;
    const uint8_t* wp0 = w_q + (int64_t)expert * w_stride_e + (wcol + (lane & 15)) * w_stride_n + q16;
    const uint8_t* wp1 = wp0 + 16 * w_stride_n;
    const int wsb = (int)((wcol - n0) / 128);   // this wave's 128-column scale block within the tile

    // All scales of the tile go to LDS once: A scales [kb][row], weight scales [block][kb].
    for (int i = threadIdx.x; i < nkb * BM; i += NT) {
        const int kb = i / BM, rr = i % BM;
        const int row = row0 + rr < row_end ? row0 + rr : row_end - 1;
        sa_lds[kb][rr] = a_s[(int64_t)row * a_s_stride + kb];
    }
    const int64_t nblk = (N - n0) >= 256 ? 2 : 1;
    for (int i = threadIdx.x; i < 2 * nkb; i += NT) {
        const int blk = i / nkb, kb = i % nkb;
        const int64_t b = n0 / 128 + (blk < nblk ? blk : 0);
        ws_lds[blk][kb] = w_s[(int64_t)expert * w_s_stride_e + b * w_s_stride_n + kb];
    }

    // A staging: chunk c of the BM x 128 K-step -> row c/8, byte 16*(c%8); stored in fragment order.
    // Threads beyond the tile's chunks load a valid chunk too (never stored).
    int64_t a_src[A_PER_THREAD];
    int a_dst[A_PER_THREAD];
#pragma unroll
    for (int j = 0; j < A_PER_THREAD; j++) {
        const int c0 = threadIdx.x + j * NT;
        const int c = c0 < A_CHUNKS ? c0 : c0 % A_CHUNKS;
        const int rr = c / 8, ch = c % 8;
        int row = row0 + rr;
        if (row >= row_end) row = row_end - 1;     // padding rows: any valid row, outputs dropped
        a_src[j] = (int64_t)row * a_stride + ch * 16;
        // fragment order: sub-tile rr/16, lane (rr%16) + 16*(ch%4), half ch/4
        a_dst[j] = (rr / 16) * 2048 + ((rr % 16) + 16 * (ch % 4)) * 32 + (ch / 4) * 16;
    }

    // A K steps pass through S register stages (step kb in stage kb % S) on their way to LDS, W K
    // steps through an S-slot register ring.  Every load in the loop is unconditional (indices
    // past the last step are clamped to it; those steps skip their multiply), so the compiler can
    // count loads in flight exactly: loads retire in order, and a load it cannot count would make
    // a step wait for all of them.  Each step's A is requested before its W, so copying A step
    // kb+1 into LDS never waits on W steps issued after it, and W keeps S-1 steps of lead.
    v4i a_reg[S][A_PER_THREAD];
    auto load_a = [&](int kb, int stage) {
#pragma unroll
        for (int j = 0; j < A_PER_THREAD; j++)
            a_reg[stage][j] = *reinterpret_cast<const v4i*>(a_q + a_src[j] + (int64_t)kb * 128);
    };
    auto store_a = [&](int stage, int buf) {
#pragma unroll
        for (int j = 0; j < A_PER_THREAD; j++)
            if (A_CHUNKS % NT == 0 || threadIdx.x + j * NT < A_CHUNKS)
                *reinterpret_cast<v4i*>(&a_lds[buf][a_dst[j]]) = a_reg[stage][j];
    };
    v4i w_ring[S][2 * TPW];
    auto load_w = [&](int kb, v4i* w) {
        const int64_t o = (int64_t)kb * 128;
        w[0] = *reinterpret_cast<const v4i*>(wp0 + o);
        w[1] = *reinterpret_cast<const v4i*>(wp0 + o + 64);
        if constexpr (TPW == 2) {
            w[2] = *reinterpret_cast<const v4i*>(wp1 + o);
            w[3] = *reinterpret_cast<const v4i*>(wp1 + o + 64);
        }
    };

    v4f acc[MS][TPW];
#pragma unroll
    for (int m = 0; m < MS; m++)
#pragma unroll
        for (int c = 0; c < TPW; c++) acc[m][c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    const int last = nkb - 1;
    // prologue: A steps 0 and 1, W steps 0..S-2 requested; A step 0 in LDS
    load_a(0, 0);
    load_a(1 < last ? 1 : last, 1 % S);
#pragma unroll
    for (int s = 0; s < S - 1; s++) load_w(s < last ? s : last, w_ring[s]);
    store_a(0, 0);
    __syncthreads();
    const int nsteps = (nkb + S - 1) / S * S;
    for (int kb0 = 0; kb0 < nsteps; kb0 += S) {
#pragma unroll
        for (int s = 0; s < S; s++) {
            const int kb = kb0 + s;
            // A step kb+2 into the stage step kb-1 left, W step kb+S-1 into the slot freed last step
            load_a(kb + 2 < last ? kb + 2 : last, (s + 2) % S);
            load_w(kb + S - 1 < last ? kb + S - 1 : last, w_ring[(s + S - 1) % S]);
            const int buf = kb & 1;
            if (kb < nkb) {
                const float sw = ws_lds[wsb][kb];
                v8i b[TPW];
#pragma unroll
                for (int c = 0; c < TPW; c++)
                    b[c] = __builtin_shufflevector(w_ring[s][2 * c], w_ring[s][2 * c + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int m = 0; m < MS; m++) {
                    const v8i a = *reinterpret_cast<const v8i*>(&a_lds[buf][m * 2048 + lane * 32]);
                    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
                    const v4f sa = *reinterpret_cast<const v4f*>(&sa_lds[kb][m * 16 + 4 * (lane / 16)]);
                    const v4f sc = sa * sw;
#pragma unroll
                    for (int c = 0; c < TPW; c++) acc[m][c] += mfma16x16x128_e4m3(a, b[c], zero) * sc;
                }
            }
            store_a((s + 1) % S, buf ^ 1);            // A step kb+1 (requested a step ago)
            __syncthreads();
        }
    }
    // ---- epilogue: lane holds rows m*16 + 4*(lane/16) + i, column lane%16 of each sub-tile ----
#pragma unroll
    for (int m = 0; m < MS; m++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int row = row0 + m * 16 + 4 * (lane / 16) + i;
            if (cols && row < row_end) {
                const int64_t o = (int64_t)row * out_stride + n0 + wave * CPW + (lane & 15);
#pragma unroll
                for (int c = 0; c < TPW; c++) store_from_f32<OUT_DT>(out, o + 16 * c, acc[m][c][i]);
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
    if (E > kMaxExpertsScan || K / 128 > kGgMaxKb) return MOE_ERR_SHAPE;
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
