// Block-FP8 grouped GEMM for prefill: rows sorted by expert, each expert's rows
// times that expert's weights ("perf(dsfp4): pick the grouped-prefill tile
// from route density on sm_89": the M tile follows rows per expert and
// BLOCK_K is 128, one block-scale pair per K step).
//
// MI355X design.
//  * Tile BM x 256 x 128 with 8 waves of 32 columns; each wave owns its
//    columns for all BM rows, so a wave's columns sit inside one 128x128
//    weight-scale block and the weight scale is one scalar per K step.  A last tile may hold only 128 columns
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
//    per-wave prefetch (measured); BM = 128 runs one workgroup per CU.
//  * Per K step: p = W*A^T with a fresh 16x16x128 e4m3 MFMA (weights as the
//    row operand, so a lane's four results are four columns of one A row),
//    then acc += p * (a_s[row][kb] * w_s[kb]) in fp32 with one scale per lane;
//    the epilogue stores the four columns as one vector, or, for a 2-byte
//    output, eight columns after two lane swaps (store_tile_out).  All scales of the tile are
//    staged in LDS before the loop, and the loop issues no load behind a
//    branch: vector loads retire in order, so a late small load or a load the
//    compiler cannot count would make a step wait for every load in flight.
//  * Work map: M tiles are (expert, 0..ceil(rows_e/BM)-1) and a tile is (M
//    tile, 256-column N tile).  The kernel is persistent: the grid is the
//    number of workgroups the device holds at once (fixed by scalars, so the
//    launch can be captured); each workgroup scans the device offsets once into
//    an LDS table of every expert's first M tile, then walks its share of the
//    live tiles.  The live tiles are cut into 8 equal contiguous ranges, one per
//    XCD (the dispatcher deals workgroups to the 8 XCDs round-robin), and an
//    XCD's workgroups take its range in order, so the tiles in flight on an XCD
//    are neighbouring N tiles of neighbouring M tiles: their A rows and weight
//    tiles meet in that XCD's L2, and every XCD gets the same number of tiles.
//  * MXFP4 weights (the FP4 variant): a lane's 32 K elements of a step are one
//    MX block, 16 contiguous bytes, and the block's E8M0 scale is applied inside
//    v_mfma_scale_f32_16x16x128_f8f6f4, so the weight stream is half the bytes
//    and there is no per-block fp32 weight scale.  The scale bytes do not ride
//    in the ring: a 4-byte load per row and step touches 16 rows for 64 bytes,
//    and those loads cost as much as the weights.  Each wave instead copies its
//    32 rows' scales for 32 steps into LDS with row-contiguous loads (one per
//    lane per row pair) and reads a step's dword from there.
//  * A tile's expert is a binary search of the LDS table; its scales are
//    loaded row-contiguous, all requests in flight before the LDS stores.
//  * Fused activation requant (the gate/up GEMM of a prefill step with the
//    gated activation in its epilogue): a tile covers one 128-column act group;
//    each wave's two 16-column sub-tiles are gate rows and the matching up rows
//    of W13, so a lane holds gate and up of the same four columns of one row and
//    forms h = act(gate)*up from the fp32 accumulators.  The group amax is a
//    lane shuffle plus an 8-wave LDS max, then s = amax/448 and the codes
//    e4m3(h/s) (moe_act_quant's quotients) leave as one 4-byte store per lane;
//    the [rows][2I] GEMM output is never written.
#include <atomic>

#include "device.h"
#include "host.h"

namespace moe {

constexpr int kXcds = 8;
constexpr int kMaxExpertsScan = 1024;            // experts handled by the in-kernel scan
constexpr int kGgMaxKb = 64;                     // K/128 blocks whose scales a tile keeps in LDS (K <= 8192)
constexpr int kScRow = 132;                      // MXFP4: LDS bytes per weight row of a 128-block scale chunk

// Tile configuration per M tile: always 8 waves of two 16-column MFMA tiles, 256 columns (which
// halves how often the A tile is re-read compared with a 128-column tile).  Up to 64 rows the
// registers stay under 128, so two workgroups share a CU (4 waves per SIMD) and hide each other's
// latency; the weight ring shrinks as the M tile grows.  128 rows (an expert's whole row range at
// high route density, so each weight byte enters the CU once) need about 200 registers: one
// workgroup per CU (2 waves per SIMD) with a deeper weight ring instead.
template <int BM> struct GgCfg {
    static constexpr int WAVES = 8;
    static constexpr int TPW = 2;                                   // 16-column MFMA tiles per wave
    static constexpr int BN = 16 * TPW * WAVES;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int S = BM >= 128 ? 4 : (BM >= 64 ? 3 : 4);   // weight ring depth (K steps)
    static constexpr int WAVES_PER_EU = BM >= 128 ? 2 : 4;          // occupancy the registers are sized for
};

// Arguments of one grouped GEMM launch (pointers and strides as in moe_bf8_grouped_gemm).  The fused
// SiLU-mul requant variant (N = 2I) writes codes q and scales s instead of out.
struct GgArgs {
    const uint8_t* a_q;
    int64_t a_stride;
    const float* a_s;
    int64_t a_s_stride;
    const uint8_t* w_q;
    int64_t w_stride_e, w_stride_n;
    const float* w_s;
    int64_t w_s_stride_e, w_s_stride_n;
    int n_experts;
    int64_t N, K;
    const int32_t* offsets;
    int m_rows;
    int n_tiles_n, per_xcd, step_m, step_n;   // tile walk (see the kernel)
    void* out;
    int64_t out_stride;
    uint8_t* q;                               // fused: codes [rows][q_stride], I used
    int64_t q_stride;
    float* s;                                 // fused: scales [rows][s_stride], I/128 used
    int64_t s_stride;
    int act;                                  // fused: gated activation (moe_act 1..5)
    // MXFP4 weights (W4 variant): w_q holds [e][n][K/2] bytes (strides in bytes), w4s [e][n][K/32] E8M0
    const uint8_t* w4s;
    int64_t w4s_stride_e, w4s_stride_n;
    // weight addressing (set by set_weight_layout): row-major [e][n][k] with row stride w_stride_n, or
    // packed (moe_pack_weights: per expert, per 16-row group, per K step, one block in operand order)
    bool w_packed;
    int64_t w_group;                          // bytes from one 16-row group to the next
    int64_t w_kstep;                          // bytes from one K step to the next within a group
    int64_t w_khalf;                          // block-FP8: bytes from a lane's first 16-byte piece to its second
};

// Fills the weight addressing of g for w_stride_n (MOE_W_PACKED: the packed order) and row_bytes = K
// (block-FP8) or K/2 (MXFP4).  A K step is 128 bytes of a row (block-FP8) or 64 (MXFP4).
inline void set_weight_layout(GgArgs& g, bool w4) {
    const int64_t row_bytes = w4 ? g.K / 2 : g.K, step = w4 ? 64 : 128;
    g.w_packed = g.w_stride_n == MOE_W_PACKED;
    g.w_group = g.w_packed ? 16 * row_bytes : 16 * g.w_stride_n;
    g.w_kstep = g.w_packed ? 16 * step : step;
    g.w_khalf = g.w_packed ? 1024 : 64;
}

// LDS byte offset, within a 16-row A sub-tile (2 KiB), of piece h of MFMA lane `lane`: h = 0 holds the
// row's K bytes 16q .. 16q+15 and h = 1 bytes 64+16q .. +15 (q = lane/16), the order the weight pieces
// take.  The 128 pieces are 16-byte slots 64h + lane with the low three bits XORed by 4h + q, so the 8
// lanes an LDS cycle serves read 8 different slots of a 128-byte span, and so do the 8 chunks of one A
// row (chunk 4h + q) that 8 consecutive threads write (without the XOR, reads were 2-way and writes
// 8-way conflicts).
__device__ __forceinline__ int a_piece_offset(int lane, int h) {
    return 16 * ((64 * h + lane) ^ (4 * h + ((lane >> 4) & 3)));
}

// Byte offset, from w_q, of this lane's first weight piece of the 16-row group that starts at row r16
// (a multiple of 16) of expert e.  Row-major: row r16 + lane%16, bytes 16*(lane/16) of each K step (and
// 64 more for the second piece).  Packed: the pieces of a step are stored in lane order.
__device__ __forceinline__ int64_t w_lane_offset(const GgArgs& g, int expert, int64_t r16, int lane) {
    return (int64_t)expert * g.w_stride_e + (r16 / 16) * g.w_group +
           (g.w_packed ? 16 * (int64_t)lane : (lane & 15) * g.w_stride_n + (lane / 16) * 16);
}

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

// Fused epilogue: acc[m][0] holds gate and acc[m][1] up for row m*16 + lane%16, act columns
// 128*n_tile + 16*wave + 4*(lane/16) + i.  h = act(gate)*up in fp32; per row, the amax of the 128
// columns (4 lanes by shuffle, then the 8 waves through LDS), s = amax/448 (correctly rounded), codes
// e4m3(h/s) (zero codes when s == 0) with moe_act_quant's e4m3_codes, so the codes are
// the same bits.  ACT is fixed per instantiation: no per-element switch.
template <int BM, int ACT>
__device__ __forceinline__ void act_quant_epilogue_t(const GgArgs& g, v4f (&acc)[BM / 16][2], int row0, int row_end,
                                                     int n_tile, int lane, int wave, float (*amax_lds)[BM]) {
    using C = GgCfg<BM>;
    constexpr int MS = BM / 16;
#pragma unroll
    for (int m = 0; m < MS; m++) {
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float gt = acc[m][0][i], up = acc[m][1][i];
            acc[m][0][i] = gated_act_t<ACT>(gt, up);             // h replaces gate
            a = __builtin_fmaxf(a, __builtin_fabsf(acc[m][0][i]));
        }
        a = __builtin_fmaxf(a, __shfl_xor(a, 16, kWave));
        a = __builtin_fmaxf(a, __shfl_xor(a, 32, kWave));
        if (lane < 16) amax_lds[wave][m * 16 + lane] = a;
    }
    __syncthreads();
    const bool vec = (g.q_stride % 4 == 0) && (reinterpret_cast<uintptr_t>(g.q) % 4 == 0);
#pragma unroll
    for (int m = 0; m < MS; m++) {
        const int rl = m * 16 + (lane & 15);
        float amax = amax_lds[0][rl];
#pragma unroll
        for (int w = 1; w < C::WAVES; w++) amax = __builtin_fmaxf(amax, amax_lds[w][rl]);
        const float s = amax / 448.0f;
        uint32_t code[1] = {0u};
        if (s != 0.0f) {
            const float h[4] = {acc[m][0][0], acc[m][0][1], acc[m][0][2], acc[m][0][3]};
            e4m3_codes(h, s, code);
        }
        const int row = row0 + rl;
        if (row < row_end) {
            uint8_t* q = g.q + (int64_t)row * g.q_stride + (int64_t)n_tile * 128 + 16 * wave + 4 * (lane / 16);
            if (vec) {
                *reinterpret_cast<uint32_t*>(q) = code[0];
            } else {
#pragma unroll
                for (int i = 0; i < 4; i++) q[i] = (uint8_t)(code[0] >> (8 * i));
            }
            if (wave == 0 && lane < 16) g.s[(int64_t)row * g.s_stride + n_tile] = s;
        }
    }
}

// The fused epilogue with the activation chosen once per tile (wave-uniform).
template <int BM>
__device__ __forceinline__ void act_quant_epilogue(const GgArgs& g, v4f (&acc)[BM / 16][2], int row0, int row_end,
                                                   int n_tile, int lane, int wave) {
    __shared__ float amax_lds[GgCfg<BM>::WAVES][BM];     // one table for all five forms
    switch (g.act) {
        case 1: act_quant_epilogue_t<BM, 1>(g, acc, row0, row_end, n_tile, lane, wave, amax_lds); break;
        case 2: act_quant_epilogue_t<BM, 2>(g, acc, row0, row_end, n_tile, lane, wave, amax_lds); break;
        case 3: act_quant_epilogue_t<BM, 3>(g, acc, row0, row_end, n_tile, lane, wave, amax_lds); break;
        case 4: act_quant_epilogue_t<BM, 4>(g, acc, row0, row_end, n_tile, lane, wave, amax_lds); break;
        default: act_quant_epilogue_t<BM, 5>(g, acc, row0, row_end, n_tile, lane, wave, amax_lds); break;
    }
}

// Two output values of a 2-byte type packed into one word, the first in the low half.
template <int OUT_DT>
__device__ __forceinline__ uint32_t pack2_out(float x, float y) {
    if constexpr (OUT_DT == kBF16) return (uint32_t)f32_to_bf16(x) | ((uint32_t)f32_to_bf16(y) << 16);
    else return (uint32_t)f32_to_f16(x) | ((uint32_t)f32_to_f16(y) << 16);
}

// The epilogue of a plain (not fused) tile: this wave's results acc[m][c] (row m*16 + lane%16 of the tile,
// columns 16c + 4*(lane/16) + 0..3 of the wave's 32) go to out [rows][out_stride] of OUT_DT.  With a 2-byte
// output whose rows allow it, a permlane32 swap and a permlane16 swap of each word pair (gfx950 lane moves)
// leave lane 16q + r with columns 8q..8q+7 of row r, so each lane writes 16 bytes and each store covers 64
// bytes of 16 rows: with the 32-byte pieces of 8-byte stores, a 24576-route gate/up GEMM's output stores cost
// about 1.5 times as much memory time.  The swaps run in every lane (full exec), outside the row test.
// SWAP = false keeps the 8-byte stores (a tile whose registers are at their limit).
template <int OUT_DT, int MS, int TPW, bool SWAP = true>
__device__ __forceinline__ void store_tile_out(const GgArgs& g, const v4f (&acc)[MS][TPW], int row0, int row_end,
                                               int64_t col0, bool cols, int lane) {
    void* __restrict__ out = g.out;
    const int64_t out_stride = g.out_stride;
    if constexpr (SWAP && OUT_DT != kF32 && TPW == 2) {
        if (out_stride % 8 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0) {
            const int tile_rows = __builtin_amdgcn_readfirstlane(row_end - row0);
#pragma unroll
            for (int m = 0; m < MS; m++) {
                if (m * 16 >= tile_rows) break;            // sub-tiles past the tile's rows (wave-uniform)
                const auto s0 = __builtin_amdgcn_permlane32_swap(pack2_out<OUT_DT>(acc[m][0][0], acc[m][0][1]),
                                                                 pack2_out<OUT_DT>(acc[m][1][0], acc[m][1][1]), false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(pack2_out<OUT_DT>(acc[m][0][2], acc[m][0][3]),
                                                                 pack2_out<OUT_DT>(acc[m][1][2], acc[m][1][3]), false, false);
                const auto t0 = __builtin_amdgcn_permlane16_swap(s0[0], s0[1], false, false);
                const auto t1 = __builtin_amdgcn_permlane16_swap(s1[0], s1[1], false, false);
                const int row = row0 + m * 16 + (lane & 15);
                if (cols && row < row_end)
                    *reinterpret_cast<uint4*>((uint16_t*)out + (int64_t)row * out_stride + col0 + 8 * (lane / 16)) =
                        make_uint4(t0[0], t1[0], t0[1], t1[1]);
            }
            return;
        }
    }
    const bool vec4 = (out_stride % 4 == 0) && (reinterpret_cast<uintptr_t>(out) % (OUT_DT == kF32 ? 16 : 8) == 0);
#pragma unroll
    for (int m = 0; m < MS; m++) {
        const int row = row0 + m * 16 + (lane & 15);
        if (cols && row < row_end) {
            const int64_t o = (int64_t)row * out_stride + col0 + 4 * (lane / 16);
#pragma unroll
            for (int c = 0; c < TPW; c++) {
                if (vec4) {
                    store4_from_f32<OUT_DT>(out, o + 16 * c, acc[m][c]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; i++) store_from_f32<OUT_DT>(out, o + 16 * c + i, acc[m][c][i]);
                }
            }
        }
    }
}

// One tile: rows [row0, min(row0 + BM, row_end)) of expert `expert`, N tile n_tile (256 output
// columns, or act group n_tile when FUSED).  The caller's workgroup runs it with all threads; it
// leaves LDS free for the next tile (its last LDS read is before its last barrier).
template <int BM, int OUT_DT, bool FUSED, bool W4>
__device__ __forceinline__ void grouped_gemm_tile(const GgArgs& g, int expert, int row0, int row_end, int n_tile) {
    const uint8_t* __restrict__ a_q = g.a_q;
    const float* __restrict__ a_s = g.a_s;
    const uint8_t* __restrict__ w_q = g.w_q;
    const float* __restrict__ w_s = g.w_s;
    const int64_t a_stride = g.a_stride, a_s_stride = g.a_s_stride;
    const int64_t w_s_stride_e = g.w_s_stride_e, w_s_stride_n = g.w_s_stride_n;
    const int64_t N = g.N, K = g.K;
    using C = GgCfg<BM>;
    constexpr int TPW = C::TPW;
    constexpr int CPW = 16 * TPW;               // columns per wave
    constexpr int MS = BM / 16;                 // 16-row MFMA sub-tiles
    constexpr int SA = C::S;                    // A register stages
    constexpr int S = C::S;                     // W ring depth; SA divides it, so both indices stay static
    constexpr int NT = C::THREADS;
    constexpr int A_CHUNKS = BM * 8;            // 16-byte chunks of one A K-step
    constexpr int A_PER_THREAD = (A_CHUNKS + NT - 1) / NT;
    constexpr int SA_ROW = BM + 4;              // padded [kb] row of the A-scale table (16-byte aligned)
    __shared__ __attribute__((aligned(32))) uint8_t a_lds[2][BM * 128];
    __shared__ __attribute__((aligned(16))) float sa_lds[kGgMaxKb * SA_ROW];   // A scales, [kb][row]
    __shared__ float ws_lds[2][kGgMaxKb];                                       // weight scales, [block][kb]
    // MXFP4: each wave's E8M0 bytes of its 32 weight rows, 128 blocks (32 K steps) at a time; a row
    // takes kScRow bytes so the 16 rows one read touches fall in different banks
    __shared__ __attribute__((aligned(16))) uint8_t sc_lds[W4 ? C::WAVES * 32 * kScRow : 4];

    // A fresh copy of the thread index per tile: without it the compiler hoists every thread-index
    // expression of the tile out of the caller's tile loop and keeps them all live across it.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const int nkb = (int)(K / 128);
    const int64_t n0 = (int64_t)n_tile * C::BN;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const bool cols = FUSED || n0 + wv * CPW < N;   // a last 256-column tile may hold only 128 columns
    // weight fragment pointers: wave owns columns n0 + CPW*wave + [0, CPW), TPW 16-column sub-tiles.
    // The idle waves of a 128-column last tile read valid columns (their results are dropped), so
    // the loop has no branch around its loads.  Fused: sub-tile 0 is gate rows 128*n_tile + 16*wave +
    // [0, 16), sub-tile 1 the matching up rows I + ..., with scale blocks n_tile and I/128 + n_tile.
    const int64_t I = N / 2;
    const int64_t wcol = FUSED ? (int64_t)n_tile * 128 + 16 * wv : (cols ? n0 + wv * CPW : n0);
    const uint8_t* wp0 = w_q + w_lane_offset(g, expert, wcol, lane);
    const uint8_t* wp1 = wp0 + (FUSED ? I / 16 : 1) * g.w_group;
    const int64_t kstep = g.w_kstep, khalf = g.w_khalf;
    // MXFP4 scales.  A chunk is 128 blocks (32 K steps) of the wave's 32 rows: lanes 0-31 read one row's
    // 128 bytes as 32 dwords and lanes 32-63 the next row, 16 loads per lane, all requested before the
    // first LDS store.  In a step the lane's K block is 4 kb + lane/16; it reads the row's dword of the
    // step from LDS and takes its byte.
    uint8_t* const sc_wave = sc_lds + wave * 32 * kScRow;
    // (a wave-uniform row base plus one 32-bit lane offset, so the 16 addresses cost no vector registers)
    const uint8_t* const sc_base = W4 ? g.w4s + (int64_t)expert * g.w4s_stride_e + wcol * g.w4s_stride_n : nullptr;
    const int64_t sc_sub = (FUSED ? I : 16) * g.w4s_stride_n;     // sub-tile 1 rows
    uint32_t sc_v[16];
    auto sc_issue = [&](int kb0, int i0, int ni) {  // words i0 .. i0+ni-1 of the chunk from step kb0
        int l = lane;
        asm volatile("" : "+v"(l));                 // per call: keeps the lane terms out of the step loop
        const bool in = (l & 31) < nkb - kb0;     // a chunk stage may load a step beyond the chunk: unused
        const uint32_t lo = (uint32_t)((l >> 5) * g.w4s_stride_n + 4 * (l & 31));
#pragma unroll
        for (int i = i0; i < i0 + ni; i++) {        // rows 2i + lane/32 of the wave: sub-tile i/8
            const uint8_t* u = sc_base + (i / 8) * sc_sub + (2 * (i % 8)) * g.w4s_stride_n + 4 * (int64_t)kb0;
            sc_v[i] = in ? *reinterpret_cast<const uint32_t*>(u + lo) : 0u;
        }
    };
    auto sc_commit = [&](int i0, int ni) {
#pragma unroll
        for (int i = i0; i < i0 + ni; i++)
            *reinterpret_cast<uint32_t*>(sc_wave + (2 * i + (lane >> 5)) * kScRow + 4 * (lane & 31)) = sc_v[i];
    };
    const int sshift = 8 * (lane / 16);
    const int wsb = FUSED ? 0 : (int)((wcol - n0) / 128);   // this wave's 128-column scale block

    // All scales of the tile go to LDS once: A scales [kb][row] (wave w reads rows w, w + WAVES, ...,
    // lane = K block, so each request is one contiguous row of scales), weight scales [block][kb]
    // (waves 0 and 1, one 128-column block each).  Every load is requested before the first LDS
    // store, and no index needs a division by the block count.
    constexpr int SA_ROWS = BM / C::WAVES;      // A-scale rows per wave
    const int kbl = lane < nkb ? lane : nkb - 1;
    float sa_v[SA_ROWS];
#pragma unroll
    for (int j = 0; j < SA_ROWS; j++) {
        const int rr = wave + j * C::WAVES;
        const int row = row0 + rr < row_end ? row0 + rr : row_end - 1;
        sa_v[j] = a_s[(int64_t)row * a_s_stride + kbl];
    }
    const int64_t nblk = (N - n0) >= 256 ? 2 : 1;
    float ws_v = 0.0f;
    if (!W4 && wave < 2) {
        const int64_t b = FUSED ? (wave == 0 ? n_tile : I / 128 + n_tile) : n0 / 128 + (wave < nblk ? wave : 0);
        ws_v = w_s[(int64_t)expert * w_s_stride_e + b * w_s_stride_n + kbl];
    }
    if (lane < nkb) {
#pragma unroll
        for (int j = 0; j < SA_ROWS; j++) sa_lds[lane * SA_ROW + wave + j * C::WAVES] = sa_v[j];
        if (!W4 && wave < 2) ws_lds[wave][lane] = ws_v;
    }

    // A staging: chunk c of the BM x 128 K-step -> row c/8, byte 16*(c%8); stored in fragment order.
    // Threads beyond the tile's chunks load a valid chunk too (never stored).
    int64_t a_src[A_PER_THREAD];
    int a_dst[A_PER_THREAD];
    const int a_p0 = a_piece_offset(lane, 0), a_p1 = a_piece_offset(lane, 1);   // this lane's MFMA pieces
#pragma unroll
    for (int j = 0; j < A_PER_THREAD; j++) {
        const int c0 = tid + j * NT;
        const int c = c0 < A_CHUNKS ? c0 : c0 % A_CHUNKS;
        const int rr = c / 8, ch = c % 8;
        int row = row0 + rr;
        if (row >= row_end) row = row_end - 1;     // padding rows: any valid row, outputs dropped
        a_src[j] = (int64_t)row * a_stride + ch * 16;
        // fragment order: sub-tile rr/16, lane (rr%16) + 16*(ch%4), piece ch/4
        a_dst[j] = (rr / 16) * 2048 + a_piece_offset((rr % 16) + 16 * (ch % 4), ch / 4);
    }

    // A K steps pass through SA register stages (step kb in stage kb % SA) on their way to LDS, W K
    // steps through an S-slot register ring.  Every load in the loop is unconditional (indices
    // past the last step are clamped to it; those steps skip their multiply), so the compiler can
    // count loads in flight exactly: loads retire in order, and a load it cannot count would make
    // a step wait for all of them.  Each step's A is requested before its W, so copying A step
    // kb+1 into LDS never waits on W steps issued after it, and W keeps S-1 steps of lead.
    v4i a_reg[SA][A_PER_THREAD];
    auto load_a = [&](int kb, int stage) {
#pragma unroll
        for (int j = 0; j < A_PER_THREAD; j++)
            a_reg[stage][j] = *reinterpret_cast<const v4i*>(a_q + a_src[j] + (int64_t)kb * 128);
    };
    auto store_a = [&](int stage, int buf) {
#pragma unroll
        for (int j = 0; j < A_PER_THREAD; j++)
            if (A_CHUNKS % NT == 0 || tid + j * NT < A_CHUNKS)
                *reinterpret_cast<v4i*>(&a_lds[buf][a_dst[j]]) = a_reg[stage][j];
    };
    v4i w_ring[S][2 * TPW];
    auto load_w = [&](int kb, v4i* w) {
        const int64_t o = (int64_t)kb * kstep;
        if constexpr (W4) {
            w[0] = *reinterpret_cast<const v4i*>(wp0 + o);
            w[1] = *reinterpret_cast<const v4i*>(wp1 + o);
            return;
        }
        w[0] = *reinterpret_cast<const v4i*>(wp0 + o);
        w[1] = *reinterpret_cast<const v4i*>(wp0 + o + khalf);
        if constexpr (TPW == 2) {
            w[2] = *reinterpret_cast<const v4i*>(wp1 + o);
            w[3] = *reinterpret_cast<const v4i*>(wp1 + o + khalf);
        }
    };

    v4f acc[MS][TPW];
#pragma unroll
    for (int m = 0; m < MS; m++)
#pragma unroll
        for (int c = 0; c < TPW; c++) acc[m][c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    const int last = nkb - 1;
    const int tile_rows = __builtin_amdgcn_readfirstlane(row_end - row0);
    // prologue: the first scale chunk, then A and W steps 0..S-2 (each A step ahead of its W step)
    // requested; scales and A step 0 in LDS (the chunk's loads are the oldest, so its stores wait for
    // nothing else)
    if constexpr (W4) sc_issue(0, 0, 16);
#pragma unroll
    for (int s = 0; s < S - 1; s++) {
        load_a(s < last ? s : last, s % SA);
        load_w(s < last ? s : last, w_ring[s]);
    }
    if constexpr (W4) sc_commit(0, 16);
    store_a(0, 0);
    __syncthreads();
    const int nsteps = (nkb + S - 1) / S * S;
    // MXFP4: a scale chunk spans kScSteps K steps (a multiple of S, at most 32); sc_kb is its first step
    constexpr int kScSteps = 32 / S * S;
    int sc_kb = 0;
    for (int kb0 = 0; kb0 < nsteps; kb0 += S) {
        if constexpr (W4) {
            if (kb0 - sc_kb == kScSteps && kb0 < nkb) {  // next chunk (K > 32 steps): this wave's rows only,
                sc_kb = kb0;                              // a few words at a time to bound the registers
                wave_lds_fence();
#pragma unroll
                for (int i0 = 0; i0 < 16; i0 += 4) {
                    sc_issue(kb0, i0, 4);
                    sc_commit(i0, 4);
                }
                wave_lds_fence();
            }
        }
#pragma unroll
        for (int s = 0; s < S; s++) {
            const int kb = kb0 + s;
            // A and W step kb+S-1 into the stage and slot step kb-1 left.  A runs as far ahead as W:
            // loads retire in order, so waiting for A step kb+1 at the end of this step waits for no
            // W step beyond kb, and W keeps S-1 steps of lead through the whole step
            load_a(kb + S - 1 < last ? kb + S - 1 : last, (s + S - 1) % SA);
            load_w(kb + S - 1 < last ? kb + S - 1 : last, w_ring[(s + S - 1) % S]);
            const int buf = kb & 1;
            if (kb < nkb) {
                uint32_t scw[TPW];                        // MXFP4: the E8M0 dword of the step, per sub-tile
                if constexpr (W4) {
#pragma unroll
                    for (int c = 0; c < TPW; c++)
                        scw[c] = *reinterpret_cast<const uint32_t*>(sc_wave + (16 * c + (lane & 15)) * kScRow +
                                                                    4 * (kb - sc_kb));
                }
                float sw[TPW];                            // sub-tile c's weight scale (fused: gate, up)
#pragma unroll
                for (int c = 0; c < TPW; c++) sw[c] = W4 ? 1.0f : ws_lds[FUSED ? c : wsb][kb];
                v8i b[TPW];
                uint32_t e8[TPW];
#pragma unroll
                for (int c = 0; c < TPW; c++) {
                    b[c] = __builtin_shufflevector(w_ring[s][2 * c], w_ring[s][2 * c + 1], 0, 1, 2, 3, 4, 5, 6, 7);
                    if constexpr (W4) e8[c] = (scw[c] >> sshift) & 0xFFu;
                }
#pragma unroll
                for (int m = 0; m < MS; m++) {
                    // 16-row sub-tiles past the tile's rows are skipped (wave-uniform): an expert with
                    // 96 rows in a 128-row tile does 6 of the 8
                    if (MS > 4 && m * 16 >= tile_rows) continue;
                    // W is the MFMA's row operand and A its column operand, so a lane's four results
                    // share one A row (lane % 16) and take a single scale
                    const v8i a = __builtin_shufflevector(*reinterpret_cast<const v4i*>(&a_lds[buf][m * 2048 + a_p0]),
                                                          *reinterpret_cast<const v4i*>(&a_lds[buf][m * 2048 + a_p1]),
                                                          0, 1, 2, 3, 4, 5, 6, 7);
                    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
                    const float sa = sa_lds[kb * SA_ROW + m * 16 + (lane & 15)];
#pragma unroll
                    for (int c = 0; c < TPW; c++) {
                        if constexpr (W4)
                            acc[m][c] += mfma16x16x128_fp4_e4m3(w_ring[s][c], e8[c], a, zero) * sa;
                        else
                            acc[m][c] += mfma16x16x128_e4m3(b[c], a, zero) * (sa * sw[c]);
                    }
                }
            }
            store_a((s + 1) % SA, buf ^ 1);           // A step kb+1 (requested a step ago)
            __syncthreads();
        }
    }
    if constexpr (FUSED) {
        act_quant_epilogue<BM>(g, acc, row0, row_end, n_tile, lane, wave);
        return;
    }
    // ---- epilogue: lane holds row m*16 + lane%16, columns 4*(lane/16) + i of each 16-column sub-tile (the
    // 32-row block-FP8 tile, at 128 registers, keeps 8-byte stores: the swapped words would spill) ----
    store_tile_out<OUT_DT, MS, TPW, !(BM == 32 && !W4)>(g, acc, row0, row_end, n0 + wave * CPW, cols, lane);
}

// ---------------------------------------------------------------------------
// BM = 128: the tiles of a workgroup as one continuous K-step pipeline.  One workgroup fills a CU at this
// tile size, so nothing else on the CU hides a tile's start (the ring refilling from empty) or its
// epilogue (stores, or the fused activation requant).  Here the lookahead loads of a tile's last steps
// already fetch the next tile's first steps, and the next tile's A (and block-FP8 weight) scales,
// requested at the start of the tile before, are written into the other half of a double-buffered scale
// table once that tile's first group of K steps is under way.  MXFP4: each wave's E8M0 chunk of the next
// tile is requested before the epilogue and written to LDS after it (requested in the last group
// instead, its 16 registers stay live through the whole K loop and the long-K launches ran 3-5% slower).
// A tile's epilogue then runs while the next tile's first weight and A steps are in flight.  Every tile takes
// nsteps = ceil(K/128 / S) * S steps (the steps past K/128 only keep the ring in phase), so a step's
// ring slot and A stage are its index within the S-step group, as in grouped_gemm_tile.

// The wave-uniform position of one tile.
struct TileId {
    int expert, row0, row_end, n_tile;
};

template <int BM, int OUT_DT, bool FUSED, bool W4>
__device__ __forceinline__ void grouped_gemm_walk128(const GgArgs& g, const int* cum_lds, const int* off_lds, int t,
                                                     int hi, int m_tile, int n_tile) {
    using C = GgCfg<BM>;
    constexpr int TPW = C::TPW;
    constexpr int CPW = 16 * TPW;
    constexpr int MS = BM / 16;
    constexpr int S = C::S;
    constexpr int SA = C::S;
    constexpr int NT = C::THREADS;
    constexpr int A_CHUNKS = BM * 8;
    constexpr int A_PER_THREAD = (A_CHUNKS + NT - 1) / NT;
    constexpr int SA_ROW = BM + 4;
    constexpr int SA_ROWS = BM / C::WAVES;
    __shared__ __attribute__((aligned(32))) uint8_t a_lds[2][BM * 128];
    __shared__ __attribute__((aligned(16))) float sa_lds[2][kGgMaxKb * SA_ROW];   // [tile parity][kb][row]
    __shared__ float ws_lds[2][2][W4 ? 1 : kGgMaxKb];                              // [tile parity][block][kb]
    // MXFP4: each wave's E8M0 bytes of its 32 weight rows, 32 K steps at a time (as grouped_gemm_tile)
    __shared__ __attribute__((aligned(16))) uint8_t sc_lds[W4 ? C::WAVES * 32 * kScRow : 4];

    const uint8_t* __restrict__ a_q = g.a_q;
    const float* __restrict__ a_s = g.a_s;
    const uint8_t* __restrict__ w_q = g.w_q;
    const float* __restrict__ w_s = g.w_s;
    const int64_t N = g.N, K = g.K, I = N / 2;
    const int n_experts = g.n_experts, n_tiles_n = g.n_tiles_n, per_xcd = g.per_xcd;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int nkb = (int)(K / 128);
    const int last = nkb - 1;
    const int nsteps = (nkb + S - 1) / S * S;
    const int kbl = lane < nkb ? lane : nkb - 1;
    const int sshift = 8 * (lane / 16);
    uint8_t* const sc_wave = sc_lds + wave * 32 * kScRow;

    auto lookup = [&](int mt, int nt) {
        int e_lo = 0, e_hi = n_experts - 1;
        while (e_lo < e_hi) {
            const int mid = (e_lo + e_hi + 1) / 2;
            if (__builtin_amdgcn_readfirstlane(cum_lds[mid]) <= mt)
                e_lo = mid;
            else
                e_hi = mid - 1;
        }
        TileId ti;
        ti.expert = e_lo;
        ti.row0 = __builtin_amdgcn_readfirstlane(off_lds[e_lo]) + (mt - __builtin_amdgcn_readfirstlane(cum_lds[e_lo])) * BM;
        ti.row_end = __builtin_amdgcn_readfirstlane(off_lds[e_lo + 1]);
        ti.n_tile = nt;
        return ti;
    };
    auto advance = [&]() {
        t += per_xcd;
        m_tile += g.step_m;
        n_tile += g.step_n;
        if (n_tile >= n_tiles_n) {
            n_tile -= n_tiles_n;
            m_tile++;
        }
    };

    // per-lane addressing of a tile (the layout of each piece is grouped_gemm_tile's)
    struct Addr {
        const uint8_t* wp0;
        const uint8_t* wp1;
        int64_t a_src[A_PER_THREAD];
    };
    auto wcol_of = [&](const TileId& ti) -> int64_t {
        const int64_t n0 = (int64_t)ti.n_tile * C::BN;
        const bool cols = FUSED || n0 + wv * CPW < N;
        return FUSED ? (int64_t)ti.n_tile * 128 + 16 * wv : (cols ? n0 + wv * CPW : n0);
    };
    auto addr_of = [&](const TileId& ti) {
        Addr ad;
        const int64_t wcol = wcol_of(ti);
        ad.wp0 = w_q + w_lane_offset(g, ti.expert, wcol, lane);
        ad.wp1 = ad.wp0 + (FUSED ? I / 16 : 1) * g.w_group;
#pragma unroll
        for (int j = 0; j < A_PER_THREAD; j++) {
            const int c0 = tid + j * NT;
            const int c = c0 < A_CHUNKS ? c0 : c0 % A_CHUNKS;
            int row = ti.row0 + c / 8;
            if (row >= ti.row_end) row = ti.row_end - 1;
            ad.a_src[j] = (int64_t)row * g.a_stride + (c % 8) * 16;
        }
        return ad;
    };
    int a_dst[A_PER_THREAD];
#pragma unroll
    for (int j = 0; j < A_PER_THREAD; j++) {
        const int c0 = tid + j * NT;
        const int c = c0 < A_CHUNKS ? c0 : c0 % A_CHUNKS;
        const int rr = c / 8, ch = c % 8;
        a_dst[j] = (rr / 16) * 2048 + a_piece_offset((rr % 16) + 16 * (ch % 4), ch / 4);
    }
    const int a_p0 = a_piece_offset(lane, 0), a_p1 = a_piece_offset(lane, 1);   // this lane's MFMA pieces

    // a tile's scales: requested into registers (lane = K block), written to one half of the tables
    struct Scales {
        float sa[SA_ROWS];
        float ws;
    };
    auto scales_of = [&](const TileId& ti) {
        Scales sv;
#pragma unroll
        for (int j = 0; j < SA_ROWS; j++) {
            const int rr = wave + j * C::WAVES;
            const int row = ti.row0 + rr < ti.row_end ? ti.row0 + rr : ti.row_end - 1;
            sv.sa[j] = a_s[(int64_t)row * g.a_s_stride + kbl];
        }
        sv.ws = 0.0f;
        if (!W4 && wave < 2) {
            const int64_t n0 = (int64_t)ti.n_tile * C::BN;
            const int64_t nblk = (N - n0) >= 256 ? 2 : 1;
            const int64_t b = FUSED ? (wave == 0 ? ti.n_tile : I / 128 + ti.n_tile) : n0 / 128 + (wave < nblk ? wave : 0);
            sv.ws = w_s[(int64_t)ti.expert * g.w_s_stride_e + b * g.w_s_stride_n + kbl];
        }
        return sv;
    };
    auto commit_scales = [&](const Scales& sv, int tp) {
        if (lane < nkb) {
#pragma unroll
            for (int j = 0; j < SA_ROWS; j++) sa_lds[tp][lane * SA_ROW + wave + j * C::WAVES] = sv.sa[j];
            if (!W4 && wave < 2) ws_lds[tp][wave][lane] = sv.ws;
        }
    };
    // MXFP4: this wave's E8M0 chunk of a tile from K step kb0 (32 steps of its 32 rows; lanes 0-31 one row,
    // 32-63 the next), as 16 dwords per lane
    struct Chunk {
        uint32_t w[W4 ? 16 : 1];
    };
    auto chunk_of = [&](const TileId& ti, int kb0) {
        Chunk ck;
        if constexpr (W4) {
            const uint8_t* base = g.w4s + (int64_t)ti.expert * g.w4s_stride_e + wcol_of(ti) * g.w4s_stride_n;
            const int64_t sub = (FUSED ? I : 16) * g.w4s_stride_n;
            int l = lane;
            asm volatile("" : "+v"(l));
            const bool in = (l & 31) < nkb - kb0;
            const uint32_t lo = (uint32_t)((l >> 5) * g.w4s_stride_n + 4 * (l & 31));
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const uint8_t* u = base + (i / 8) * sub + (2 * (i % 8)) * g.w4s_stride_n + 4 * (int64_t)kb0;
                ck.w[i] = in ? *reinterpret_cast<const uint32_t*>(u + lo) : 0u;
            }
        }
        return ck;
    };
    auto commit_chunk = [&](const Chunk& ck) {
        if constexpr (W4) {
            wave_lds_fence();
#pragma unroll
            for (int i = 0; i < 16; i++)
                *reinterpret_cast<uint32_t*>(sc_wave + (2 * i + (lane >> 5)) * kScRow + 4 * (lane & 31)) = ck.w[i];
            wave_lds_fence();
        }
    };

    v4i a_reg[SA][A_PER_THREAD];
    v4i w_ring[S][2 * TPW];
    auto load_a = [&](const Addr& ad, int kb, int stage) {
#pragma unroll
        for (int j = 0; j < A_PER_THREAD; j++)
            a_reg[stage][j] = *reinterpret_cast<const v4i*>(a_q + ad.a_src[j] + (int64_t)kb * 128);
    };
    auto store_a = [&](int stage, int buf) {
#pragma unroll
        for (int j = 0; j < A_PER_THREAD; j++)
            if (A_CHUNKS % NT == 0 || tid + j * NT < A_CHUNKS)
                *reinterpret_cast<v4i*>(&a_lds[buf][a_dst[j]]) = a_reg[stage][j];
    };
    const int64_t kstep = g.w_kstep, khalf = g.w_khalf;
    auto load_w = [&](const Addr& ad, int kb, v4i* w) {
        const int64_t o = (int64_t)kb * kstep;
        if constexpr (W4) {
            w[0] = *reinterpret_cast<const v4i*>(ad.wp0 + o);
            w[1] = *reinterpret_cast<const v4i*>(ad.wp1 + o);
            return;
        }
        w[0] = *reinterpret_cast<const v4i*>(ad.wp0 + o);
        w[1] = *reinterpret_cast<const v4i*>(ad.wp0 + o + khalf);
        if constexpr (TPW == 2) {
            w[2] = *reinterpret_cast<const v4i*>(ad.wp1 + o);
            w[3] = *reinterpret_cast<const v4i*>(ad.wp1 + o + khalf);
        }
    };

    if (t >= hi) return;
    TileId cur = lookup(m_tile, n_tile);
    advance();
    bool has_next = t < hi;
    TileId nxt = has_next ? lookup(m_tile, n_tile) : cur;
    Addr ca = addr_of(cur);
    Addr na = addr_of(nxt);
    int tp = 0;                                      // half of the scale tables the current tile reads
    // prologue of the first tile: its scales, A and W steps 0..S-2, A step 0 into LDS
    {
        const Chunk c0 = chunk_of(cur, 0);
        const Scales s0 = scales_of(cur);
#pragma unroll
        for (int s = 0; s < S - 1; s++) {
            load_a(ca, s < last ? s : last, s % SA);
            load_w(ca, s < last ? s : last, w_ring[s]);
        }
        commit_chunk(c0);
        commit_scales(s0, 0);
    }
    store_a(0, 0);
    __syncthreads();
    int par = 0;                                     // A buffer of the current step
    for (;;) {
        const Scales sn = scales_of(nxt);            // the next tile's scales, written after the first group
        v4f acc[MS][TPW];
#pragma unroll
        for (int m = 0; m < MS; m++)
#pragma unroll
            for (int c = 0; c < TPW; c++) acc[m][c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        const int64_t n0 = (int64_t)cur.n_tile * C::BN;
        const bool cols = FUSED || n0 + wv * CPW < N;
        const int wsb = FUSED ? 0 : (int)((wcol_of(cur) - n0) / 128);
        const int tile_rows = __builtin_amdgcn_readfirstlane(cur.row_end - cur.row0);
        const float* sa_t = sa_lds[tp];
        int sc_kb = 0;                               // MXFP4: first K step of the chunk in sc_lds
        constexpr int kScSteps = 32 / S * S;
        for (int kb0 = 0; kb0 < nsteps; kb0 += S) {
            if constexpr (W4) {
                if (kb0 - sc_kb == kScSteps && kb0 < nkb) {   // next chunk of this tile (K > 32 steps)
                    sc_kb = kb0;
                    commit_chunk(chunk_of(cur, kb0));
                }
            }
#pragma unroll
            for (int s = 0; s < S; s++) {
                const int kb = kb0 + s;
                // the lookahead step: this tile's (its last step again past K/128), or, once it runs past
                // this tile's steps, the next tile's first steps (all loads unconditional: the pointers
                // are selected)
                const int la = kb + S - 1;
                const bool nx = la >= nsteps;
                const int ls = nx ? (la - nsteps < last ? la - nsteps : last) : (la < last ? la : last);
                Addr sel;
                sel.wp0 = nx ? na.wp0 : ca.wp0;
                sel.wp1 = nx ? na.wp1 : ca.wp1;
#pragma unroll
                for (int j = 0; j < A_PER_THREAD; j++) sel.a_src[j] = nx ? na.a_src[j] : ca.a_src[j];
                load_a(sel, ls, (s + S - 1) % SA);
                load_w(sel, ls, w_ring[(s + S - 1) % S]);
                if (kb < nkb) {
                    uint32_t e8[TPW];                     // MXFP4: the E8M0 byte of the step, per sub-tile
                    if constexpr (W4) {
#pragma unroll
                        for (int c = 0; c < TPW; c++)
                            e8[c] = (*reinterpret_cast<const uint32_t*>(sc_wave + (16 * c + (lane & 15)) * kScRow +
                                                                        4 * (kb - sc_kb)) >> sshift) & 0xFFu;
                    }
                    float sw[TPW];
#pragma unroll
                    for (int c = 0; c < TPW; c++) sw[c] = W4 ? 1.0f : ws_lds[tp][FUSED ? c : wsb][kb];
                    v8i b[TPW];
#pragma unroll
                    for (int c = 0; c < TPW; c++)
                        b[c] = __builtin_shufflevector(w_ring[s][2 * c], w_ring[s][2 * c + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                    for (int m = 0; m < MS; m++) {
                        if (MS > 4 && m * 16 >= tile_rows) continue;
                        const v8i a = __builtin_shufflevector(
                            *reinterpret_cast<const v4i*>(&a_lds[par][m * 2048 + a_p0]),
                            *reinterpret_cast<const v4i*>(&a_lds[par][m * 2048 + a_p1]), 0, 1, 2, 3, 4, 5, 6, 7);
                        const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
                        const float sa = sa_t[kb * SA_ROW + m * 16 + (lane & 15)];
#pragma unroll
                        for (int c = 0; c < TPW; c++) {
                            if constexpr (W4)
                                acc[m][c] += mfma16x16x128_fp4_e4m3(w_ring[s][c], e8[c], a, zero) * sa;
                            else
                                acc[m][c] += mfma16x16x128_e4m3(b[c], a, zero) * (sa * sw[c]);
                        }
                    }
                }
                store_a((s + 1) % SA, par ^ 1);     // A step kb+1 (the next tile's step 0 after the last step)
                __syncthreads();
                par ^= 1;
            }
            // after the first group (its loads issued, so the wait below covers only old requests): the
            // next tile's scales into the other half of the tables, read first after the tile boundary
            if (kb0 == 0 && has_next) commit_scales(sn, tp ^ 1);
        }
        // the tile's epilogue, with the next tile's first S-1 steps in flight (MXFP4: and its first E8M0
        // chunk; nxt is the current tile again after the last one)
        const Chunk cn = chunk_of(nxt, 0);
        if constexpr (FUSED) {
            act_quant_epilogue<BM>(g, acc, cur.row0, cur.row_end, cur.n_tile, lane, wave);
        } else {
            store_tile_out<OUT_DT, MS, TPW>(g, acc, cur.row0, cur.row_end, n0 + wave * CPW, cols, lane);
        }
        if (!has_next) return;
        commit_chunk(cn);                            // this wave's reads of the chunk ended with its last step
        cur = nxt;
        ca = na;
        tp ^= 1;
        advance();
        has_next = t < hi;
        nxt = has_next ? lookup(m_tile, n_tile) : cur;
        na = addr_of(nxt);
    }
}

template <int BM, int OUT_DT, bool FUSED, bool W4, bool WALK>
__global__ void __launch_bounds__(GgCfg<BM>::THREADS) __attribute__((amdgpu_waves_per_eu(GgCfg<BM>::WAVES_PER_EU, 8)))
grouped_gemm_kernel(GgArgs g) {
    const int32_t* __restrict__ offsets = g.offsets;
    const int n_experts = g.n_experts, m_rows = g.m_rows, n_tiles_n = g.n_tiles_n, per_xcd = g.per_xcd;
    const int step_m = g.step_m, step_n = g.step_n;
    using C = GgCfg<BM>;
    constexpr int NT = C::THREADS;
    constexpr int E_PER_THREAD = kMaxExpertsScan / NT;
    __shared__ int cum_lds[kMaxExpertsScan + 1];    // first M tile of each expert; [E] = live M tiles
    __shared__ int off_lds[kMaxExpertsScan + 1];    // expert row offsets
    __shared__ int scan_lds[C::WAVES];

    // ---- tile table, once per workgroup ----
    int local = 0, my_tiles[E_PER_THREAD];
#pragma unroll
    for (int i = 0; i < E_PER_THREAD; i++) {
        const int e = threadIdx.x * E_PER_THREAD + i;
        int t = 0;
        if (e < n_experts) {
            // offsets clamped to [0, m_rows] so that malformed offsets never reach past the rows
            const int o0 = min(max(offsets[e], 0), m_rows), o1 = min(max(offsets[e + 1], o0), m_rows);
            off_lds[e] = o0;
            if (e == n_experts - 1) off_lds[e + 1] = o1;
            t = (o1 - o0 + BM - 1) / BM;
        }
        my_tiles[i] = t;
        local += t;
    }
    int run = block_exclusive_scan<C::WAVES>(local, scan_lds);
#pragma unroll
    for (int i = 0; i < E_PER_THREAD; i++) {
        const int e = threadIdx.x * E_PER_THREAD + i;
        if (e < n_experts) cum_lds[e] = run;
        run += my_tiles[i];
    }
    if (threadIdx.x == NT - 1) cum_lds[n_experts] = run;     // threads past the experts hold no tiles
    __syncthreads();

    // ---- this workgroup's share: XCD range [lo, hi), every per_xcd-th tile from its slot ----
    const int64_t live = (int64_t)__builtin_amdgcn_readfirstlane(cum_lds[n_experts]) * n_tiles_n;
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int lo = (int)(live * xcd / kXcds), hi = (int)(live * (xcd + 1) / kXcds);
    int t = lo + slot;
    // (M tile, N tile) of t, advanced by (step_m, step_n) = divmod(per_xcd, n_tiles_n) per tile
    int m_tile = t / n_tiles_n, n_tile = t - m_tile * n_tiles_n;
    if constexpr (WALK) {
        grouped_gemm_walk128<BM, OUT_DT, FUSED, W4>(g, cum_lds, off_lds, t, hi, m_tile, n_tile);
    } else {
    for (; t < hi; t += per_xcd) {
        // last expert whose first tile <= m_tile; the table values are made wave-uniform so the tile's
        // addresses stay scalar
        int e_lo = 0, e_hi = n_experts - 1;
        while (e_lo < e_hi) {
            const int mid = (e_lo + e_hi + 1) / 2;
            if (__builtin_amdgcn_readfirstlane(cum_lds[mid]) <= m_tile)
                e_lo = mid;
            else
                e_hi = mid - 1;
        }
        const int expert = e_lo;
        const int row0 = __builtin_amdgcn_readfirstlane(off_lds[expert]) +
                         (m_tile - __builtin_amdgcn_readfirstlane(cum_lds[expert])) * BM;
        const int row_end = __builtin_amdgcn_readfirstlane(off_lds[expert + 1]);
        grouped_gemm_tile<BM, OUT_DT, FUSED, W4>(g, expert, row0, row_end, n_tile);
        m_tile += step_m;
        n_tile += step_n;
        if (n_tile >= n_tiles_n) {
            n_tile -= n_tiles_n;
            m_tile++;
        }
    }
    }
}

// Workgroups of one configuration the device holds at once (cached per device and variant).
template <int BM, int OUT_DT, bool FUSED, bool W4, bool WALK>
static int gg_resident_blocks() {
    using C = GgCfg<BM>;
    static std::atomic<int> cached[64];   // concurrent first calls may both fill it, with the same value
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int c = cached[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, grouped_gemm_kernel<BM, OUT_DT, FUSED, W4, WALK>, C::THREADS,
                                                         0) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        c = per_cu * cus > 0 ? per_cu * cus : -1;
        cached[dev].store(c, std::memory_order_relaxed);
    }
    return c > 0 ? c : 0;
}

// Fills the tile walk of g (N tiles of BN columns, or I/128 act groups when fused) and launches.
template <int BM, int OUT_DT, bool FUSED, bool W4, bool WALK>
static int launch_grouped_walk(hipStream_t st, GgArgs g) {
    using C = GgCfg<BM>;
    if (g.N % 128 != 0 || (FUSED && g.N % 256 != 0)) return MOE_ERR_SHAPE;
    const int64_t n_tiles_n = FUSED ? g.N / 256 : ceil_div(g.N, C::BN);
    // m_rows fits an int (the entry points reject more); the tile count must too
    if (n_tiles_n * (ceil_div((int64_t)g.m_rows, BM) + g.n_experts) > 0x7FFFFFFF - (1 << 20))
        return MOE_ERR_SHAPE;
    const int wgs = gg_resident_blocks<BM, OUT_DT, FUSED, W4, WALK>();
    if (wgs < kXcds) return MOE_ERR_HIP;
    g.n_tiles_n = (int)n_tiles_n;
    g.per_xcd = wgs / kXcds;
    g.step_m = g.per_xcd / g.n_tiles_n;
    g.step_n = g.per_xcd % g.n_tiles_n;
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, OUT_DT, FUSED, W4, WALK>), dim3((unsigned)(g.per_xcd * kXcds)),
                       dim3(C::THREADS), 0, st, g);
    return launch_status();
}

// BM = 128 runs a workgroup's tiles as one pipeline (grouped_gemm_walk128).  With MXFP4 weights only up
// to kW4WalkMaxKb K steps per tile: at the 24576-route prefill (E = 256, I = 1024) it took the down GEMM
// (8 steps) from 290 to 260-265 us at H = 4096 and from 155 to 141 us at H = 2048, and the H = 2048
// gate/up GEMM (16 steps) 1-3 % faster, but the H = 4096 gate/up GEMM (32 steps) ran 1-5 % slower than
// with tiles one at a time.
constexpr int kW4WalkMaxKb = 16;

template <int BM, int OUT_DT, bool FUSED, bool W4>
static int launch_grouped(hipStream_t st, const GgArgs& g) {
    if constexpr (BM == 128 && !W4)
        return launch_grouped_walk<BM, OUT_DT, FUSED, W4, true>(st, g);
    else if constexpr (BM == 128)
        return g.K / 128 <= kW4WalkMaxKb ? launch_grouped_walk<BM, OUT_DT, FUSED, W4, true>(st, g)
                                         : launch_grouped_walk<BM, OUT_DT, FUSED, W4, false>(st, g);
    else
        return launch_grouped_walk<BM, OUT_DT, FUSED, W4, false>(st, g);
}

template <int BM, bool W4>
static int launch_grouped_dt(hipStream_t st, int out_dt, bool fused, const GgArgs& g) {
    if (fused) return launch_grouped<BM, kF32, true, W4>(st, g);
    if (out_dt == MOE_F32) return launch_grouped<BM, kF32, false, W4>(st, g);
    if (out_dt == MOE_BF16) return launch_grouped<BM, kBF16, false, W4>(st, g);
    return launch_grouped<BM, kF16, false, W4>(st, g);
}

template <bool W4>
static int grouped_launch_w(hipStream_t st, int block_m, int out_dt, bool fused, const GgArgs& g) {
    switch (block_m) {
        case 16: return launch_grouped_dt<16, W4>(st, out_dt, fused, g);
        case 32: return launch_grouped_dt<32, W4>(st, out_dt, fused, g);
        case 64: return launch_grouped_dt<64, W4>(st, out_dt, fused, g);
        case 128: return launch_grouped_dt<128, W4>(st, out_dt, fused, g);
        default: return MOE_ERR_SHAPE;
    }
}

static int grouped_launch_bm(hipStream_t st, int block_m, int out_dt, bool fused, const GgArgs& g) {
    if (g.n_experts > kMaxExpertsScan || g.K / 128 > kGgMaxKb) return MOE_ERR_SHAPE;
    return g.w4s ? grouped_launch_w<true>(st, block_m, out_dt, fused, g)
                 : grouped_launch_w<false>(st, block_m, out_dt, fused, g);
}

int grouped_gemm_launch(hipStream_t st, int block_m, const uint8_t* a_q, int64_t a_stride, const float* a_s,
                        int64_t a_s_stride, const uint8_t* w_q, int64_t w_stride_e, int64_t w_stride_n,
                        const float* w_s, int64_t w_s_stride_e, int64_t w_s_stride_n, int64_t E, int64_t N,
                        int64_t K, const int32_t* offsets, int64_t m_rows, void* out, int out_dt,
                        int64_t out_stride) {
    GgArgs g{};
    g.a_q = a_q; g.a_stride = a_stride; g.a_s = a_s; g.a_s_stride = a_s_stride;
    g.w_q = w_q; g.w_stride_e = w_stride_e; g.w_stride_n = w_stride_n;
    g.w_s = w_s; g.w_s_stride_e = w_s_stride_e; g.w_s_stride_n = w_s_stride_n;
    g.n_experts = (int)E; g.N = N; g.K = K; g.offsets = offsets; g.m_rows = (int)m_rows;
    g.out = out; g.out_stride = out_stride;
    set_weight_layout(g, false);
    return grouped_launch_bm(st, block_m, out_dt, false, g);
}

// MXFP4 weights: w4 [E][N][K/2] bytes, w4s [E][N][K/32] E8M0 (strides in bytes); out as the plain GEMM, or
// (act > 0) the fused gated-activation requant into q/s.
int mxfp4_grouped_gemm_launch(hipStream_t st, int block_m, int act, const uint8_t* a_q, int64_t a_stride,
                              const float* a_s, int64_t a_s_stride, const uint8_t* w4, int64_t w4_stride_e,
                              int64_t w4_stride_n, const uint8_t* w4s, int64_t w4s_stride_e, int64_t w4s_stride_n,
                              int64_t E, int64_t N, int64_t K, const int32_t* offsets, int64_t m_rows, void* out,
                              int out_dt, int64_t out_stride, uint8_t* q, int64_t q_stride, float* s,
                              int64_t s_stride) {
    GgArgs g{};
    g.a_q = a_q; g.a_stride = a_stride; g.a_s = a_s; g.a_s_stride = a_s_stride;
    g.w_q = w4; g.w_stride_e = w4_stride_e; g.w_stride_n = w4_stride_n;
    g.w4s = w4s; g.w4s_stride_e = w4s_stride_e; g.w4s_stride_n = w4s_stride_n;
    g.n_experts = (int)E; g.N = N; g.K = K; g.offsets = offsets; g.m_rows = (int)m_rows;
    g.out = out; g.out_stride = out_stride;
    g.q = q; g.q_stride = q_stride; g.s = s; g.s_stride = s_stride; g.act = act;
    set_weight_layout(g, true);
    return grouped_launch_bm(st, block_m, out_dt, act > 0, g);
}

int grouped_gemm_act_quant_launch(hipStream_t st, int block_m, int act, const uint8_t* a_q, int64_t a_stride,
                                  const float* a_s, int64_t a_s_stride, const uint8_t* w_q, int64_t w_stride_e,
                                  int64_t w_stride_n, const float* w_s, int64_t w_s_stride_e,
                                  int64_t w_s_stride_n, int64_t E, int64_t I, int64_t K, const int32_t* offsets,
                                  int64_t m_rows, uint8_t* q, int64_t q_stride, float* s, int64_t s_stride) {
    GgArgs g{};
    g.a_q = a_q; g.a_stride = a_stride; g.a_s = a_s; g.a_s_stride = a_s_stride;
    g.w_q = w_q; g.w_stride_e = w_stride_e; g.w_stride_n = w_stride_n;
    g.w_s = w_s; g.w_s_stride_e = w_s_stride_e; g.w_s_stride_n = w_s_stride_n;
    g.n_experts = (int)E; g.N = 2 * I; g.K = K; g.offsets = offsets; g.m_rows = (int)m_rows;
    g.q = q; g.q_stride = q_stride; g.s = s; g.s_stride = s_stride; g.act = act;
    set_weight_layout(g, false);
    return grouped_launch_bm(st, block_m, MOE_F32, true, g);
}

}  // namespace moe
