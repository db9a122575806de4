// One decode step of the routed experts in two launches ("perf(moe): skip
// inactive block-fp8 decode routes": gate/up, activation, down and reduction
// for a batch-1 step under graph replay; a negative slot writes zero tiles and
// reads nothing of that route).
//
// MI355X design.  A decode step streams every active route's W13 and W2 once
// and nothing else is large, so the step is an HBM stream; what costs time
// beyond the stream is kernel boundaries and dependent memory round trips.
// Cross-workgroup handoff inside one kernel needs agent-scope release/acquire
// (an L2 write-back and invalidate on this 8-XCD part) or device-scope
// polling, both of which measured slower than one extra launch, so the step is:
//
//  * launch 1 (gate/up + SiLU): route r, 8 activation columns.  The 16 MFMA
//    columns of the tile are 8 gate rows of W13 and the 8 matching up rows, so
//    after the split-K sum the tile forms h = SiLU(gate)*up for its columns.
//    All of K = H is split over 8 waves; each wave quantizes the 128-column
//    groups of the bf16 token row it needs (amax/448, v/s -> e4m3) into LDS
//    while its weight loads are in flight, runs one 16x16x128 e4m3 MFMA per K
//    block and scales the block partial by a_s[kb] * w_s[row/128][kb].  The
//    8 waves' partials are summed in LDS in wave order; C1 and h are stored.
//  * launch 2 (requant + down + reduce): token t, 8 (or, when H/16 tiles
//    already give one workgroup per CU, 16) rows of W2 for all of t's routes; wave j owns route j.  It loads the route's h (2 columns per lane
//    per 128-group) before its W2 rows, so the 1x128 requant (amax/448,
//    v/s -> e4m3, via LDS into MFMA operand order) runs while the weights are
//    in flight, then multiplies and parks the route's fp32 C2 rows in LDS and
//    the workspace.  An 8-row tile uses the 16 MFMA columns as two K
//    streams, so a token has H/8 tiles to spread the W2 stream over every
//    CU.  Wave 0 sums the routes in ascending j with their routing weights
//    and writes the bf16 output.
//
// Group maxima use DPP row moves and row broadcasts (no LDS round trips), and
// every load a wave needs early (token row, h) is issued before its weight
// loads, since loads retire in order.
//
// Results are deterministic: split-K partials and routes are combined in a
// fixed order, and no floating-point atomics are used.
#include "device.h"
#include "host.h"
#include "decode_args.h"

namespace moe {

constexpr int kFdTile = 16;
constexpr int kFdWaves = 8;
constexpr int kFdUnroll = 2;
constexpr int kFdMaxNkb2 = 8;          // I/128 handled with W2 rows held in registers
constexpr int kDnRows = 8;             // W2 rows per narrow down tile
constexpr int kWideDownTiles = 256;    // 16-row down tiles from this many tiles per step on (one per CU)


__device__ __forceinline__ v8i frag(uint4 lo, uint4 hi) {
    v8i f;
    f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
    f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
    return f;
}

__device__ __forceinline__ v8i frag(v4i lo, v4i hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Launch 1.  Tile = route r, act columns [8*j8, 8*j8+8): MFMA columns 0..7 are
// gate rows 8*j8.., columns 8..15 the matching up rows I+8*j8.., so the tile
// can form h = SiLU(gate)*up for its 8 columns after the split-K sum.
__global__ void __launch_bounds__(kWave * kFdWaves) decode_gateup_kernel(FusedDecodeArgs a) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int b = blockIdx.x;
    const int64_t r = b / a.tiles_a;
    const int64_t c0 = (int64_t)(b % a.tiles_a) * 8;            // first act column
    const int64_t N = 2 * (int64_t)a.I;
    const int slot = a.slots[r];
    __shared__ float red[kFdWaves][kFdTile];
    __shared__ __attribute__((aligned(16))) uint8_t xq[kFdWaves][kFdUnroll][128];
    const int col = lane & 15;                                   // MFMA column of this lane
    const int64_t wr = col < 8 ? c0 + col : a.I + c0 + (col - 8); // its W13 row
    if (slot < 0) {
        if (threadIdx.x < kFdTile) {
            const int64_t rr = threadIdx.x < 8 ? c0 + threadIdx.x : a.I + c0 + (threadIdx.x - 8);
            a.c1[r * N + rr] = 0.0f;
            if (threadIdx.x < 8) a.h[r * a.I + c0 + threadIdx.x] = 0.0f;
        }
        return;
    }
    const int nkb = a.H / 128;
    const int kb0 = wave * nkb / kFdWaves, kb1 = (wave + 1) * nkb / kFdWaves;
    const int q16 = (lane / 16) * 16;
    const uint8_t* wrow = a.w13 + (int64_t)slot * N * a.H + wr * a.H + q16;
    const float* wsrow = a.w13s + (int64_t)slot * (N / 128) * nkb + (wr / 128) * nkb;  // per-lane scale row
    const uint16_t* xrow = a.x + (r / a.topk) * a.H;
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int kb = kb0; kb < kb1; kb += kFdUnroll) {
        v4i blo[kFdUnroll], bhi[kFdUnroll], alo[kFdUnroll], ahi[kFdUnroll];
        float sa[kFdUnroll], sw[kFdUnroll];
        uint32_t pair[kFdUnroll];
        // token row first: its quantization then overlaps the weight stream (loads retire in order)
#pragma unroll
        for (int u = 0; u < kFdUnroll; u++)
            if (kb + u < kb1) pair[u] = reinterpret_cast<const uint32_t*>(xrow + (int64_t)(kb + u) * 128)[lane];
#pragma unroll
        for (int u = 0; u < kFdUnroll; u++) {
            if (kb + u < kb1) {
                const uint8_t* wp = wrow + (int64_t)(kb + u) * 128;
                blo[u] = *reinterpret_cast<const v4i*>(wp);
                bhi[u] = *reinterpret_cast<const v4i*>(wp + 64);
                sw[u] = wsrow[kb + u];
            }
        }
#pragma unroll
        for (int u = 0; u < kFdUnroll; u++) {
            if (kb + u < kb1) {
                const float v0 = bf16_to_f32((uint16_t)(pair[u] & 0xFFFF));
                const float v1 = bf16_to_f32((uint16_t)(pair[u] >> 16));
                const float amax = wave_max(__builtin_fmaxf(__builtin_fabsf(v0), __builtin_fabsf(v1)));
                const float s = amax / 448.0f;
                reinterpret_cast<uint16_t*>(xq[wave][u])[lane] = (uint16_t)(s != 0.0f ? enc2_e4m3(v0 / s, v1 / s) : 0u);
                sa[u] = s;
            }
        }
        wave_lds_fence();
#pragma unroll
        for (int u = 0; u < kFdUnroll; u++) {
            if (kb + u < kb1) {
                alo[u] = *reinterpret_cast<const v4i*>(&xq[wave][u][q16]);
                ahi[u] = *reinterpret_cast<const v4i*>(&xq[wave][u][64 + q16]);
            }
        }
#pragma unroll
        for (int u = 0; u < kFdUnroll; u++) {
            if (kb + u < kb1) {
                const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
                const v4f p = mfma16x16x128_e4m3(frag(alo[u], ahi[u]), frag(blo[u], bhi[u]), z);
                acc += p * (sa[u] * sw[u]);
            }
        }
        wave_lds_fence();
    }
    if (lane < kFdTile) red[wave][lane] = acc[0];
    __syncthreads();
    if (threadIdx.x < kFdTile) {
        float t = red[0][threadIdx.x];
#pragma unroll
        for (int w = 1; w < kFdWaves; w++) t += red[w][threadIdx.x];
        const int64_t rr = threadIdx.x < 8 ? c0 + threadIdx.x : a.I + c0 + (threadIdx.x - 8);
        a.c1[r * N + rr] = t;
        const float up = __shfl_down(t, 8, kFdTile);            // lanes 0..7 get their up value
        if (threadIdx.x < 8) a.h[r * a.I + c0 + threadIdx.x] = (t / (1.0f + expf(-t))) * up;
    }
}

// Launch 2: token t, W2 rows [n0, n0+8) for all of t's routes; wave j owns
// route j (then j+8, ...).  MFMA column c holds W2 row n0 + (c & 7) on K stream
// c >> 3: stream 0 covers K blocks [0, NS), stream 1 blocks [NS, NKB2).  A row 0
// carries stream 0's activation block and A row 1 stream 1's, so C[0][c]
// (c < 8) and C[1][c] (c >= 8) are the two streams' partials of one W2 row; a
// wave holds half of its rows' weight bytes per MFMA column, and a token has
// H/8 tiles, enough to spread the W2 stream over every CU.
template <int NKB2>
__global__ void __launch_bounds__(kWave * kFdWaves) decode_down8_kernel(FusedDecodeArgs a) {
    constexpr int NS = (NKB2 + 1) / 2;
    constexpr bool kOdd = (NKB2 & 1) != 0;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int64_t t = blockIdx.x / a.tiles_c;
    const int ntile = blockIdx.x % a.tiles_c;
    const int64_t n0 = (int64_t)ntile * kDnRows;
    const int col = lane & 15, q16 = (lane / 16) * 16;
    const int strm = col >> 3;                                   // K stream of this lane's B column
    __shared__ float part[64][kDnRows];                          // routing weight x C2 of route j
    __shared__ int on[64];
    __shared__ __attribute__((aligned(16))) uint8_t hq[kFdWaves][NKB2][128];
    for (int j = wave; j < a.topk; j += kFdWaves) {
        const int64_t r = t * a.topk + j;
        const int slot = a.slots[r];
        float val = 0.0f, wgt = 0.0f;
        if (slot >= 0) {
            wgt = a.weights[r];
            // h first: its requant then overlaps the W2 stream (loads retire in order)
            const float* hrow = a.h + r * a.I + 2 * lane;
            float2 hv[NKB2];
#pragma unroll
            for (int kb = 0; kb < NKB2; kb++) hv[kb] = *reinterpret_cast<const float2*>(hrow + kb * 128);
            // W2 fragments; stream 1's missing last block (odd NKB2) reads a valid block, zeroed below
            const uint8_t* wrow = a.w2 + (int64_t)slot * a.H * a.I + (n0 + (col & 7)) * a.I + q16;
            v4i blo[NS], bhi[NS];
#pragma unroll
            for (int i = 0; i < NS; i++) {
                const int kb = strm * NS + i < NKB2 ? strm * NS + i : NKB2 - 1;
                blo[i] = *reinterpret_cast<const v4i*>(wrow + kb * 128);
                bhi[i] = *reinterpret_cast<const v4i*>(wrow + kb * 128 + 64);
            }
            const float* wsrow = a.w2s + (int64_t)slot * (a.H / 128) * NKB2 + (n0 / 128) * NKB2;
            float sa[NKB2];
#pragma unroll
            for (int kb = 0; kb < NKB2; kb++) {
                const float amax = wave_max(__builtin_fmaxf(__builtin_fabsf(hv[kb].x), __builtin_fabsf(hv[kb].y)));
                const float s = amax / 448.0f;
                const uint16_t codes = (uint16_t)(s != 0.0f ? enc2_e4m3(hv[kb].x / s, hv[kb].y / s) : 0u);
                reinterpret_cast<uint16_t*>(hq[wave][kb])[lane] = codes;
                sa[kb] = s;
                if (ntile == 0) {
                    reinterpret_cast<uint16_t*>(a.aq + r * a.I)[kb * 64 + lane] = codes;
                    if (lane == 0) a.as[r * NKB2 + kb] = s;
                }
            }
            wave_lds_fence();
            const int m = lane & 15;                                 // A row of this lane
            const v4i zero4 = {0, 0, 0, 0};
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < NS; i++) {
                const bool has1 = !(kOdd && i == NS - 1);            // stream 1 has a block at this step
                const int kbA = (m == 1 && has1) ? NS + i : i;
                v4i alo = *reinterpret_cast<const v4i*>(&hq[wave][kbA][q16]);
                v4i ahi = *reinterpret_cast<const v4i*>(&hq[wave][kbA][64 + q16]);
                const bool a_on = m == 0 || (m == 1 && has1);
                alo = a_on ? alo : zero4;
                ahi = a_on ? ahi : zero4;
                const bool b_on = strm == 0 || has1;
                const v4i bl = b_on ? blo[i] : zero4, bh = b_on ? bhi[i] : zero4;
                const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
                const v4f p = mfma16x16x128_e4m3(frag(alo, ahi), frag(bl, bh), z);
                const float f0 = sa[i] * wsrow[i];
                const float f1 = has1 ? sa[(NS + i) % NKB2] * wsrow[(NS + i) % NKB2] : 0.0f;
                acc += strm == 0 ? p[0] * f0 : p[1] * f1;
            }
            wave_lds_fence();
            val = acc + __shfl_down(acc, 8, 16);                     // lanes 0..7: stream 0 + stream 1
        } else if (ntile == 0) {
            for (int i = lane; i < a.I / 4; i += kWave) reinterpret_cast<uint32_t*>(a.aq + r * a.I)[i] = 0u;
            if (lane < NKB2) a.as[r * NKB2 + lane] = 0.0f;
        }
        if (lane < kDnRows) {
            part[j][lane] = wgt * val;
            a.c2[r * a.H + n0 + lane] = val;
        }
        if (lane == 0) on[j] = slot >= 0;
    }
    __syncthreads();
    if (threadIdx.x < kDnRows) {
        float o = 0.0f;
        for (int j = 0; j < a.topk; j++)
            if (on[j]) o += part[j][threadIdx.x];
        a.out[t * a.H + n0 + threadIdx.x] = f32_to_bf16(o);
    }
}

// Launch 2, wide form (used when H/16 tiles already fill the GPU): token t,
// 16 rows of W2, 8 waves, wave j owns route j (then j+8, ...); the routes' C2
// rows meet in LDS.  The token's slots and the routing
// weights of its active routes are fetched once into LDS.
template <int NKB2>
__global__ void __launch_bounds__(kWave * kFdWaves) decode_down16_kernel(FusedDecodeArgs a) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int64_t t = blockIdx.x / a.tiles_c;
    const int ntile = blockIdx.x % a.tiles_c;
    const int64_t n0 = (int64_t)ntile * kFdTile;
    const int q16 = (lane / 16) * 16;
    __shared__ float part[64][kFdTile];
    __shared__ int s_slot[64];
    __shared__ float s_w[64];
    __shared__ __attribute__((aligned(16))) uint8_t hq[kFdWaves][NKB2][128];
    if (threadIdx.x < a.topk) {
        const int sl = a.slots[t * a.topk + threadIdx.x];
        s_slot[threadIdx.x] = sl;
        s_w[threadIdx.x] = sl >= 0 ? a.weights[t * a.topk + threadIdx.x] : 0.0f;
    }
    __syncthreads();
    for (int j = wave; j < a.topk; j += kFdWaves) {
        const int64_t r = t * a.topk + j;
        const int slot = s_slot[j];
        float val = 0.0f;
        if (slot >= 0) {
            const float* hrow = a.h + r * a.I + 2 * lane;
            float2 hv[NKB2];
#pragma unroll
            for (int kb = 0; kb < NKB2; kb++) hv[kb] = *reinterpret_cast<const float2*>(hrow + kb * 128);
            v4i blo[NKB2], bhi[NKB2];
            const uint8_t* wrow = a.w2 + (int64_t)slot * a.H * a.I + (n0 + (lane & 15)) * a.I + q16;
#pragma unroll
            for (int kb = 0; kb < NKB2; kb++) {
                blo[kb] = *reinterpret_cast<const v4i*>(wrow + kb * 128);
                bhi[kb] = *reinterpret_cast<const v4i*>(wrow + kb * 128 + 64);
            }
            float sa[NKB2];
#pragma unroll
            for (int kb = 0; kb < NKB2; kb++) {
                const float amax = wave_max(__builtin_fmaxf(__builtin_fabsf(hv[kb].x), __builtin_fabsf(hv[kb].y)));
                const float s = amax / 448.0f;
                const uint16_t codes = (uint16_t)(s != 0.0f ? enc2_e4m3(hv[kb].x / s, hv[kb].y / s) : 0u);
                reinterpret_cast<uint16_t*>(hq[wave][kb])[lane] = codes;
                sa[kb] = s;
                if (ntile == 0) {
                    reinterpret_cast<uint16_t*>(a.aq + r * a.I)[kb * 64 + lane] = codes;
                    if (lane == 0) a.as[r * NKB2 + kb] = s;
                }
            }
            wave_lds_fence();
            const float* wsrow = a.w2s + (int64_t)slot * (a.H / 128) * NKB2 + (n0 / 128) * NKB2;
            v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kb = 0; kb < NKB2; kb++) {
                const v4i alo = *reinterpret_cast<const v4i*>(&hq[wave][kb][q16]);
                const v4i ahi = *reinterpret_cast<const v4i*>(&hq[wave][kb][64 + q16]);
                const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
                const v4f p = mfma16x16x128_e4m3(frag(alo, ahi), frag(blo[kb], bhi[kb]), z);
                acc += p * (sa[kb] * wsrow[kb]);
            }
            wave_lds_fence();
            val = acc[0];
        } else if (ntile == 0) {
            for (int i = lane; i < a.I / 4; i += kWave) reinterpret_cast<uint32_t*>(a.aq + r * a.I)[i] = 0u;
            if (lane < NKB2) a.as[r * NKB2 + lane] = 0.0f;
        }
        if (lane < kFdTile) {
            part[j][lane] = val;
            a.c2[r * a.H + n0 + lane] = val;
        }
    }
    __syncthreads();
    if (threadIdx.x < kFdTile) {
        float o = 0.0f;
        for (int j = 0; j < a.topk; j++)
            if (s_slot[j] >= 0) o += s_w[j] * part[j][threadIdx.x];
        a.out[t * a.H + n0 + threadIdx.x] = f32_to_bf16(o);
    }
}

int fused_decode_two_launch(hipStream_t st, FusedDecodeArgs a) {
    if (a.I / 128 < 1 || a.I / 128 > kFdMaxNkb2) return MOE_ERR_SHAPE;
    a.tiles_a = a.I / 8;
    a.n_a = a.T * a.topk * a.tiles_a;
    // 16-row down tiles once they alone give a workgroup per CU (each tile re-reads the token's h,
    // so fewer, wider tiles read less of it); 8-row tiles otherwise
    const bool wide = (int64_t)a.T * (a.H / kFdTile) >= kWideDownTiles;
    a.tiles_c = a.H / (wide ? kFdTile : kDnRows);
    hipLaunchKernelGGL(decode_gateup_kernel, dim3((unsigned)a.n_a), dim3(kWave * kFdWaves), 0, st, a);
    const unsigned down = (unsigned)(a.T * a.tiles_c);
    switch (a.I / 128) {
#define MOE_FD_CASE(n)                                                                                                  \
    case n:                                                                                                             \
        if (wide) hipLaunchKernelGGL((decode_down16_kernel<n>), dim3(down), dim3(kWave * kFdWaves), 0, st, a);         \
        else hipLaunchKernelGGL((decode_down8_kernel<n>), dim3(down), dim3(kWave * kFdWaves), 0, st, a);               \
        break;
        MOE_FD_CASE(1) MOE_FD_CASE(2) MOE_FD_CASE(3) MOE_FD_CASE(4)
        MOE_FD_CASE(5) MOE_FD_CASE(6) MOE_FD_CASE(7) MOE_FD_CASE(8)
#undef MOE_FD_CASE
        default: return MOE_ERR_SHAPE;
    }
    return launch_status();
}

}  // namespace moe
