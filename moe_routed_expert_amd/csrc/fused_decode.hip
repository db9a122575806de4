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
#include <atomic>

#include "device.h"
#include "host.h"
#include "decode_args.h"

namespace moe {

constexpr int kFdTile = 16;
constexpr int kFdWaves = 8;
// K blocks per batch of a gate/up wave, in both step forms: paced requests of one block finish the full
// W13 flood sooner at 8/8 active, at some cost with fewer routes active
constexpr int kFdUnroll = 1;
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

// 1x128 requant of an activation pair inside the fused step (the a3 step, held
// to tolerance): s = amax/448 exactly, codes e4m3(v/s) with v/s formed as
// v * (448 * rcp(amax)), within a few fp32 ulps of the quotient before the
// e4m3 rounding.  Groups whose amax is tiny take exact divisions.
__device__ __forceinline__ uint16_t requant_pair(float v0, float v1, float amax, float& s) {
    s = amax / 448.0f;
    if (amax >= 0x1p-100f) {
        const float inv = 448.0f * __builtin_amdgcn_rcpf(amax);
        return (uint16_t)enc2_e4m3(v0 * inv, v1 * inv);
    }
    return (uint16_t)(s != 0.0f ? enc2_e4m3(v0 / s, v1 / s) : 0u);
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
        if (threadIdx.x < 8) a.h[r * a.I + c0 + threadIdx.x] = gated_act(a.act, t, up);
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
            // the tile's W2 block scales travel with its fragments
            const float* wsrow = a.w2s + (int64_t)slot * (a.H / 128) * NKB2 + (n0 / 128) * NKB2;
            float sw[NKB2];
#pragma unroll
            for (int kb = 0; kb < NKB2; kb++) sw[kb] = wsrow[kb];
            float sa[NKB2];
#pragma unroll
            for (int kb = 0; kb < NKB2; kb++) {
                const float amax = wave_max(__builtin_fmaxf(__builtin_fabsf(hv[kb].x), __builtin_fabsf(hv[kb].y)));
                float s;
                const uint16_t codes = requant_pair(hv[kb].x, hv[kb].y, amax, s);
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
                const float f0 = sa[i] * sw[i];
                const float f1 = has1 ? sa[(NS + i) % NKB2] * sw[(NS + i) % NKB2] : 0.0f;
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
// rows meet in LDS.  Each wave reads its route's slot itself, so its h and W2
// loads wait for that one load only; the routing weight is read (for an active
// route only) after them and is first needed at the end.
template <int NKB2>
__global__ void __launch_bounds__(kWave * kFdWaves) decode_down16_kernel(FusedDecodeArgs a) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int64_t t = blockIdx.x / a.tiles_c;
    const int ntile = blockIdx.x % a.tiles_c;
    const int64_t n0 = (int64_t)ntile * kFdTile;
    const int q16 = (lane / 16) * 16;
    __shared__ float part[64][kFdTile];                          // routing weight x C2 of route j (+0 if inactive)
    __shared__ __attribute__((aligned(16))) uint8_t hq[kFdWaves][NKB2][128];
    for (int j = wave; j < a.topk; j += kFdWaves) {
        const int64_t r = t * a.topk + j;
        const int slot = a.slots[r];
        float val = 0.0f, wgt = 0.0f;
        if (slot >= 0) {
            // h first: its requant then overlaps the W2 stream (loads retire in order)
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
            // the tile's W2 block scales travel with its fragments
            const float* wsrow = a.w2s + (int64_t)slot * (a.H / 128) * NKB2 + (n0 / 128) * NKB2;
            float sw[NKB2];
#pragma unroll
            for (int kb = 0; kb < NKB2; kb++) sw[kb] = wsrow[kb];
            wgt = a.weights[r];
            float sa[NKB2];
#pragma unroll
            for (int kb = 0; kb < NKB2; kb++) {
                const float amax = wave_max(__builtin_fmaxf(__builtin_fabsf(hv[kb].x), __builtin_fabsf(hv[kb].y)));
                float s;
                const uint16_t codes = requant_pair(hv[kb].x, hv[kb].y, amax, s);
                reinterpret_cast<uint16_t*>(hq[wave][kb])[lane] = codes;
                sa[kb] = s;
                if (ntile == 0) {
                    reinterpret_cast<uint16_t*>(a.aq + r * a.I)[kb * 64 + lane] = codes;
                    if (lane == 0) a.as[r * NKB2 + kb] = s;
                }
            }
            wave_lds_fence();
            v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kb = 0; kb < NKB2; kb++) {
                const v4i alo = *reinterpret_cast<const v4i*>(&hq[wave][kb][q16]);
                const v4i ahi = *reinterpret_cast<const v4i*>(&hq[wave][kb][64 + q16]);
                const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
                const v4f p = mfma16x16x128_e4m3(frag(alo, ahi), frag(blo[kb], bhi[kb]), z);
                acc += p * (sa[kb] * sw[kb]);
            }
            wave_lds_fence();
            val = acc[0];
        } else if (ntile == 0) {
            for (int i = lane; i < a.I / 4; i += kWave) reinterpret_cast<uint32_t*>(a.aq + r * a.I)[i] = 0u;
            if (lane < NKB2) a.as[r * NKB2 + lane] = 0.0f;
        }
        if (lane < kFdTile) {
            // an inactive route adds +0, which leaves the sum unchanged (it is never -0: it starts at +0)
            part[j][lane] = slot >= 0 ? wgt * val : 0.0f;
            a.c2[r * a.H + n0 + lane] = val;
        }
    }
    __syncthreads();
    if (threadIdx.x < kFdTile) {
        float o = 0.0f;
        for (int j = 0; j < a.topk; j++) o += part[j][threadIdx.x];
        a.out[t * a.H + n0 + threadIdx.x] = f32_to_bf16(o);
    }
}



// ---------------------------------------------------------------------------
// One-launch step.  The grid holds both roles: gate/up tiles of 8*M act columns
// (block ids [0, n_a)) and 8-row down tiles after them.  With tiles that wide
// every block is resident at once on an idle GPU, so the W2 stream of the down
// tiles runs beside the W13 stream instead of after a kernel boundary.
//
// Hand-off.  Each XCD has its own L2, so h must reach the device-coherent
// level without a whole-L2 write-back per tile.  h travels as (value, tag)
// pairs in 64-bit words written with agent-scope atomic stores (coherent
// across XCDs), so a reader sees either the old or the new pair, never half of
// each.  The tag is the call's epoch: every tile keeps a private epoch word in
// the control block that counts the calls since the workspace was initialized
// (each call adds one, whether or not the route is active), so all tiles agree
// on the current call's tag without talking to each other.  After its h, a
// gate/up tile stores the tag into its ready word (in several copies, so that
// each line is polled by a fraction of the readers); it never waits for its
// stores to complete and counts nothing.  A down tile polls the ready words of
// the route's gate/up tiles (one small load per poll) until all but a few are
// set, then reads h with plain loads that the XCD's L2 shares among its down
// tiles, and checks every tag; each element still carrying an old tag (a late
// tile, a ready word seen before its tile's h, a stale line) is re-polled on
// its own with coherent loads until its tag matches, so the last tiles' h comes
// back with the poll that sees it.  Measured on one MI355X (2048/768, 8/8
// active), ready words cut the step from 14.1-15.7 us (a route counter that
// each gate/up tile bumped after waiting for its h stores) to about 13.1-13.5
// us, and not waiting for the last few of them saved about 0.4 us more;
// polling all of h with coherent loads was slower (every poll moved 12.6 MB).
// Down tiles have higher block ids than every gate/up tile they wait for, and
// workgroups are dispatched in block order, so every awaited tile is already
// running or done and the waits always end.  A wait is still bounded; if one
// ever gave up, the error word of the control block is set.

constexpr int kSpinLimit = 1 << 15;    // polls before a wait gives up (tens of milliseconds)
constexpr int kCtlLine = kDecodeCtlLineWords;

// Control block (32-bit words): word 0 is the error word; from word kCtlLine on
// come the epoch word of each gate/up tile, then that of each (token, down tile,
// route) triple; then kDecodeFlagCopies copies of every gate/up tile's ready
// word (its tag once its h is out), and the tagged h at decode_tagged_h_offset.
__device__ __forceinline__ uint32_t* gateup_epoch(const FusedDecodeArgs& a, int b) { return a.ctl + kCtlLine + b; }
__device__ __forceinline__ uint32_t* down_epochs(const FusedDecodeArgs& a, int64_t t, int ntile) {
    return a.ctl + kCtlLine + a.n_a + ((int64_t)t * a.tiles_c + ntile) * a.topk;
}

__device__ __forceinline__ void store_coherent(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_tagged(uint64_t* p, float v, uint32_t tag) {
    __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_coherent(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t load_coherent(const uint32_t* p) {
    return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kLateTiles = 4;   // ready words a down tile may still miss when it starts reading h

// This lane's 2*NKB2 h values of route r (columns kb*128 + 2*lane and +1; each plain load covers 512
// contiguous bytes).  First polls the ready words of the route's gate/up tiles (one 4-byte word per
// tile, one load per poll) until at most kLateTiles of them lack `tag`, then reads h with plain
// loads, which the XCD's L2 shares between the down tiles on it (h is never in an L2 at the start of
// a call: a kernel boundary lies between).  Every element whose tag is still old (its tile was late,
// its ready word became visible before its h, or a stale line was hit) is then re-polled on its own
// with coherent loads until it carries `tag`: the last tiles' h arrives with the poll that sees it,
// without a second round trip after a ready word.  False if the spin limit ran out first.
template <int NKB2>
__device__ __forceinline__ bool wait_route_h(const FusedDecodeArgs& a, int64_t r, uint32_t tag, bool shape_ok,
                                             float (&v)[2 * NKB2]) {
    if (!shape_ok) {                   // the hand-off words belong to another shape: do not wait on them
#pragma unroll
        for (int i = 0; i < 2 * NKB2; i++) v[i] = 0.0f;
        return false;
    }
    // the copy this block polls: a copy's line is polled by 1/kDecodeFlagCopies of the down tiles
    const int copy = (int)(blockIdx.x % kDecodeFlagCopies);
    // lanes past the route's tiles read tile 0's word again: no lane branches around a load
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t* ep = a.flags + ((int64_t)copy * a.T * a.topk + r) * a.flag_stride + (lane < a.tiles_a ? lane : 0);
    int it = 0;
    for (; it < kSpinLimit; it++) {
        if (__popcll(__builtin_amdgcn_ballot_w64(lane < a.tiles_a && load_coherent(ep) != tag)) <= kLateTiles) break;
        __builtin_amdgcn_s_sleep(1);
    }
    if (it >= kSpinLimit) return false;
    asm volatile("" ::: "memory");     // the plain loads below stay after the poll
    const uint64_t* p = a.hx + r * a.I + 2 * lane;
    uint32_t stale = 0;                // bit i: element i still carries an old tag
#pragma unroll
    for (int kb = 0; kb < NKB2; kb++) {
        const uint4 w = *reinterpret_cast<const uint4*>(p + kb * 128);
        if (w.y != tag) stale |= 1u << (2 * kb);
        if (w.w != tag) stale |= 1u << (2 * kb + 1);
        v[2 * kb] = __uint_as_float(w.x);
        v[2 * kb + 1] = __uint_as_float(w.z);
    }
    if (__builtin_amdgcn_ballot_w64(stale != 0) == 0) return true;
    for (; it < kSpinLimit; it++) {
#pragma unroll
        for (int i = 0; i < 2 * NKB2; i++) {
            if (stale & (1u << i)) {
                const uint64_t w = load_coherent(p + (i >> 1) * 128 + (i & 1));
                if ((uint32_t)(w >> 32) == tag) {
                    v[i] = __uint_as_float((uint32_t)w);
                    stale &= ~(1u << i);
                }
            }
        }
        if (__builtin_amdgcn_ballot_w64(stale != 0) == 0) return true;
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}

// Gate/up tile b of the one-launch step: route r, act columns [c0, c0 + 8M).
// Column group g is one MFMA: columns 0..7 are gate rows c0+8g.., columns 8..15
// the matching up rows I+c0+8g..  Each wave owns K blocks [kb0, kb1) of all M
// groups and shares one quantized token-row operand between them.
template <int M>
__device__ __forceinline__ void gateup_tile_m(const FusedDecodeArgs& a, int b) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int64_t r = b / a.tiles_a;
    const int64_t c0 = (int64_t)(b % a.tiles_a) * 8 * M;
    const int64_t N = 2 * (int64_t)a.I;
    uint32_t slot_bits, epoch;
    scalar_read2(a.slots + r, gateup_epoch(a, b), slot_bits, epoch);
    const int slot = (int)slot_bits;
    const uint32_t tag = epoch + 1;
    __shared__ float red[kFdWaves][M][kFdTile];
    __shared__ __attribute__((aligned(16))) uint8_t xq[kFdWaves][kFdUnroll][128];
    const int col = lane & 15;
    if (slot < 0) {
        if (threadIdx.x < kFdTile * M) {
            const int g = threadIdx.x / kFdTile, c = threadIdx.x % kFdTile;
            const int64_t rr = c < 8 ? c0 + 8 * g + c : a.I + c0 + 8 * g + (c - 8);
            a.c1[r * N + rr] = 0.0f;
            if (c < 8) a.h[r * a.I + c0 + 8 * g + c] = 0.0f;
        }
        if (threadIdx.x == 0) store_coherent(gateup_epoch(a, b), tag);
        return;
    }
    const int nkb = a.H / 128;
    const int kb0 = wave * nkb / kFdWaves, kb1 = (wave + 1) * nkb / kFdWaves;
    const int q16 = (lane / 16) * 16;
    const uint8_t* wrow[M];
    const float* wsrow[M];
#pragma unroll
    for (int g = 0; g < M; g++) {
        const int64_t wr = col < 8 ? c0 + 8 * g + col : a.I + c0 + 8 * g + (col - 8);
        wrow[g] = a.w13 + (int64_t)slot * N * a.H + wr * a.H + q16;
        wsrow[g] = a.w13s + (int64_t)slot * (N / 128) * nkb + (wr / 128) * nkb;
    }
    const uint16_t* xrow = a.x + (r / a.topk) * a.H;
    v4f acc[M];
#pragma unroll
    for (int g = 0; g < M; g++) acc[g] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    for (int kb = kb0; kb < kb1; kb += kFdUnroll) {
        v4i blo[M][kFdUnroll], bhi[M][kFdUnroll];
        float sa[kFdUnroll], sw[M][kFdUnroll];
        uint32_t pair[kFdUnroll];
        // token row first: its quantization then overlaps the weight stream (loads retire in order)
#pragma unroll
        for (int u = 0; u < kFdUnroll; u++)
            if (kb + u < kb1) pair[u] = reinterpret_cast<const uint32_t*>(xrow + (int64_t)(kb + u) * 128)[lane];
#pragma unroll
        for (int g = 0; g < M; g++)
#pragma unroll
            for (int u = 0; u < kFdUnroll; u++) {
                if (kb + u < kb1) {
                    const uint8_t* wp = wrow[g] + (int64_t)(kb + u) * 128;
                    blo[g][u] = *reinterpret_cast<const v4i*>(wp);
                    bhi[g][u] = *reinterpret_cast<const v4i*>(wp + 64);
                    sw[g][u] = wsrow[g][kb + u];
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
        // one K block at a time: its token-row fragment from LDS, then its M products
#pragma unroll
        for (int u = 0; u < kFdUnroll; u++) {
            if (kb + u < kb1) {
                const v4i alo = *reinterpret_cast<const v4i*>(&xq[wave][u][q16]);
                const v4i ahi = *reinterpret_cast<const v4i*>(&xq[wave][u][64 + q16]);
#pragma unroll
                for (int g = 0; g < M; g++) {
                    const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
                    const v4f p = mfma16x16x128_e4m3(frag(alo, ahi), frag(blo[g][u], bhi[g][u]), z);
                    acc[g] += p * (sa[u] * sw[g][u]);
                }
            }
        }
        wave_lds_fence();
    }
#pragma unroll
    for (int g = 0; g < M; g++)
        if (lane < kFdTile) red[wave][g][lane] = acc[g][0];
    __syncthreads();
    if (threadIdx.x < kFdTile * M) {
        const int g = threadIdx.x / kFdTile, c = threadIdx.x % kFdTile;
        float t = red[0][g][c];
#pragma unroll
        for (int w = 1; w < kFdWaves; w++) t += red[w][g][c];
        const float up = __shfl_down(t, 8, kFdTile);            // lanes c < 8 get their up value
        const int64_t hc = r * a.I + c0 + 8 * g + c;
        const float hv = gated_act(a.act, t, up);
        if (c < 8) store_tagged(&a.hx[hc], hv, tag);           // the hand-off: first out
        // then the tile's ready-word copies, which readers poll before they load h (a hint: h's own
        // tags decide, so a copy may become visible before the h stores), and its epoch word
        if (threadIdx.x < kDecodeFlagCopies)
            store_coherent(a.flags + ((int64_t)threadIdx.x * a.T * a.topk + r) * a.flag_stride + b % a.tiles_a, tag);
        if (threadIdx.x == 0) store_coherent(gateup_epoch(a, b), tag);
        if (c < 8) a.h[hc] = hv;
        const int64_t rr = c < 8 ? c0 + 8 * g + c : a.I + c0 + 8 * g + (c - 8);
        a.c1[r * N + rr] = t;
    }
}

// h of route r in a down tile's wave, requantized per 1x128 group: waits for the
// call's h (wait_route_h), transposes it through the wave's LDS rows so that
// lane l owns columns 16*(l%8) .. +15 of 128-group l/8 (lanes past the last group
// repeat it and store nothing), and writes the codes as MFMA operands into hq.
// A group's maximum is then an in-lane maximum and three DPP steps.
template <int NKB2>
struct RouteAct {
    float sa[NKB2];     // scale of each group (wave-uniform)
    uint32_t q[4];      // this lane's 16 codes
    float s;            // this lane's group scale
    int rg, rc;         // this lane's group and first column in it
    bool owner;         // whether this lane's codes are its own (stored)
};

template <int NKB2>
__device__ __forceinline__ bool route_act(const FusedDecodeArgs& a, int64_t r, uint32_t tag, bool shape_ok,
                                          float* hfw, uint8_t (*hqw)[128], RouteAct<NKB2>& ra) {
    const int lane = threadIdx.x & (kWave - 1);
    float hp[2 * NKB2];
    const bool ok = wait_route_h<NKB2>(a, r, tag, shape_ok, hp);
#pragma unroll
    for (int kb = 0; kb < NKB2; kb++)
        *reinterpret_cast<float2*>(&hfw[kb * 128 + 2 * lane]) = make_float2(hp[2 * kb], hp[2 * kb + 1]);
    wave_lds_fence();
    ra.owner = (lane >> 3) < NKB2;
    ra.rg = ra.owner ? (lane >> 3) : NKB2 - 1;
    ra.rc = (lane & 7) * 16;
    float hv[16];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float4 f = *reinterpret_cast<const float4*>(&hfw[ra.rg * 128 + ra.rc + 4 * i]);
        hv[4 * i] = f.x; hv[4 * i + 1] = f.y; hv[4 * i + 2] = f.z; hv[4 * i + 3] = f.w;
    }
    float m16 = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) m16 = __builtin_fmaxf(m16, __builtin_fabsf(hv[i]));
    const float amax = group8_max(m16);
    if (amax >= 0x1p-100f) {
        ra.s = amax / 448.0f;
        // |v| * inv stays below 448 * (1 + 2^-21), which the conversion rounds to 448 as a clamp
        // to +-448 would, so the products go to it unclamped
        const float inv = 448.0f * __builtin_amdgcn_rcpf(amax);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(hv[4 * i] * inv, hv[4 * i + 1] * inv, 0, false);
            ra.q[i] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(hv[4 * i + 2] * inv, hv[4 * i + 3] * inv, lo, true);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            float s2;
            const uint32_t lo = requant_pair(hv[4 * i], hv[4 * i + 1], amax, s2);
            const uint32_t hi = requant_pair(hv[4 * i + 2], hv[4 * i + 3], amax, ra.s);
            ra.q[i] = lo | (hi << 16);
        }
    }
    if (ra.owner) *reinterpret_cast<uint4*>(&hqw[ra.rg][ra.rc]) = make_uint4(ra.q[0], ra.q[1], ra.q[2], ra.q[3]);
#pragma unroll
    for (int kb = 0; kb < NKB2; kb++)
        ra.sa[kb] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ra.s), 8 * kb));
    wave_lds_fence();
    return ok;
}

// Down tile b of the one-launch step: token t, 8 rows of W2 for all of t's
// routes, wave j owning route j (then j+8, ...).  As decode_down8_kernel (the
// 16 MFMA columns are the 8 rows on two K streams), but the W2 fragments are
// requested before the route's h is ready.
template <int NKB2>
__device__ __forceinline__ void down8_tile(const FusedDecodeArgs& a, int b) {
    constexpr int NS = (NKB2 + 1) / 2;                         // W2 blocks per lane
    constexpr bool kOdd = (NKB2 & 1) != 0;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int64_t t = b / a.tiles_c;
    const int ntile = b % a.tiles_c;
    const int64_t n0 = (int64_t)ntile * kDnRows;
    const int col = lane & 15, q16 = (lane / 16) * 16;
    const int strm = col >> 3;
    uint32_t* epochs = down_epochs(a, t, ntile);
    __shared__ float part[64][kDnRows];
    __shared__ __attribute__((aligned(16))) uint8_t hq[kFdWaves][NKB2][128];
    __shared__ __attribute__((aligned(16))) float hf[kFdWaves][NKB2 * 128];
    bool timed_out = false, shape_ok = true;
    for (int j = wave_uniform(wave); j < a.topk; j += kFdWaves) {
        const int64_t r = t * a.topk + j;
        // through the scalar cache: a vector load here would return only after this CU's share of
        // the W13 stream, and the W2 stream could not start before it.  Word 1 of the control block
        // is the shape the workspace was initialized for.
        uint32_t slot_bits, epoch, sig;
        scalar_read3(a.slots + r, epochs + j, a.ctl + 1, slot_bits, epoch, sig);
        shape_ok = sig == a.sig;
        const int slot = (int)slot_bits;
        const uint32_t tag = epoch + 1;
        float val = 0.0f, wgt = 0.0f;
        if (slot >= 0) {
            // the W2 fragments go out first, behind nothing but the slot id
            const uint8_t* wrow = a.w2 + (int64_t)slot * a.H * a.I + (n0 + (col & 7)) * a.I + q16;
            v4i blo[NS], bhi[NS];
#pragma unroll
            for (int i = 0; i < NS; i++) {
                // odd NKB2: stream 1's missing last block reads a valid one, zeroed below
                const int kb = strm * NS + i < NKB2 ? strm * NS + i : NKB2 - 1;
                blo[i] = *reinterpret_cast<const v4i*>(wrow + kb * 128);
                bhi[i] = *reinterpret_cast<const v4i*>(wrow + kb * 128 + 64);
            }
            wgt = a.weights[r];
            // the tile's W2 block scales travel with its fragments
            const float* wsrow = a.w2s + (int64_t)slot * (a.H / 128) * NKB2 + (n0 / 128) * NKB2;
            float sw[NKB2];
#pragma unroll
            for (int kb = 0; kb < NKB2; kb++) sw[kb] = wsrow[kb];
            RouteAct<NKB2> ra;
            if (!route_act<NKB2>(a, r, tag, shape_ok, hf[wave], hq[wave], ra)) timed_out = true;
            // A row 0 carries stream 0's block, A row 1 stream 1's; C[0][c < 8] and C[1][c >= 8] are
            // the two streams' partials of W2 row n0 + (c & 7)
            const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
            const int m = lane & 15;
            const v4i zero4 = {0, 0, 0, 0};
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < NS; i++) {
                const bool has1 = !(kOdd && i == NS - 1);
                const int kbA = (m == 1 && has1) ? NS + i : i;
                v4i alo = *reinterpret_cast<const v4i*>(&hq[wave][kbA][q16]);
                v4i ahi = *reinterpret_cast<const v4i*>(&hq[wave][kbA][64 + q16]);
                const bool a_on = m == 0 || (m == 1 && has1);
                alo = a_on ? alo : zero4;
                ahi = a_on ? ahi : zero4;
                const bool b_on = strm == 0 || has1;
                const v4i bl = b_on ? blo[i] : zero4, bh = b_on ? bhi[i] : zero4;
                const v4f p = mfma16x16x128_e4m3(frag(alo, ahi), frag(bl, bh), z);
                const float f0 = ra.sa[i] * sw[i];
                const float f1 = has1 ? ra.sa[(NS + i) % NKB2] * sw[(NS + i) % NKB2] : 0.0f;
                acc += strm == 0 ? p[0] * f0 : p[1] * f1;
            }
            wave_lds_fence();
            val = acc + __shfl_down(acc, 8, 16);
            if (ntile == 0 && ra.owner) {
                *reinterpret_cast<uint4*>(a.aq + r * a.I + ra.rg * 128 + ra.rc) = make_uint4(ra.q[0], ra.q[1], ra.q[2], ra.q[3]);
                if ((lane & 7) == 0) a.as[r * NKB2 + ra.rg] = ra.s;
            }
        } else if (ntile == 0) {
            for (int i = lane; i < a.I / 4; i += kWave) reinterpret_cast<uint32_t*>(a.aq + r * a.I)[i] = 0u;
            if (lane < NKB2) a.as[r * NKB2 + lane] = 0.0f;
        }
        if (lane < kDnRows) {
            // an inactive route adds +0, which leaves the sum unchanged (it is never -0: it starts at +0)
            part[j][lane] = slot >= 0 ? wgt * val : 0.0f;
            a.c2[r * a.H + n0 + lane] = val;
        }
        if (lane == 0) store_coherent(epochs + j, tag);
    }
    __shared__ int failed;
    if (threadIdx.x == 0) failed = 0;
    __syncthreads();
    if ((timed_out || !shape_ok) && lane == 0) {
        store_coherent(a.ctl, shape_ok ? kDecodeErrWait : kDecodeErrShape);
        failed = 1;
    }
    __syncthreads();
    if (threadIdx.x < kDnRows) {
        float o = 0.0f;
        for (int j = 0; j < a.topk; j++) o += part[j][threadIdx.x];
        // rows whose inputs never arrived are NaN, so a failed step is visible in its output too
        a.out[t * a.H + n0 + threadIdx.x] = failed ? (uint16_t)0x7FC0u : f32_to_bf16(o);
    }
}

template <int NKB2, int M>
__global__ void __launch_bounds__(kWave * kFdWaves) decode_step_kernel(FusedDecodeArgs a) {
    if ((int)blockIdx.x < a.n_a) gateup_tile_m<M>(a, (int)blockIdx.x);
    else down8_tile<NKB2>(a, (int)blockIdx.x - a.n_a);
}

// Workgroups of decode_step_kernel<NKB2, M> that fit on the current device at once (0 if unknown).
// The value is cached per device; concurrent first calls may both compute it, and store the same value.
template <int NKB2, int M>
int step_resident_blocks() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int c = cached[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_step_kernel<NKB2, M>, kWave * kFdWaves, 0) !=
                hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        c = per_cu * cus > 0 ? per_cu * cus : -1;
        cached[dev].store(c, std::memory_order_relaxed);
    }
    return c > 0 ? c : 0;
}

// Launches the one-launch step if its blocks all fit on the device at once; returns 1 if it did not
// launch (the caller then runs the two-launch step), else a status.
template <int NKB2, int M>
int try_step(hipStream_t st, FusedDecodeArgs a) {
    a.tiles_a = a.I / (8 * M);
    a.n_a = a.T * a.topk * a.tiles_a;
    a.tiles_c = a.H / kDnRows;
    a.hx = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(a.ctl) + decode_tagged_h_offset(a.T, a.H, a.I, a.topk));
    a.flags = a.ctl + decode_flag_offset(a.T, a.H, a.I, a.topk);
    a.flag_stride = (int)decode_flag_stride(a.I);
    a.sig = decode_ctl_signature(a.T, a.H, a.I, a.topk);
    const int64_t blocks = (int64_t)a.n_a + (int64_t)a.T * a.tiles_c;
    if (blocks > step_resident_blocks<NKB2, M>()) return 1;
    hipLaunchKernelGGL((decode_step_kernel<NKB2, M>), dim3((unsigned)blocks), dim3(kWave * kFdWaves), 0, st, a);
    return launch_status();
}

template <int NKB2>
int try_step_m(hipStream_t st, const FusedDecodeArgs& a) {
    // the tile width the control block was sized for
    if (decode_step_m(a.I) == 3) return try_step<NKB2, 3>(st, a);
    if ((a.I / 8) % 2 == 0) return try_step<NKB2, 2>(st, a);
    return 1;
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

int fused_decode_one_launch(hipStream_t st, FusedDecodeArgs a) {
    if (!a.ctl || !decode_one_launch_ok(a.T, a.H, a.I, a.topk)) return 1;
    switch (a.I / 128) {
        case 1: return try_step_m<1>(st, a);
        case 2: return try_step_m<2>(st, a);
        case 3: return try_step_m<3>(st, a);
        case 4: return try_step_m<4>(st, a);
        case 5: return try_step_m<5>(st, a);
        case 6: return try_step_m<6>(st, a);
        case 7: return try_step_m<7>(st, a);
        case 8: return try_step_m<8>(st, a);
        default: return 1;
    }
}

}  // namespace moe
