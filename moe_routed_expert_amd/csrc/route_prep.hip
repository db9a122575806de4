// Routing prep of a prefill step: top-k experts and renormalized weights per
// token, then the (expert, token)-ordered route maps the gather and the grouped
// GEMM consume ("[MoE] Gather the cutlass MoE activation and its scales in one
// launch", Motivation: the activation is replicated once per routed expert
// through a dst2src map of m * topk entries; "perf(dsfp4): pick the
// grouped-prefill tile from route density on sm_89", Measurements: the
// grouped GEMM works on the routes of each expert).
//
// MI355X design: three small launches, deterministic without floating-point
// atomics.
//  * topk + count (one 256-thread workgroup per chunk of 16 tokens): a token
//    owns one 16-lane DPP row and each lane holds E/16 of its logits as
//    ordered 64-bit keys (monotone float bits, then the inverted expert index),
//    so "larger logit, ties to the lower index" is one unsigned compare and the
//    keys are distinct.  Round j takes the row's largest key below round j-1's
//    winner; the row maximum is four DPP moves (quad permutes, half-mirror,
//    mirror).  The weights exp(l_j - l_max) / sum_i exp(l_i - l_max) are the
//    softmax over all experts renormalized over the top-k (its denominator
//    cancels).  The chunk sets one bit per (expert, token) in LDS and writes
//    each expert's count, chunk-major.
//  * scan (one workgroup): threads own 4 experts by a group of chunks; one batch
//    of 16-byte loads gives group sums, LDS prefix sums over groups and a
//    workgroup scan over experts give the expert offsets and, per (group,
//    expert), the first row of that expert in that group.
//  * scatter (one workgroup per chunk): its expert bases are the group's first
//    rows plus the counts of the earlier chunks of its group (loads issued
//    beside the expert-id loads); it rebuilds the bit sets, and a route's row is
//    its expert's base plus the number of lower tokens of the chunk with that
//    expert (popcount), so rows follow (expert, token) order.
#include <hip/hip_runtime.h>

#include "device.h"
#include "host.h"

namespace moe {
namespace {

constexpr int kRpChunk = 16;                  // tokens per chunk: one bit-set word per expert
constexpr int kRpRow = 16;                    // lanes per token (one DPP row)
constexpr int kRpThreads = kRpChunk * kRpRow; // one pass over the chunk
constexpr int kRpMaxE = 1024;
constexpr int kRpMaxTopk = 64;
constexpr int kRpScanThreads = 1024;
constexpr int kRpMaxGroups = 64;              // chunk groups of the scan

// Chunk counts and bases are [chunk][experts rounded up to 4] int32.
__host__ __device__ inline int64_t rp_row_words(int64_t E) { return (E + 3) / 4 * 4; }

// Order-preserving map of a float to uint32 (-0 as +0, NaN as -inf), larger float -> larger code.
__device__ __forceinline__ uint32_t rp_mono(float v) {
    uint32_t u = __float_as_uint(v);
    if (v != v) u = 0xFF800000u;
    if (u == 0x80000000u) u = 0u;
    return (u >> 31) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float rp_unmono(uint32_t m) {
    return __uint_as_float((m >> 31) ? (m & 0x7FFFFFFFu) : ~m);
}

template <int CTRL>
__device__ __forceinline__ uint32_t rp_dpp(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

// DPP controls: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.  After the four
// steps every lane of a 16-lane row holds the row's combined value.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint64_t rp_max_step(uint64_t k) {
    const uint64_t o = ((uint64_t)rp_dpp<CTRL>((uint32_t)(k >> 32)) << 32) | rp_dpp<CTRL>((uint32_t)k);
    return o > k ? o : k;
}

__device__ __forceinline__ uint64_t rp_row_max(uint64_t k) {
    k = rp_max_step<kDppXor1>(k);
    k = rp_max_step<kDppXor2>(k);
    k = rp_max_step<kDppHalfMirror>(k);
    return rp_max_step<kDppMirror>(k);
}

template <int CTRL>
__device__ __forceinline__ float rp_sum_step(float x) {
    return x + __uint_as_float(rp_dpp<CTRL>(__float_as_uint(x)));
}

__device__ __forceinline__ float rp_row_sum(float x) {
    x = rp_sum_step<kDppXor1>(x);
    x = rp_sum_step<kDppXor2>(x);
    x = rp_sum_step<kDppHalfMirror>(x);
    return rp_sum_step<kDppMirror>(x);
}

__device__ void rp_build_masks(const int32_t* ids_lds, int n_tok, int topk, uint32_t* mask) {
    for (int i = threadIdx.x; i < n_tok * topk; i += blockDim.x) atomicOr(&mask[ids_lds[i]], 1u << (i / topk));
}

// VPL: logits per lane, E <= 16 * VPL.
template <int VPL>
__global__ void __launch_bounds__(kRpThreads)
route_topk_count_kernel(const float* __restrict__ logits, int64_t logits_stride, int T, int E, int topk,
                        int32_t* __restrict__ expert_ids, float* __restrict__ weights, int32_t* __restrict__ counts) {
    __shared__ int32_t ids_lds[kRpChunk * kRpMaxTopk];
    __shared__ float val_lds[kRpChunk * kRpMaxTopk];
    __shared__ uint32_t mask[kRpMaxE];
    const int l16 = threadIdx.x % kRpRow;
    const int tt = threadIdx.x / kRpRow;          // token of this row within the chunk
    const int c = blockIdx.x;
    const int t0 = c * kRpChunk;
    const int n_tok = T - t0 < kRpChunk ? T - t0 : kRpChunk;
    for (int i = threadIdx.x; i < E; i += kRpThreads) mask[i] = 0u;
    if (tt < n_tok) {                             // whole rows are active or idle together
        const int t = t0 + tt;
        const float* row = logits + (int64_t)t * logits_stride;
        float v[VPL];
#pragma unroll
        for (int i = 0; i < VPL; i++) {
            const int e = i * kRpRow + l16;
            v[i] = row[e < E ? e : E - 1];        // in bounds for every lane; keys below drop e >= E
        }
        uint64_t key[VPL];
#pragma unroll
        for (int i = 0; i < VPL; i++) {
            const int e = i * kRpRow + l16;
            key[i] = e < E ? ((uint64_t)rp_mono(v[i]) << 32) | (uint32_t)~e : 0ull;   // real keys are > 0
        }
        uint64_t prev = ~0ull;
        for (int j = 0; j < topk; j++) {
            uint64_t f[VPL];                      // candidates of this round, then a depth-log2(VPL) max tree
#pragma unroll
            for (int i = 0; i < VPL; i++) f[i] = key[i] < prev ? key[i] : 0ull;
#pragma unroll
            for (int w = VPL / 2; w >= 1; w /= 2)
#pragma unroll
                for (int i = 0; i < w; i++) f[i] = f[i] > f[i + w] ? f[i] : f[i + w];
            const uint64_t best = rp_row_max(f[0]);
            prev = best;
            if (l16 == 0) {
                ids_lds[tt * topk + j] = (int)~(uint32_t)best;
                val_lds[tt * topk + j] = rp_unmono((uint32_t)(best >> 32));
            }
        }
        // weights: lane l16 handles routes l16, l16 + 16, ...  (the row's LDS writes come from this
        // wave, and LDS serves a wave's accesses in order)
        const float lm = val_lds[tt * topk];
        float part = 0.0f;
        for (int j = l16; j < topk; j += kRpRow) part += expf(val_lds[tt * topk + j] - lm);
        const float sum = rp_row_sum(part);
        for (int j = l16; j < topk; j += kRpRow) {
            expert_ids[(int64_t)t * topk + j] = ids_lds[tt * topk + j];
            weights[(int64_t)t * topk + j] = expf(val_lds[tt * topk + j] - lm) / sum;
        }
    }
    __syncthreads();
    rp_build_masks(ids_lds, n_tok, topk, mask);
    __syncthreads();
    const int64_t rw = rp_row_words(E);
    for (int e = threadIdx.x; e < rw; e += kRpThreads) counts[(int64_t)c * rw + e] = e < E ? __popc(mask[e]) : 0;
}

// Chunk groups of the scan: thread (q, g) owns experts 4q..4q+3 over chunks [g * per, (g + 1) * per).
struct RpGroups {
    int Q, G, per;
};

__host__ __device__ inline RpGroups rp_groups(int nc, int E) {
    RpGroups r;
    r.Q = (int)rp_row_words(E) / 4;
    r.G = kRpScanThreads / r.Q;
    if (r.G > kRpMaxGroups) r.G = kRpMaxGroups;
    r.per = (nc + r.G - 1) / r.G;
    return r;
}

// Expert offsets (offsets[e] = routes of experts below e) and, per (group, expert), the expert's first row
// in the group: first[g][e] = offsets[e] + sum over the chunks of earlier groups of counts[c][e].
__global__ void __launch_bounds__(kRpScanThreads)
route_scan_kernel(const int32_t* __restrict__ counts, int nc, int E, int32_t* __restrict__ first,
                  int32_t* __restrict__ expert_offsets) {
    __shared__ __align__(16) int gsum[kRpScanThreads * 4];   // [group][expert], groups * rw <= 4096
    __shared__ int total[kRpMaxE];
    __shared__ int wsum[kRpScanThreads / kWave];
    const int rw = (int)rp_row_words(E);
    const RpGroups gr = rp_groups(nc, E);
    const int q = threadIdx.x % gr.Q, g = threadIdx.x / gr.Q;
    const bool owner = g < gr.G;
    const int r0 = owner ? g * gr.per : 0;
    const int r1 = owner ? (r0 + gr.per < nc ? r0 + gr.per : nc) : 0;
    int4 s = make_int4(0, 0, 0, 0);
#pragma unroll 16
    for (int r = r0; r < r1; r++) {
        const int4 x = reinterpret_cast<const int4*>(counts + (int64_t)r * rw)[q];
        s.x += x.x;
        s.y += x.y;
        s.z += x.z;
        s.w += x.w;
    }
    if (owner) reinterpret_cast<int4*>(gsum + g * rw)[q] = s;
    __syncthreads();
    // exclusive prefix over groups, per expert; totals
    for (int e = threadIdx.x; e < rw; e += kRpScanThreads) {
        int run = 0;
        for (int gg = 0; gg < gr.G; gg++) {
            const int x = gsum[gg * rw + e];
            gsum[gg * rw + e] = run;
            run += x;
        }
        total[e] = run;
    }
    __syncthreads();
    // workgroup exclusive scan of the expert totals (one expert per thread, E <= 1024)
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int mine = threadIdx.x < E ? total[threadIdx.x] : 0;
    int x = mine;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(x, d, kWave);
        if (lane >= d) x += y;
    }
    if (lane == kWave - 1) wsum[wave] = x;
    __syncthreads();
    int off = x - mine;
    for (int w = 0; w < wave; w++) off += wsum[w];
    __syncthreads();                              // every thread has read total[] before it is overwritten
    if (threadIdx.x < rw) total[threadIdx.x] = threadIdx.x < E ? off : 0;
    if (threadIdx.x < E) {
        expert_offsets[threadIdx.x] = off;
        if (threadIdx.x == E - 1) expert_offsets[E] = off + mine;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < gr.G * rw; i += kRpScanThreads) first[i] = total[i % rw] + gsum[i];
}

__global__ void __launch_bounds__(kRpThreads)
route_scatter_kernel(const int32_t* __restrict__ expert_ids, const int32_t* __restrict__ counts,
                     const int32_t* __restrict__ first, int T, int E, int topk, int nc,
                     int32_t* __restrict__ dst2src, int32_t* __restrict__ route_rows) {
    constexpr int kIdsPerThread = kRpChunk * kRpMaxTopk / kRpThreads;
    __shared__ int32_t ids_lds[kRpChunk * kRpMaxTopk];
    __shared__ uint32_t mask[kRpMaxE];
    __shared__ int32_t base[kRpMaxE];
    const int c = blockIdx.x;
    const int t0 = c * kRpChunk;
    const int n_tok = T - t0 < kRpChunk ? T - t0 : kRpChunk;
    const int n = n_tok * topk;
    const int64_t rw = rp_row_words(E);
    const RpGroups gr = rp_groups(nc, E);
    const int g = c / gr.per;
    int idv[kIdsPerThread];
#pragma unroll
    for (int k = 0; k < kIdsPerThread; k++) {
        const int i = threadIdx.x + k * kRpThreads;
        idv[k] = i < n ? expert_ids[(int64_t)t0 * topk + i] : 0;
    }
    for (int e = threadIdx.x; e < E; e += kRpThreads) {
        int b = first[(int64_t)g * rw + e];
#pragma unroll 8
        for (int cc = g * gr.per; cc < c; cc++) b += counts[(int64_t)cc * rw + e];
        base[e] = b;
        mask[e] = 0u;
    }
#pragma unroll
    for (int k = 0; k < kIdsPerThread; k++) {
        const int i = threadIdx.x + k * kRpThreads;
        if (i < n) ids_lds[i] = idv[k];
    }
    __syncthreads();
    rp_build_masks(ids_lds, n_tok, topk, mask);
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kRpThreads) {
        const int tt = i / topk;
        const int e = ids_lds[i];
        const int row = base[e] + __popc(mask[e] & ((1u << tt) - 1u));
        dst2src[row] = t0 + tt;
        route_rows[(int64_t)t0 * topk + i] = row;
    }
}

// T == 0: every expert offset is zero.
__global__ void route_zero_offsets_kernel(int E, int32_t* __restrict__ expert_offsets) {
    for (int e = threadIdx.x; e <= E; e += blockDim.x) expert_offsets[e] = 0;
}

int64_t rp_chunks(int64_t T) { return (T + kRpChunk - 1) / kRpChunk; }

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_route_prep_workspace_size(int64_t T, int64_t E) {
    if (T < 0 || E < 1 || E > kRpMaxE) return 0;
    const int64_t words = (rp_chunks(T) + kRpMaxGroups) * rp_row_words(E);   // counts, then first rows
    return (size_t)((words * 4 + 255) / 256 * 256) + 256;
}

extern "C" int moe_route_prep(const float* logits, int64_t logits_stride, int64_t T, int64_t E, int64_t topk,
                              int32_t* expert_ids, float* weights, int32_t* dst2src, int32_t* route_rows,
                              int32_t* expert_offsets, void* workspace, size_t ws_bytes, void* stream) {
    if (T < 0 || E < 1 || E > kRpMaxE || topk < 1 || topk > E || topk > kRpMaxTopk) return MOE_ERR_SHAPE;
    if (T * topk > 0x7FFFFFFF || T > 0x7FFFFFFF) return MOE_ERR_SHAPE;
    if (!expert_offsets || !workspace) return MOE_ERR_NULL;
    if (T > 0 && (!logits || !expert_ids || !weights || !dst2src || !route_rows)) return MOE_ERR_NULL;
    if (T > 0 && logits_stride < E) return MOE_ERR_SHAPE;
    if (ws_bytes < moe_route_prep_workspace_size(T, E)) return MOE_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MOE_ERR_ALIGN;
    auto st = as_stream(stream);
    if (T == 0) {
        hipLaunchKernelGGL(route_zero_offsets_kernel, dim3(1), dim3(1024), 0, st, (int)E, expert_offsets);
        return launch_status();
    }
    const int64_t nc = rp_chunks(T);
    int32_t* counts = (int32_t*)workspace;
    int32_t* first = counts + nc * rp_row_words(E);
    const dim3 grid((unsigned)nc), block(kRpThreads);
    if (E <= 4 * kRpRow)
        hipLaunchKernelGGL(route_topk_count_kernel<4>, grid, block, 0, st, logits, logits_stride, (int)T, (int)E,
                           (int)topk, expert_ids, weights, counts);
    else if (E <= 16 * kRpRow)
        hipLaunchKernelGGL(route_topk_count_kernel<16>, grid, block, 0, st, logits, logits_stride, (int)T, (int)E,
                           (int)topk, expert_ids, weights, counts);
    else
        hipLaunchKernelGGL(route_topk_count_kernel<64>, grid, block, 0, st, logits, logits_stride, (int)T, (int)E,
                           (int)topk, expert_ids, weights, counts);
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kRpScanThreads), 0, st, counts, (int)nc, (int)E, first,
                       expert_offsets);
    hipLaunchKernelGGL(route_scatter_kernel, grid, block, 0, st, expert_ids, counts, first, (int)T, (int)E,
                       (int)topk, (int)nc, dst2src, route_rows);
    return launch_status();
}
