// Arguments of the two decode launches, shared by the host entry point and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct FusedDecodeArgs {
    const uint16_t* x;       // [T][H] bf16 token rows
    const int32_t* slots;    // [T][topk], < 0 = inactive route
    const float* weights;    // [T][topk] routing weights
    const uint8_t* w13;      // [S][2I][H] fp8
    const float* w13s;       // [S][2I/128][H/128]
    const uint8_t* w2;       // [S][H][I] fp8
    const float* w2s;        // [S][H/128][I/128]
    float* c1;               // [R][2I] gate/up output
    float* h;                // [R][I] SiLU(gate)*up
    uint8_t* aq;             // [R][I] fp8 activation
    float* as;               // [R][I/128]
    float* c2;               // [R][H] down output
    uint16_t* out;           // [T][H] bf16
    int T, H, I, topk;
    int tiles_a;             // gate/up tiles per route (set by the launcher)
    int tiles_c;             // down tiles per token (set by the launcher)
    int n_a;                 // gate/up tiles in total (set by the launcher)
};

// Enqueues the two decode launches on `st`.  Requires I/128 in [1, 8].
int fused_decode_two_launch(hipStream_t st, FusedDecodeArgs a);

}  // namespace moe
