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
    uint32_t* ctl;           // control block of the one-launch step (decode_ctl_bytes)
    int T, H, I, topk;
    int act;                 // gated activation (moe_act 1..5)
    int tiles_a;             // gate/up tiles per route (set by the launcher)
    int tiles_c;             // down tiles per token (set by the launcher)
    int n_a;                 // gate/up tiles in total (set by the launcher)
};

// Enqueues the two decode launches on `st`.  Requires I/128 in [1, 8].
int fused_decode_two_launch(hipStream_t st, FusedDecodeArgs a);

// Words per line of the control block: each counter sits on its own 128-byte line.
constexpr int kDecodeCtlLineWords = 32;

// W2 rows per down tile of the one-launch step.
constexpr int kDecodeDownRows = 8;

// Largest number of last-seen words (routes x down tiles) the one-launch step keeps.
constexpr int64_t kDecodeMaxLastSeen = 1 << 18;

// Shapes the one-launch step can take: I/128 in [1, 8], I/8 even or a multiple of 3, H/128 <= 16
// (one 2-block K step per wave) and a bounded control block.  Whether a call takes it also depends on
// the device: every block must fit at once.
inline bool decode_one_launch_ok(int64_t T, int64_t H, int64_t I, int64_t topk) {
    return I / 128 >= 1 && I / 128 <= 8 && ((I / 8) % 2 == 0 || (I / 8) % 3 == 0) && H / 128 <= 16 &&
           H % kDecodeDownRows == 0 && T * topk * (H / kDecodeDownRows) <= kDecodeMaxLastSeen;
}

// Bytes of the control block: the error word's line, a counter line and a publish line per route,
// and one last-seen word per (route, down tile) for shapes the one-launch step can take.
inline int64_t decode_ctl_bytes(int64_t T, int64_t H, int64_t I, int64_t topk) {
    const int64_t R = T * topk;
    const int64_t seen = decode_one_launch_ok(T, H, I, topk) ? R * (H / kDecodeDownRows) : 0;
    return 4 * (kDecodeCtlLineWords * (1 + 2 * R) + seen);
}

// Enqueues the decode step as one launch when the shape allows it and all its blocks fit on the
// device at once; returns 1 without launching otherwise, else a status.
int fused_decode_one_launch(hipStream_t st, FusedDecodeArgs a);

}  // namespace moe
