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
    uint64_t* hx;            // [R][I] tagged h of the one-launch step (set by the launcher)
    uint32_t* flags;         // ready-word copies of the one-launch step (set by the launcher)
    int flag_stride;         // words per route in one copy (set by the launcher)
    int T, H, I, topk;
    int act;                 // gated activation (moe_act 1..5)
    uint32_t sig;            // decode_ctl_signature of (T, H, I, topk) (set by the launcher)
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

// Largest number of down-tile epoch words (routes x down tiles) the one-launch step keeps.
constexpr int64_t kDecodeMaxLastSeen = 1 << 18;

// Shapes the one-launch step can take: I/128 in [1, 8], I/8 even or a multiple of 3, H/128 <= 16
// (one 2-block K step per wave) and a bounded control block.  Whether a call takes it also depends on
// the device: every block must fit at once.
inline bool decode_one_launch_ok(int64_t T, int64_t H, int64_t I, int64_t topk) {
    return I / 128 >= 1 && I / 128 <= 8 && ((I / 8) % 2 == 0 || (I / 8) % 3 == 0) && H / 128 <= 16 &&
           H % kDecodeDownRows == 0 && T * topk * (H / kDecodeDownRows) <= kDecodeMaxLastSeen;
}

// Act columns per gate/up tile of the one-launch step are 8 * decode_step_m(I).
inline int decode_step_m(int64_t I) { return (I / 8) % 3 == 0 ? 3 : 2; }

// Epoch words of the one-launch step: one per gate/up tile and one per (token, down tile, route).
inline int64_t decode_epoch_words(int64_t T, int64_t H, int64_t I, int64_t topk) {
    return T * topk * (I / (8 * decode_step_m(I))) + T * (H / kDecodeDownRows) * topk;
}

// Copies of each gate/up tile's ready word (readers spread their polls over them) and words per
// route in one copy (the route's gate/up tiles, padded to whole 128-byte lines).
constexpr int kDecodeFlagCopies = 8;
inline int64_t decode_flag_stride(int64_t I) {
    const int64_t tiles = I / (8 * decode_step_m(I));
    return (tiles + kDecodeCtlLineWords - 1) / kDecodeCtlLineWords * kDecodeCtlLineWords;
}

// Word offset, inside the control block, of the ready-word copies ([copy][route][flag stride]).
inline int64_t decode_flag_offset(int64_t T, int64_t H, int64_t I, int64_t topk) {
    const int64_t w = kDecodeCtlLineWords + decode_epoch_words(T, H, I, topk);
    return (w + kDecodeCtlLineWords - 1) / kDecodeCtlLineWords * kDecodeCtlLineWords;
}

// Byte offset, inside the control block, of the tagged h ([T*topk][I] 64-bit words).
inline int64_t decode_tagged_h_offset(int64_t T, int64_t H, int64_t I, int64_t topk) {
    const int64_t w = decode_flag_offset(T, H, I, topk) + kDecodeFlagCopies * T * topk * decode_flag_stride(I);
    return (4 * w + 255) / 256 * 256;
}

// Bytes of the control block: the error word's line and, for shapes the one-launch step can take,
// its epoch words, the ready-word copies and the tagged h.
inline int64_t decode_ctl_bytes(int64_t T, int64_t H, int64_t I, int64_t topk) {
    if (!decode_one_launch_ok(T, H, I, topk)) return 4 * kDecodeCtlLineWords;
    return decode_tagged_h_offset(T, H, I, topk) + 8 * T * topk * I;
}

// Word 1 of the control block: the shape the workspace was initialized for, packed exactly for every
// shape the one-launch step takes (T < 2^16, topk <= 64, H/128 <= 16, I/128 <= 8), bit 31 set.  The
// one-launch step compares it with its own shape before it trusts any hand-off word.
inline uint32_t decode_ctl_signature(int64_t T, int64_t H, int64_t I, int64_t topk) {
    return 0x80000000u | (uint32_t)(T & 0xFFFF) | (uint32_t)((topk - 1) & 63) << 16 |
           (uint32_t)((H / 128 - 1) & 15) << 22 | (uint32_t)((I / 128 - 1) & 7) << 26;
}

// Values of the error word (word 0 of the control block) after a one-launch step.
constexpr uint32_t kDecodeErrWait = 1;    // a hand-off wait gave up
constexpr uint32_t kDecodeErrShape = 2;   // the workspace was initialized for another shape

// Enqueues the decode step as one launch when the shape allows it and all its blocks fit on the
// device at once; returns 1 without launching otherwise, else a status.
int fused_decode_one_launch(hipStream_t st, FusedDecodeArgs a);

}  // namespace moe
