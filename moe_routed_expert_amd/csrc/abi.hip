// Host entry points of libmoe_routed that are not tied to one kernel file:
// status text, the M-tile picker, argument checks of the block-FP8 GEMM, and
// the fused decode step with its workspace.
#include <string.h>

#include <mutex>

#include "device.h"
#include "host.h"
#include "decode_args.h"

namespace moe {

int slot_gemm_launch(hipStream_t st, bool a_is_bf16, const void* a, int64_t a_stride, const float* a_s,
                     int64_t a_s_stride, const uint8_t* w_q, int64_t w_stride_e, int64_t w_stride_n,
                     const float* w_s, int64_t w_s_stride_e, int64_t w_s_stride_n, int64_t N, int64_t K,
                     const int32_t* slots, int64_t rows, int64_t a_row_div, void* out, int out_dt,
                     int64_t out_stride);
int grouped_gemm_launch(hipStream_t st, int block_m, const uint8_t* a_q, int64_t a_stride, const float* a_s,
                        int64_t a_s_stride, const uint8_t* w_q, int64_t w_stride_e, int64_t w_stride_n,
                        const float* w_s, int64_t w_s_stride_e, int64_t w_s_stride_n, int64_t E, int64_t N,
                        int64_t K, const int32_t* offsets, int64_t m_rows, void* out, int out_dt,
                        int64_t out_stride);
int grouped_gemm_act_quant_launch(hipStream_t st, int block_m, int act, const uint8_t* a_q, int64_t a_stride,
                                  const float* a_s, int64_t a_s_stride, const uint8_t* w_q, int64_t w_stride_e,
                                  int64_t w_stride_n, const float* w_s, int64_t w_s_stride_e,
                                  int64_t w_s_stride_n, int64_t E, int64_t I, int64_t K, const int32_t* offsets,
                                  int64_t m_rows, uint8_t* q, int64_t q_stride, float* s, int64_t s_stride);
int mxfp4_grouped_gemm_launch(hipStream_t st, int block_m, int act, const uint8_t* a_q, int64_t a_stride,
                              const float* a_s, int64_t a_s_stride, const uint8_t* w4, int64_t w4_stride_e,
                              int64_t w4_stride_n, const uint8_t* w4s, int64_t w4s_stride_e, int64_t w4s_stride_n,
                              int64_t E, int64_t N, int64_t K, const int32_t* offsets, int64_t m_rows, void* out,
                              int out_dt, int64_t out_stride, uint8_t* q, int64_t q_stride, float* s,
                              int64_t s_stride);
int topk_reduce_launch(hipStream_t st, const void* y, int y_dt, int64_t y_stride, const int32_t* slot_ids,
                       const int32_t* route_rows, const float* weights, int64_t T, int64_t topk, int64_t H,
                       uint16_t* out, int64_t out_stride);



// Per host thread, so that concurrent callers never write one buffer at once.
static thread_local char g_last_hip_error[256] = "no HIP error recorded";

void note_hip_error(hipError_t e) {
    const char* s = hipGetErrorString(e);
    strncpy(g_last_hip_error, s ? s : "unknown HIP error", sizeof(g_last_hip_error) - 1);
    g_last_hip_error[sizeof(g_last_hip_error) - 1] = 0;
}

namespace {

// Clears the control block and writes the shape signature into its word 1.
__global__ void init_ctl_kernel(uint32_t* p, int64_t n, uint32_t sig) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = i == 1 ? sig : 0u;
}

struct DecodeLayout {
    int64_t off[7];   // c1, h, aq, as, c2, ctl, total
};

int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

DecodeLayout decode_layout(int64_t T, int64_t H, int64_t I, int64_t topk) {
    const int64_t R = T * topk;
    DecodeLayout L;
    int64_t o = 0;
    L.off[0] = o; o = align256(o + R * 2 * I * 4);            // c1 f32
    L.off[1] = o; o = align256(o + R * I * 4);                // h f32
    L.off[2] = o; o = align256(o + R * I);                    // aq fp8
    L.off[3] = o; o = align256(o + R * ceil_div(I, 128) * 4); // as f32
    L.off[4] = o; o = align256(o + R * H * 4);                // c2 f32
    L.off[5] = o; o = align256(o + decode_ctl_bytes(T, H, I, topk));  // ctl: hand-off words
    L.off[6] = o;
    return L;
}

// The weight bank of a grouped-mode GEMM: row-major with row stride w_stride_n >= row_bytes, or packed
// (w_stride_n == MOE_W_PACKED, moe_pack_weights) with expert stride >= N * row_bytes.
int weight_bank_ok(const uint8_t* w, int64_t w_stride_e, int64_t w_stride_n, int64_t n_experts, int64_t N,
                   int64_t row_bytes) {
    if (w_stride_n == MOE_W_PACKED) {
        if (n_experts > 1 && w_stride_e < N * row_bytes) return MOE_ERR_SHAPE;
        if (!aligned16(w) || w_stride_e % 16) return MOE_ERR_ALIGN;
        return MOE_OK;
    }
    if (w_stride_n < row_bytes || (n_experts > 1 && w_stride_e < N * w_stride_n)) return MOE_ERR_SHAPE;
    if (!aligned16(w) || w_stride_n % 16 || w_stride_e % 16) return MOE_ERR_ALIGN;
    return MOE_OK;
}

bool decode_shape_ok(int64_t T, int64_t H, int64_t I, int64_t topk) {
    return T >= 0 && H > 0 && I > 0 && H <= 65536 && I <= 65536 && topk >= 1 && topk <= 64 && H % 128 == 0 &&
           I % 128 == 0 && T * topk <= 65535;
}

// Scratch of moe_fused_decode_noalloc: a fixed device array standing in for the caller's workspace.  Each
// GPU the library runs on holds its own copy until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: host code uses the address hipGetSymbolAddress returns
// for the current device.
constexpr size_t kNoallocScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

struct NoallocDevice {
    void* ptr = nullptr;                       // device address of `scratch` on this device
    int64_t shape[4] = {-1, -1, -1, -1};       // (T, H, I, topk) its control block was last initialized for
};
std::mutex g_noalloc_mu;
NoallocDevice g_noalloc[64];

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_abi_version(void) { return MOE_ABI_VERSION; }

extern "C" const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "a required pointer is NULL";
        case MOE_ERR_SHAPE: return "a size, stride, mode or enum is out of range";
        case MOE_ERR_DTYPE: return "unsupported element type";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_ALIGN: return "a pointer or stride breaks the required 16-byte alignment";
        case MOE_ERR_HIP: return "the HIP runtime rejected a launch (see moe_last_hip_error)";
        case MOE_ERR_SCRATCH: return "the step needs more than the library's fixed 4 MiB decode scratch";
        default: return "unknown status";
    }
}

extern "C" const char* moe_last_hip_error(void) { return g_last_hip_error; }

extern "C" int moe_pick_block_m(int64_t routes, int64_t experts) {
    // The tile grows with rows per expert r as on the pages, with MI355X's own thresholds from a
    // sweep of every tile: r <= 8 -> 16 (6 rows), r <= 64 -> 64 (24 and 48 rows), else 128 (96 rows:
    // an expert's rows in one tile, so each weight byte is streamed once).
    if (routes <= 0 || experts <= 0) return 16;
    const int64_t r = ceil_div(routes, experts);
    return r <= 8 ? 16 : (r <= 64 ? 64 : 128);
}

extern "C" int moe_grouped_block_m(int64_t routes, int64_t experts, int64_t K, int mxfp4, int packed, int fused) {
    // The tile the grouped GEMMs take for block_m = 0, from an interleaved sweep of every tile at 48 to
    // 24576 routes over 256 experts (H = 4096, I = 1024), both weight formats and bank layouts, plain and
    // fused.  The 128-row tiles run a workgroup's tiles as one pipeline when a tile has at most 16 K steps
    // (block-FP8: always), so they win wherever that pipeline outweighs their single workgroup per CU.
    //   block-FP8, row-major, plain: 128 at every density (3-15 % ahead of the density rule's tile);
    //   block-FP8, row-major, fused: the density rule (the pipeline's epilogue costs more at few rows);
    //   block-FP8, packed: 16 up to 8 rows per expert, then 128 for K <= 2048 (down: 6 % ahead) or 64,
    //   then 128;
    //   MXFP4: 16 up to 8 rows per expert, then 32 (packed) or 64 (row-major) up to 64, then 128, or 64
    //   for packed banks with K > 2048 (the 128-row tiles run those one at a time: 4-12 % slower).
    if (routes <= 0 || experts <= 0) return 16;
    const int64_t r = ceil_div(routes, experts);
    const bool short_k = K / 128 <= 16;
    if (!mxfp4) {
        if (!packed) return fused ? moe_pick_block_m(routes, experts) : 128;
        if (r <= 8) return 16;
        if (r <= 64) return short_k ? 128 : 64;
        return 128;
    }
    if (r <= 8) return 16;
    if (r <= 64) return packed ? 32 : 64;
    return packed && !short_k ? 64 : 128;
}

extern "C" int moe_bf8_grouped_gemm(const uint8_t* a_q, int64_t a_stride, const float* a_s, int64_t a_s_stride,
                                    const uint8_t* w_q, int64_t w_stride_e, int64_t w_stride_n,
                                    const float* w_s, int64_t w_s_stride_e, int64_t w_s_stride_n,
                                    int64_t n_experts, int64_t N, int64_t K,
                                    int mode, const int32_t* expert_offsets, const int32_t* slot_ids,
                                    int64_t m_rows, int64_t a_row_div, int32_t block_m,
                                    void* out, int out_dt, int64_t out_stride, void* stream) {
    if (mode != MOE_MODE_GROUPED && mode != MOE_MODE_SLOT) return MOE_ERR_SHAPE;
    if (!dtype_ok(out_dt)) return MOE_ERR_DTYPE;
    if (m_rows < 0 || m_rows > 0x7FFFFFFF || n_experts < 0 || N <= 0 || K <= 0) return MOE_ERR_SHAPE;
    if (K % 128 != 0 || N % 16 != 0) return MOE_ERR_SHAPE;
    if (m_rows == 0) return MOE_OK;
    if (!out) return MOE_ERR_NULL;
    if (out_stride < N) return MOE_ERR_SHAPE;
    const int64_t kb = K / 128, nb = ceil_div(N, 128);
    const bool empty_bank = n_experts == 0;
    if (!empty_bank) {
        if (!w_q || !w_s || !a_q || !a_s) return MOE_ERR_NULL;
        if (a_stride < K || a_s_stride < kb || w_s_stride_n < kb) return MOE_ERR_SHAPE;
        if (n_experts > 1 && w_s_stride_e < nb * w_s_stride_n) return MOE_ERR_SHAPE;
        if (mode == MOE_MODE_SLOT && w_stride_n == MOE_W_PACKED) return MOE_ERR_SHAPE;
        const int rc = weight_bank_ok(w_q, w_stride_e, w_stride_n, n_experts, N, K);
        if (rc != MOE_OK) return rc;
        if (!aligned16(a_q) || a_stride % 16) return MOE_ERR_ALIGN;
    }
    auto st = as_stream(stream);
    if (mode == MOE_MODE_SLOT) {
        if (!slot_ids) return MOE_ERR_NULL;
        if (a_row_div < 1) return MOE_ERR_SHAPE;
        return slot_gemm_launch(st, false, a_q, a_stride, a_s, a_s_stride, w_q, w_stride_e, w_stride_n, w_s,
                                w_s_stride_e, w_s_stride_n, N, K, slot_ids, m_rows, a_row_div, out, out_dt,
                                out_stride);
    }
    if (empty_bank) return MOE_ERR_SHAPE;
    if (!expert_offsets) return MOE_ERR_NULL;
    if (N % 128 != 0) return MOE_ERR_SHAPE;
    int bm = block_m == 0 ? moe_grouped_block_m(m_rows, n_experts, K, 0, w_stride_n == MOE_W_PACKED, 0) : block_m;
    if (bm != 16 && bm != 32 && bm != 64 && bm != 128) return MOE_ERR_SHAPE;
    return grouped_gemm_launch(st, bm, a_q, a_stride, a_s, a_s_stride, w_q, w_stride_e, w_stride_n, w_s,
                               w_s_stride_e, w_s_stride_n, n_experts, N, K, expert_offsets, m_rows, out, out_dt,
                               out_stride);
}

extern "C" int moe_bf8_grouped_gemm_act_quant(const uint8_t* a_q, int64_t a_stride, const float* a_s,
                                              int64_t a_s_stride, const uint8_t* w_q, int64_t w_stride_e,
                                              int64_t w_stride_n, const float* w_s, int64_t w_s_stride_e,
                                              int64_t w_s_stride_n, int64_t n_experts, int64_t I, int64_t K,
                                              const int32_t* expert_offsets, int64_t m_rows, int32_t block_m,
                                              int act, uint8_t* out_q, int64_t q_stride, float* out_s,
                                              int64_t s_stride, void* stream) {
    if (m_rows < 0 || m_rows > 0x7FFFFFFF || n_experts < 1 || n_experts > 1024 || I < 128 || I % 128 || K < 128 ||
        K % 128 || K > 8192)
        return MOE_ERR_SHAPE;
    if (act < MOE_ACT_SILU_MUL || act > MOE_ACT_MUL) return MOE_ERR_SHAPE;
    if (block_m != 0 && block_m != 16 && block_m != 32 && block_m != 64 && block_m != 128) return MOE_ERR_SHAPE;
    if (m_rows == 0) return MOE_OK;
    if (!a_q || !a_s || !w_q || !w_s || !expert_offsets || !out_q || !out_s) return MOE_ERR_NULL;
    const int64_t kb = K / 128, nb = 2 * I / 128;
    if (a_stride < K || a_s_stride < kb || w_s_stride_n < kb || q_stride < I || s_stride < I / 128)
        return MOE_ERR_SHAPE;
    if (n_experts > 1 && w_s_stride_e < nb * w_s_stride_n) return MOE_ERR_SHAPE;
    const int rc = weight_bank_ok(w_q, w_stride_e, w_stride_n, n_experts, 2 * I, K);
    if (rc != MOE_OK) return rc;
    if (!aligned16(a_q) || a_stride % 16) return MOE_ERR_ALIGN;
    const int bm = block_m == 0 ? moe_grouped_block_m(m_rows, n_experts, K, 0, w_stride_n == MOE_W_PACKED, 1) : block_m;
    return grouped_gemm_act_quant_launch(as_stream(stream), bm, act, a_q, a_stride, a_s, a_s_stride, w_q,
                                         w_stride_e, w_stride_n, w_s, w_s_stride_e, w_s_stride_n, n_experts, I, K,
                                         expert_offsets, m_rows, out_q, q_stride, out_s, s_stride);
}

namespace {

// Checks shared by the two MXFP4 entry points (N = 2I for the fused one); MOE_OK when the operands fit.
int mxfp4_args_ok(const uint8_t* a_q, int64_t a_stride, const float* a_s, int64_t a_s_stride,
                  const uint8_t* w4, int64_t w4_stride_e, int64_t w4_stride_n, const uint8_t* w4s,
                  int64_t w4s_stride_e, int64_t w4s_stride_n, int64_t n_experts, int64_t N, int64_t K,
                  const int32_t* expert_offsets) {
    if (!a_q || !a_s || !w4 || !w4s || !expert_offsets) return MOE_ERR_NULL;
    if (a_stride < K || a_s_stride < K / 128 || w4s_stride_n < K / 32) return MOE_ERR_SHAPE;
    if (n_experts > 1 && w4s_stride_e < N * w4s_stride_n) return MOE_ERR_SHAPE;
    const int rc = weight_bank_ok(w4, w4_stride_e, w4_stride_n, n_experts, N, K / 2);
    if (rc != MOE_OK) return rc;
    if (!aligned16(a_q) || a_stride % 16) return MOE_ERR_ALIGN;
    if (reinterpret_cast<uintptr_t>(w4s) % 4 || w4s_stride_n % 4 || w4s_stride_e % 4) return MOE_ERR_ALIGN;
    return MOE_OK;
}

}  // namespace

extern "C" int moe_mxfp4_grouped_gemm(const uint8_t* a_q, int64_t a_stride, const float* a_s, int64_t a_s_stride,
                                      const uint8_t* w4, int64_t w4_stride_e, int64_t w4_stride_n,
                                      const uint8_t* w4_s, int64_t w4s_stride_e, int64_t w4s_stride_n,
                                      int64_t n_experts, int64_t N, int64_t K, const int32_t* expert_offsets,
                                      int64_t m_rows, int32_t block_m, void* out, int out_dt, int64_t out_stride,
                                      void* stream) {
    if (!dtype_ok(out_dt)) return MOE_ERR_DTYPE;
    if (m_rows < 0 || m_rows > 0x7FFFFFFF || n_experts < 1 || n_experts > 1024 || N < 128 || N % 128 || K < 128 ||
        K % 128 || K > 8192)
        return MOE_ERR_SHAPE;
    if (block_m != 0 && block_m != 16 && block_m != 32 && block_m != 64 && block_m != 128) return MOE_ERR_SHAPE;
    if (m_rows == 0) return MOE_OK;
    if (!out) return MOE_ERR_NULL;
    if (out_stride < N) return MOE_ERR_SHAPE;
    const int rc = mxfp4_args_ok(a_q, a_stride, a_s, a_s_stride, w4, w4_stride_e, w4_stride_n, w4_s, w4s_stride_e,
                                 w4s_stride_n, n_experts, N, K, expert_offsets);
    if (rc != MOE_OK) return rc;
    const int bm = block_m == 0 ? moe_grouped_block_m(m_rows, n_experts, K, 1, w4_stride_n == MOE_W_PACKED, 0) : block_m;
    return mxfp4_grouped_gemm_launch(as_stream(stream), bm, 0, a_q, a_stride, a_s, a_s_stride, w4, w4_stride_e,
                                     w4_stride_n, w4_s, w4s_stride_e, w4s_stride_n, n_experts, N, K, expert_offsets,
                                     m_rows, out, out_dt, out_stride, nullptr, 0, nullptr, 0);
}

extern "C" int moe_mxfp4_grouped_gemm_act_quant(const uint8_t* a_q, int64_t a_stride, const float* a_s,
                                                int64_t a_s_stride, const uint8_t* w4, int64_t w4_stride_e,
                                                int64_t w4_stride_n, const uint8_t* w4_s, int64_t w4s_stride_e,
                                                int64_t w4s_stride_n, int64_t n_experts, int64_t I, int64_t K,
                                                const int32_t* expert_offsets, int64_t m_rows, int32_t block_m,
                                                int act, uint8_t* out_q, int64_t q_stride, float* out_s,
                                                int64_t s_stride, void* stream) {
    if (m_rows < 0 || m_rows > 0x7FFFFFFF || n_experts < 1 || n_experts > 1024 || I < 128 || I % 128 || K < 128 ||
        K % 128 || K > 8192)
        return MOE_ERR_SHAPE;
    if (act < MOE_ACT_SILU_MUL || act > MOE_ACT_MUL) return MOE_ERR_SHAPE;
    if (block_m != 0 && block_m != 16 && block_m != 32 && block_m != 64 && block_m != 128) return MOE_ERR_SHAPE;
    if (m_rows == 0) return MOE_OK;
    if (!out_q || !out_s) return MOE_ERR_NULL;
    if (q_stride < I || s_stride < I / 128) return MOE_ERR_SHAPE;
    const int rc = mxfp4_args_ok(a_q, a_stride, a_s, a_s_stride, w4, w4_stride_e, w4_stride_n, w4_s, w4s_stride_e,
                                 w4s_stride_n, n_experts, 2 * I, K, expert_offsets);
    if (rc != MOE_OK) return rc;
    const int bm = block_m == 0 ? moe_grouped_block_m(m_rows, n_experts, K, 1, w4_stride_n == MOE_W_PACKED, 1) : block_m;
    return mxfp4_grouped_gemm_launch(as_stream(stream), bm, act, a_q, a_stride, a_s, a_s_stride, w4, w4_stride_e,
                                     w4_stride_n, w4_s, w4s_stride_e, w4s_stride_n, n_experts, 2 * I, K,
                                     expert_offsets, m_rows, nullptr, MOE_F32, 0, out_q, q_stride, out_s, s_stride);
}

extern "C" size_t moe_fused_decode_workspace_size(int64_t T, int64_t H, int64_t I, int64_t topk) {
    if (!decode_shape_ok(T, H, I, topk)) return 0;
    return (size_t)decode_layout(T, H, I, topk).off[6];
}

extern "C" int moe_fused_decode_workspace_layout(int64_t T, int64_t H, int64_t I, int64_t topk, int64_t offsets[7]) {
    if (!offsets) return MOE_ERR_NULL;
    if (!decode_shape_ok(T, H, I, topk)) return MOE_ERR_SHAPE;
    DecodeLayout L = decode_layout(T, H, I, topk);
    for (int i = 0; i < 7; i++) offsets[i] = L.off[i];
    return MOE_OK;
}

extern "C" int moe_fused_decode_workspace_init(void* workspace, size_t ws_bytes, int64_t T, int64_t H, int64_t I,
                                               int64_t topk, void* stream) {
    if (!decode_shape_ok(T, H, I, topk)) return MOE_ERR_SHAPE;
    if (!workspace) return MOE_ERR_NULL;
    DecodeLayout L = decode_layout(T, H, I, topk);
    if ((int64_t)ws_bytes < L.off[6]) return MOE_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MOE_ERR_ALIGN;
    const int64_t words = (L.off[6] - L.off[5]) / 4;
    hipLaunchKernelGGL(init_ctl_kernel, dim3((unsigned)ceil_div(words, 256)), dim3(256), 0, as_stream(stream),
                       (uint32_t*)((char*)workspace + L.off[5]), words, decode_ctl_signature(T, H, I, topk));
    return launch_status();
}

extern "C" int moe_fused_decode(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t I, int64_t topk, int act,
                                const int32_t* slot_ids, const float* weights, int64_t n_slots,
                                const uint8_t* w13_q, const float* w13_s,
                                const uint8_t* w2_q, const float* w2_s,
                                void* workspace, size_t ws_bytes, uint16_t* out_bf16, void* stream) {
    if (!decode_shape_ok(T, H, I, topk) || n_slots < 0) return MOE_ERR_SHAPE;
    if (act < MOE_ACT_SILU_MUL || act > MOE_ACT_MUL) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    if (!x_bf16 || !slot_ids || !weights || !workspace || !out_bf16) return MOE_ERR_NULL;
    if (n_slots > 0 && (!w13_q || !w13_s || !w2_q || !w2_s)) return MOE_ERR_NULL;
    DecodeLayout L = decode_layout(T, H, I, topk);
    if ((int64_t)ws_bytes < L.off[6]) return MOE_ERR_WORKSPACE;
    if (!aligned16(workspace) || (n_slots > 0 && (!aligned16(w13_q) || !aligned16(w2_q))) ||
        (reinterpret_cast<uintptr_t>(x_bf16) & 3u))
        return MOE_ERR_ALIGN;
    const int64_t R = T * topk;
    char* ws = (char*)workspace;
    float* c1 = (float*)(ws + L.off[0]);
    float* hbuf = (float*)(ws + L.off[1]);
    uint8_t* aq = (uint8_t*)(ws + L.off[2]);
    float* as = (float*)(ws + L.off[3]);
    float* c2 = (float*)(ws + L.off[4]);
    const int64_t gH = H / 128, gI = I / 128, g2I = 2 * I / 128;
    auto st = as_stream(stream);
    if (gI <= 8) {
        // one launch when the step fits on the device at once, else gate/up launch + down/reduce launch
        FusedDecodeArgs a;
        a.x = x_bf16; a.slots = slot_ids; a.weights = weights;
        a.w13 = w13_q; a.w13s = w13_s; a.w2 = w2_q; a.w2s = w2_s;
        a.c1 = c1; a.h = hbuf; a.aq = aq; a.as = as; a.c2 = c2; a.out = out_bf16;
        a.ctl = (uint32_t*)(ws + L.off[5]);
        a.T = (int)T; a.H = (int)H; a.I = (int)I; a.topk = (int)topk; a.act = act;
        a.tiles_a = 0; a.tiles_c = 0; a.n_a = 0;
        const int rc = fused_decode_one_launch(st, a);
        return rc == 1 ? fused_decode_two_launch(st, a) : rc;
    }
    // wider intermediate sizes: four launches
    // 1) gate/up per route, quantizing the bf16 token row on the fly
    int rc = slot_gemm_launch(st, true, x_bf16, H, nullptr, 0, w13_q, 2 * I * H, H, w13_s, g2I * gH, gH, 2 * I, H,
                              slot_ids, R, topk, c1, MOE_F32, 2 * I);
    // 2) act(gate)*up + 1x128 requant over every route (zero tiles stay zero)
    if (rc == MOE_OK) rc = moe_act_quant(c1, MOE_F32, 2 * I, R, I, act, aq, I, as, gI, stream);
    // 3) down per route
    if (rc == MOE_OK)
        rc = slot_gemm_launch(st, false, aq, I, as, gI, w2_q, H * I, I, w2_s, gH * gI, gI, H, I, slot_ids, R, 1, c2,
                              MOE_F32, H);
    // 4) routing-weighted reduce
    if (rc == MOE_OK) rc = topk_reduce_launch(st, c2, MOE_F32, H, slot_ids, nullptr, weights, T, topk, H, out_bf16, H);
    return rc;
}

extern "C" int moe_fused_decode_noalloc(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t I, int64_t topk, int act,
                                        const int32_t* slot_ids, const float* weights, int64_t n_slots,
                                        const uint8_t* w13_q, const float* w13_s, const uint8_t* w2_q,
                                        const float* w2_s, uint16_t* out_bf16, void* stream) {
    if (!decode_shape_ok(T, H, I, topk) || n_slots < 0) return MOE_ERR_SHAPE;
    if (act < MOE_ACT_SILU_MUL || act > MOE_ACT_MUL) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    const DecodeLayout L = decode_layout(T, H, I, topk);
    if (L.off[6] > (int64_t)kNoallocScratchBytes) return MOE_ERR_SCRATCH;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        note_hip_error(e);
        return MOE_ERR_HIP;
    }
    if (dev < 0 || dev >= 64) return MOE_ERR_HIP;
    void* ws = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_noalloc_mu);
        NoallocDevice& d = g_noalloc[dev];
        if (!d.ptr) {                                  // once per device, with that device current
            void* p = nullptr;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p) {
                note_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
                return MOE_ERR_HIP;
            }
            d.ptr = p;
        }
        ws = d.ptr;
        if (d.shape[0] != T || d.shape[1] != H || d.shape[2] != I || d.shape[3] != topk) {
            // another shape's control block: clear it (a fill kernel, no memset node) and record the shape
            const int rc = moe_fused_decode_workspace_init(ws, kNoallocScratchBytes, T, H, I, topk, stream);
            if (rc != MOE_OK) return rc;
            d.shape[0] = T; d.shape[1] = H; d.shape[2] = I; d.shape[3] = topk;
        }
    }
    return moe_fused_decode(x_bf16, T, H, I, topk, act, slot_ids, weights, n_slots, w13_q, w13_s, w2_q, w2_s, ws,
                            kNoallocScratchBytes, out_bf16, stream);
}
