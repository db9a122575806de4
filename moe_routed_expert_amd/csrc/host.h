// Host-side helpers shared by the entry points of libmoe_routed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_routed.h"

namespace moe {

// Records the text of a failed HIP call for moe_last_hip_error().
void note_hip_error(hipError_t e);

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool dtype_ok(int dt) { return dt == MOE_BF16 || dt == MOE_F32 || dt == MOE_F16; }

// Checks the launch that was just enqueued.
inline int launch_status() {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        note_hip_error(e);
        return MOE_ERR_HIP;
    }
    return MOE_OK;
}

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace moe
