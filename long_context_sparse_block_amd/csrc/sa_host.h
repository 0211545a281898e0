// Host-side helpers of the C ABI: error text, argument checks, stride handling.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sparse_attn.h"

namespace sa_host {

// Record a HIP error for sa_last_hip_error() and return SA_ERR_HIP.
sa_status record_hip_error(hipError_t e, const char* where);

// hipGetLastError() after a launch: SA_OK or SA_ERR_HIP (recorded).
sa_status check_launch(const char* where);

// Strides (in elements) of one [B, H, N, d] tensor.
struct Strides {
  int64_t b, h, s;
};

// Fill q, k, v, o strides from the caller's HOST int64 [4][3] array (or the
// contiguous defaults when NULL) and check them: positive sequence stride >= d,
// non-negative batch/head strides, and every stride a multiple of `align`
// elements (16-byte rows).
sa_status resolve_strides(const int64_t* strides, int32_t B, int32_t H, int32_t H_kv, int32_t N,
                          int32_t d, int32_t align, Strides out[4]);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace sa_host
