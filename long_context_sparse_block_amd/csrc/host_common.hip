// Status strings, the thread-local HIP error text and stride checks.
#include <stddef.h>
#include <stdio.h>
#include <string.h>

#include "sa_host.h"

namespace {
thread_local char g_last_error[256] = "";
}

namespace sa_host {

sa_status record_hip_error(hipError_t e, const char* where) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
  return SA_ERR_HIP;
}

sa_status check_launch(const char* where) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return record_hip_error(e, where);
  return SA_OK;
}

sa_status resolve_strides(const int64_t* strides, int32_t B, int32_t H, int32_t H_kv, int32_t N,
                          int32_t d, int32_t align, Strides out[4]) {
  const int32_t heads[4] = {H, H_kv, H_kv, H};
  for (int t = 0; t < 4; ++t) {
    if (strides == nullptr) {
      out[t].s = d;
      out[t].h = (int64_t)N * d;
      out[t].b = (int64_t)heads[t] * N * d;
    } else {
      out[t].b = strides[3 * t + 0];
      out[t].h = strides[3 * t + 1];
      out[t].s = strides[3 * t + 2];
    }
    if (out[t].s < d || out[t].h < 0 || out[t].b < 0) return SA_ERR_INVALID;
    if (out[t].s % align || out[t].h % align || out[t].b % align) return SA_ERR_INVALID;
  }
  (void)B;
  return SA_OK;
}

}  // namespace sa_host

extern "C" {

const char* sa_status_string(sa_status s) {
  switch (s) {
    case SA_OK: return "ok";
    case SA_ERR_NULL: return "null pointer argument";
    case SA_ERR_INVALID: return "invalid argument";
    case SA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SA_ERR_CAPACITY: return "output buffer too small";
    case SA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* sa_last_hip_error(void) { return g_last_error; }

int32_t sa_version(void) { return 1; }

}  // extern "C"

namespace {

// One lane reads the shader-clock counter (s_memtime) and the constant-rate
// counter (s_memrealtime) at the start and once at least `ticks` constant-rate
// ticks have passed (or after a bounded number of polls), and stores both
// differences.
__global__ __launch_bounds__(64) void clock_probe_kernel(int64_t* out, int64_t ticks) {
  if (threadIdx.x != 0) return;
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  uint64_t r = r0;
  for (int64_t n = 0; (int64_t)(r - r0) < ticks && n < (int64_t)1 << 32; ++n) {
    __builtin_amdgcn_s_sleep(2);
    r = __builtin_amdgcn_s_memrealtime();
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  out[0] = (int64_t)(c1 - c0);
  out[1] = (int64_t)(r - r0);
}

}  // namespace

extern "C" {

sa_status sa_clock_probe(int64_t* out, int64_t ticks, hipStream_t stream) {
  if (out == nullptr) return SA_ERR_NULL;
  if (ticks < 0 || ticks > (int64_t)100000000 * 60) return SA_ERR_INVALID;
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, stream, out, ticks);
  return sa_host::check_launch("clock_probe_kernel");
}

int32_t sa_mask_desc_layout(int64_t* out, int32_t n) {
  const int64_t v[18] = {(int64_t)sizeof(sa_mask_desc),
                         (int64_t)offsetof(sa_mask_desc, num_blocks),
                         (int64_t)offsetof(sa_mask_desc, num_groups),
                         (int64_t)offsetof(sa_mask_desc, causal),
                         (int64_t)offsetof(sa_mask_desc, win_before),
                         (int64_t)offsetof(sa_mask_desc, win_after),
                         (int64_t)offsetof(sa_mask_desc, win_clamp),
                         (int64_t)offsetof(sa_mask_desc, global_blocks),
                         (int64_t)offsetof(sa_mask_desc, num_global),
                         (int64_t)offsetof(sa_mask_desc, num_random),
                         (int64_t)offsetof(sa_mask_desc, random_blocks),
                         (int64_t)offsetof(sa_mask_desc, literal_mode),
                         (int64_t)offsetof(sa_mask_desc, literal_flags),
                         (int64_t)offsetof(sa_mask_desc, literal_p),
                         (int64_t)offsetof(sa_mask_desc, seed),
                         (int64_t)offsetof(sa_mask_desc, exclude_parts),
                         (int64_t)offsetof(sa_mask_desc, group_period),
                         (int64_t)offsetof(sa_mask_desc, period_exclude)};
  if (out == nullptr) return 18;
  for (int32_t i = 0; i < n && i < 18; ++i) out[i] = v[i];
  return 18;
}

}  // extern "C"
