// Host-side checks shared by the entry points of the library: argument
// validation, the HIP error text of the calling thread and the per-device
// XCD count.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "../../include/attn_numa.h"
#include "wg_map.hpp"

namespace attn_numa {

inline thread_local char g_err_text[256];

inline int hip_fail(hipError_t e, const char* what) {
  std::snprintf(g_err_text, sizeof(g_err_text), "HIP error in %s: %s (%d)",
                what, hipGetErrorString(e), (int)e);
  return ATTN_E_HIP;
}

inline bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// Validates the shape; on success stores the row-block count and grid size.
inline int check_shape(int B, int H_Q, int H_KV, int N, int* M_out, int* W_out) {
  if (B <= 0 || H_Q <= 0 || H_KV <= 0 || N <= 0) return ATTN_E_SHAPE;
  if (H_Q % H_KV != 0) return ATTN_E_SHAPE;
  const int64_t M = ((int64_t)N + kBlockM - 1) / kBlockM;
  const int64_t W = (int64_t)B * H_Q * M;
  if (W >= (int64_t(1) << 31)) return ATTN_E_SHAPE;
  *M_out = (int)M;
  *W_out = (int)W;
  return ATTN_OK;
}

constexpr int64_t kMaxHeadBytes = (int64_t(1) << 31) - (int64_t(1) << 16);

inline int check_head_dim(int N, int d) {
  if (d <= 0 || d > 128 || (d % 8) != 0) return ATTN_E_HEAD_DIM;
  // One head must fit a buffer resource, with room for the out-of-range
  // offset (2^31) plus a tile offset and an instruction offset below 2^32.
  if ((int64_t)N * d * 2 > kMaxHeadBytes) return ATTN_E_SHAPE;
  return ATTN_OK;
}

constexpr int kMaxDevices = 64;
inline std::once_flag g_xcd_once[kMaxDevices];
inline int g_xcd[kMaxDevices];

inline int env_xcd_override() {
  const char* s = std::getenv("ATTN_NUM_XCD");
  if (!s || !*s) return 0;
  char* end = nullptr;
  long v = std::strtol(s, &end, 10);
  if (end == s || *end != '\0' || v < 1 || v > 64) return 0;
  return (int)v;
}

inline int device_xcd_count(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return ATTN_E_NO_DEVICE;
  if (dev < 0 || dev >= kMaxDevices) return ATTN_E_NO_DEVICE;
  std::call_once(g_xcd_once[dev], [dev]() {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeNumberOfXccs, dev) !=
            hipSuccess ||
        n < 1)
      n = 1;
    g_xcd[dev] = n;
  });
  *out = g_xcd[dev];
  return ATTN_OK;
}

inline int resolve_xcd(int* out) {
  int n = 0;
  int devs = 0;
  if (hipGetDeviceCount(&devs) != hipSuccess || devs <= 0)
    return ATTN_E_NO_DEVICE;
  const int over = env_xcd_override();
  if (over > 0) {
    *out = over;
    return ATTN_OK;
  }
  int rc = device_xcd_count(&n);
  if (rc != ATTN_OK) return rc;
  *out = n;
  return ATTN_OK;
}

}  // namespace attn_numa
