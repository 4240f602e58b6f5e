// C ABI of the attention forward pass (attn_fwd, attn_fwd_split,
// attn_fwd_split_noalloc, attn_split_chunk, attn_merge in
// include/attn_numa.h): argument validation, the split-KV and packing
// choices, and the launches on the caller's stream.  No entry point
// allocates or synchronises; attn_fwd_split_noalloc keeps its split partials
// in the library's fixed device array.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/attn_numa.h"
#include "attn_fwd_kernel.hpp"
#include "fwd_launch.hpp"
#include "host_util.hpp"
#include "merge_kernel.hpp"
#include "wg_map.hpp"

namespace attn_numa {
namespace {

// Keys per split: ceil(N_kv / S) rounded up to whole 32-key tiles.
int64_t split_chunk(int N_kv, int S) {
  const int64_t per = ((int64_t)N_kv + S - 1) / S;
  return (per + kBlockN - 1) / kBlockN * kBlockN;
}


// pack: group the G = H_Q / H_KV query heads of each KV group into one unit
// of G * N_q rows (see the kernel); used by attn_fwd_split for short N_q.
int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H_Q, int H_KV, int N_q, int N_kv, int d, int causal,
             int num_splits, float* o_ws, float* lse_ws, int mapping, bool pack,
             void* stream) {
  if (!q || !k || !v || !o) return ATTN_E_NULL;
  if (N_q <= 0 || N_kv <= 0 || num_splits < 1) return ATTN_E_SHAPE;
  int M = 0, W = 0;
  int rc = check_shape(B, H_Q, H_KV, N_q, &M, &W);
  if (rc != ATTN_OK) return rc;
  if ((int64_t)W * num_splits >= (int64_t(1) << 31)) return ATTN_E_SHAPE;
  rc = check_head_dim(N_q, d);
  if (rc != ATTN_OK) return rc;
  rc = check_head_dim(N_kv, d);
  if (rc != ATTN_OK) return rc;
  if (mapping < 0 || mapping > kMaxMapping) return ATTN_E_MAPPING;
  if (num_splits > 1 && (!o_ws || !lse_ws)) return ATTN_E_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (lse && !aligned16(lse)) || (num_splits > 1 && (!aligned16(o_ws) || !aligned16(lse_ws))))
    return ATTN_E_ALIGN;
  int X = 1;
  rc = resolve_xcd(&X);
  if (rc != ATTN_OK) return rc;
  const int G = H_Q / H_KV;
  pack = pack && G > 1 && (int64_t)G * N_q * d * 2 <= kMaxHeadBytes;
  const int H_U = pack ? H_KV : H_Q;
  const int N_rows = pack ? G * N_q : N_q;  // <= kBlockM * G when packing
  const int M_q = (N_rows + kBlockM - 1) / kBlockM;
  FwdArgs a{q, k, v, o, lse, B, H_U, H_KV, N_rows, N_q, N_kv, d, M_q,
            (int)split_chunk(N_kv, num_splits), num_splits,
            num_splits > 1 ? o_ws : nullptr, num_splits > 1 ? lse_ws : nullptr,
            B * H_U * M_q * num_splits, mapping, X,
            (float)(1.4426950408889634 / std::sqrt((double)d))};
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (N_rows <= kDecodeMaxRows)
    e = launch_decode(a, causal, s);
  else
    e = (d <= 64) ? launch_fwd_d64(a, causal, s) : launch_fwd_d128(a, causal, s);
  if (e != hipSuccess) return hip_fail(e, "attn_fwd launch");
  if (num_splits > 1) {
    const uint64_t rows = (uint64_t)B * H_Q * N_q;
    hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)((rows + kMergeWaves - 1) / kMergeWaves)),
                       dim3(64 * kMergeWaves), 0, s, o_ws, lse_ws, num_splits, rows, d,
                       static_cast<uint16_t*>(o), lse);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "attn merge launch");
  }
  return ATTN_OK;
}


// Fixed device scratch of attn_fwd_split_noalloc: the split partials (O of
// each split, then its lse) of one call.  Each GPU the library runs on holds
// its own copy until the process ends.  In host code `scratch` is only a
// stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is passed on.
static __device__ __align__(256) float scratch[ATTN_SCRATCH_BYTES / sizeof(float)];

std::once_flag g_scratch_once[kMaxDevices];
float* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of this device's scratch (the current device), or null with
// the HIP error in *err.
float* device_scratch(hipError_t* err) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? static_cast<float*>(p) : nullptr;
  });
  *err = g_scratch_err[dev];
  return g_scratch_ptr[dev];
}

// Bytes of scratch a split call needs: O partials, then lse partials from the
// next 256-byte boundary.
uint64_t scratch_lse_offset(uint64_t rows, int d) { return (rows * (uint64_t)d * 4 + 255) / 256 * 256; }

}  // namespace
}  // namespace attn_numa

using namespace attn_numa;

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H_Q, int H_KV, int N, int d, int causal, int mapping,
             void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H_Q, H_KV, N, N, d, causal, 1, nullptr,
                  nullptr, mapping, false, stream);
}

int attn_fwd_split(const void* q, const void* k, const void* v, void* o,
                   float* lse, int B, int H_Q, int H_KV, int N_q, int N_kv,
                   int d, int causal, int num_splits, float* o_ws,
                   float* lse_ws, int mapping, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H_Q, H_KV, N_q, N_kv, d, causal,
                  num_splits, o_ws, lse_ws, mapping, N_q < kBlockM, stream);
}

int attn_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o,
                           float* lse, int B, int H_Q, int H_KV, int N_q, int N_kv,
                           int d, int causal, int num_splits, int mapping, void* stream) {
  if (num_splits <= 1)
    return fwd_impl(q, k, v, o, lse, B, H_Q, H_KV, N_q, N_kv, d, causal, num_splits,
                    nullptr, nullptr, mapping, N_q < kBlockM, stream);
  // Size check first, before any device query: rows of all splits, with the
  // shape's own limits checked by fwd_impl below.
  if (B <= 0 || H_Q <= 0 || N_q <= 0) return ATTN_E_SHAPE;
  if (d <= 0 || d > 128 || (d % 8) != 0) return ATTN_E_HEAD_DIM;
  const uint64_t rows = (uint64_t)num_splits * (uint64_t)B * (uint64_t)H_Q * (uint64_t)N_q;
  const uint64_t lse_off = scratch_lse_offset(rows, d);
  if (lse_off + rows * 4 > (uint64_t)ATTN_SCRATCH_BYTES) return ATTN_E_SCRATCH;
  if (!q || !k || !v || !o) return ATTN_E_NULL;
  int devs = 0;
  if (hipGetDeviceCount(&devs) != hipSuccess || devs <= 0) return ATTN_E_NO_DEVICE;
  hipError_t e = hipSuccess;
  float* base = device_scratch(&e);
  if (!base) return hip_fail(e, "attn_fwd_split_noalloc scratch address");
  return fwd_impl(q, k, v, o, lse, B, H_Q, H_KV, N_q, N_kv, d, causal, num_splits, base,
                  base + lse_off / 4, mapping, N_q < kBlockM, stream);
}

int attn_split_chunk(int N_kv, int num_splits) {
  if (N_kv <= 0 || num_splits < 1) return ATTN_E_SHAPE;
  return (int)split_chunk(N_kv, num_splits);
}

int attn_merge(const float* o_parts, const float* lse_parts, int num_splits,
               int B, int H_Q, int N_q, int d, void* o, float* lse,
               void* stream) {
  if (!o_parts || !lse_parts || !o) return ATTN_E_NULL;
  if (num_splits < 1 || B <= 0 || H_Q <= 0 || N_q <= 0) return ATTN_E_SHAPE;
  if (d <= 0 || d > 128 || (d % 8) != 0) return ATTN_E_HEAD_DIM;
  const uint64_t rows = (uint64_t)B * H_Q * N_q;
  if ((rows + kMergeWaves - 1) / kMergeWaves >= (uint64_t(1) << 31)) return ATTN_E_SHAPE;
  if (!aligned16(o_parts) || !aligned16(lse_parts) || !aligned16(o) || (lse && !aligned16(lse)))
    return ATTN_E_ALIGN;
  int devs = 0;
  if (hipGetDeviceCount(&devs) != hipSuccess || devs <= 0) return ATTN_E_NO_DEVICE;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)((rows + kMergeWaves - 1) / kMergeWaves)),
                     dim3(64 * kMergeWaves), 0, static_cast<hipStream_t>(stream), o_parts,
                     lse_parts, num_splits, rows, d, static_cast<uint16_t*>(o), lse);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "attn_merge launch");
  return ATTN_OK;
}

}  // extern "C"
