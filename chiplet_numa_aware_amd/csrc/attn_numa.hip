// C ABI of the attention forward library (declared in include/attn_numa.h).
//
// Host side: argument validation, the per-device XCD count, choice of the
// kernel instantiation (padded head dim 64/128 x causal) and the launch on
// the caller's stream.  No entry point allocates or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/attn_numa.h"
#include "attn_fwd_kernel.hpp"
#include "host_util.hpp"
#include "merge_kernel.hpp"
#include "wg_map.hpp"

namespace attn_numa {
namespace {

// Everything one forward launch needs.
struct FwdArgs {
  const void *q, *k, *v;
  void* o;
  float* lse;
  int B, H_U, H_KV, N_rows, pos_mod, N_kv, d, M_q, kv_chunk, num_splits;
  float *o_ws, *lse_ws;
  int W, mapping, X;
  float scale_log2;
};

template <int D, bool CAUSAL, bool FULL_D>
hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, FULL_D>), dim3(a.W), dim3(kThreads), 0,
                     stream, static_cast<const uint16_t*>(a.q),
                     static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o),
                     a.lse, a.B, a.H_U, a.H_KV, a.N_rows, a.pos_mod, a.N_kv, a.d, a.M_q, a.kv_chunk,
                     a.num_splits, a.o_ws, a.lse_ws, a.mapping, a.X, a.scale_log2);
  return hipGetLastError();
}

// Picks the instantiation: padded head dim D (64 or 128), causal, and whether
// d == D (no padded columns to zero-fill).
template <int D>
hipError_t launch(const FwdArgs& a, int causal, hipStream_t s) {
  const bool full = (a.d == D);
  if (causal)
    return full ? launch_one<D, true, true>(a, s) : launch_one<D, true, false>(a, s);
  return full ? launch_one<D, false, true>(a, s) : launch_one<D, false, false>(a, s);
}

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
  if (mapping < 0 || mapping > 7) return ATTN_E_MAPPING;
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
  hipError_t e = (d <= 64) ? launch<64>(a, causal, s) : launch<128>(a, causal, s);
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

// Placement probe: one wave per workgroup; lane 0 records the XCC id the
// workgroup runs on and the coordinates the remap gives it.
__global__ void probe_kernel(int32_t* out, int B, int H_Q, int M, int mapping,
                             int X, int G) {
  if (threadIdx.x != 0) return;
  uint32_t xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  const WgCoord c = wg_map(mapping, blockIdx.x, B, H_Q, M, X, G);
  int32_t* p = out + 4 * (uint64_t)blockIdx.x;
  p[0] = (int32_t)(xcc & 0xF);
  p[1] = (int32_t)c.b;
  p[2] = (int32_t)c.h;
  p[3] = (int32_t)c.m;
}

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

int attn_wg_map(int mapping, int B, int H_Q, int H_KV, int N, int num_xcd,
                int32_t* out_host) {
  if (!out_host) return ATTN_E_NULL;
  int M = 0, W = 0;
  int rc = check_shape(B, H_Q, H_KV, N, &M, &W);
  if (rc != ATTN_OK) return rc;
  if (num_xcd < 1) return ATTN_E_SHAPE;
  if (mapping < 0 || mapping > 7) return ATTN_E_MAPPING;
  for (int w = 0; w < W; ++w) {
    const WgCoord c = wg_map(mapping, (uint32_t)w, (uint32_t)B, (uint32_t)H_Q,
                             (uint32_t)M, (uint32_t)num_xcd, (uint32_t)(H_Q / H_KV));
    out_host[3 * (int64_t)w + 0] = (int32_t)c.b;
    out_host[3 * (int64_t)w + 1] = (int32_t)c.h;
    out_host[3 * (int64_t)w + 2] = (int32_t)c.m;
  }
  return ATTN_OK;
}

int attn_block_m(void) { return kBlockM; }

int attn_num_xcd(void) {
  int X = 0;
  int rc = resolve_xcd(&X);
  return rc == ATTN_OK ? X : rc;
}

int attn_probe_placement(int mapping, int B, int H_Q, int H_KV, int N,
                         int32_t* dev_out, void* stream) {
  if (!dev_out) return ATTN_E_NULL;
  int M = 0, W = 0;
  int rc = check_shape(B, H_Q, H_KV, N, &M, &W);
  if (rc != ATTN_OK) return rc;
  if (mapping < 0 || mapping > 7) return ATTN_E_MAPPING;
  if (!aligned16(dev_out)) return ATTN_E_ALIGN;
  int X = 1;
  rc = resolve_xcd(&X);
  if (rc != ATTN_OK) return rc;
  hipLaunchKernelGGL(probe_kernel, dim3(W), dim3(64), 0,
                     static_cast<hipStream_t>(stream), dev_out, B, H_Q, M,
                     mapping, X, H_Q / H_KV);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "attn_probe_placement launch");
  return ATTN_OK;
}

const char* attn_strerror(int code) {
  switch (code) {
    case ATTN_OK: return "ok";
    case ATTN_E_NULL: return "a required pointer is NULL";
    case ATTN_E_SHAPE:
      return "bad shape (B, H_Q, H_KV, N must be > 0, H_Q % H_KV == 0, "
             "B*H_Q*ceil(N/256) < 2^31, N*d*2 <= 2^31 - 2^16, num_xcd >= 1)";
    case ATTN_E_HEAD_DIM: return "unsupported head dim (need 8 <= d <= 128, d % 8 == 0)";
    case ATTN_E_MAPPING: return "mapping must be 0..7";
    case ATTN_E_ALIGN: return "device pointer not 16-byte aligned";
    case ATTN_E_HIP:
      return g_err_text[0] ? g_err_text : "HIP runtime error";
    case ATTN_E_NO_DEVICE: return "no HIP device visible";
    default: return "unknown error code";
  }
}

}  // extern "C"
