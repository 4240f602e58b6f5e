// C ABI of the attention backward pass (attn_bwd in include/attn_numa.h):
// validation, choice of the kernel instantiation (padded head dim 64/128 x
// causal x d == D) and the three launches on the caller's stream.  Allocates
// nothing and does not synchronise.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/attn_numa.h"
#include "attn_bwd_kernel.hpp"
#include "host_util.hpp"

namespace attn_numa {
namespace {

// Everything one backward launch needs.
struct BwdArgs {
  const void *q, *k, *v, *dout;
  const float* ws;
  void *dq, *dk, *dv;
  int B, H_Q, H_KV, N, d, M_kv, M_q, mapping, X;
  float scale_log2, scale;
};

template <int D, bool CAUSAL, bool FULL_D>
hipError_t launch_bwd_one(const BwdArgs& a, hipStream_t s) {
  const auto* q = static_cast<const uint16_t*>(a.q);
  const auto* k = static_cast<const uint16_t*>(a.k);
  const auto* v = static_cast<const uint16_t*>(a.v);
  const auto* dout = static_cast<const uint16_t*>(a.dout);
  hipLaunchKernelGGL((attn_bwd_dkv_kernel<D, CAUSAL, FULL_D>),
                     dim3(a.B * a.H_KV * a.M_kv), dim3(kBwdThreads), 0, s, q, k, v, dout, a.ws,
                     static_cast<uint16_t*>(a.dk), static_cast<uint16_t*>(a.dv), a.B, a.H_Q,
                     a.H_KV, a.N, a.d, a.M_kv, a.mapping, a.X, a.scale_log2, a.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, CAUSAL, FULL_D>), dim3(a.B * a.H_Q * a.M_q),
                     dim3(kBwdThreads), 0, s, q, k, v, dout, a.ws,
                     static_cast<uint16_t*>(a.dq), a.B, a.H_Q, a.H_KV, a.N, a.d, a.M_q,
                     a.mapping, a.X, a.scale_log2, a.scale);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd(const BwdArgs& a, int causal, hipStream_t s) {
  const bool full = (a.d == D);
  if (causal)
    return full ? launch_bwd_one<D, true, true>(a, s) : launch_bwd_one<D, true, false>(a, s);
  return full ? launch_bwd_one<D, false, true>(a, s) : launch_bwd_one<D, false, false>(a, s);
}

}  // namespace
}  // namespace attn_numa

using namespace attn_numa;

extern "C" {

int attn_bwd(const void* q, const void* k, const void* v, const void* o,
             const void* dout, const float* lse, void* dq, void* dk, void* dv,
             float* ws, int B, int H_Q, int H_KV, int N, int d, int causal,
             int mapping, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !ws) return ATTN_E_NULL;
  int M = 0, W = 0;
  int rc = check_shape(B, H_Q, H_KV, N, &M, &W);
  if (rc != ATTN_OK) return rc;
  const int64_t M_b = ((int64_t)N + kBwdBlock - 1) / kBwdBlock;
  if ((int64_t)B * H_Q * M_b >= (int64_t(1) << 31)) return ATTN_E_SHAPE;
  const uint64_t rows = (uint64_t)B * H_Q * N;
  if ((rows + 3) / 4 >= (uint64_t(1) << 31)) return ATTN_E_SHAPE;
  rc = check_head_dim(N, d);
  if (rc != ATTN_OK) return rc;
  if (mapping < 0 || mapping > kMaxMapping) return ATTN_E_MAPPING;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(ws))
    return ATTN_E_ALIGN;
  int X = 1;
  rc = resolve_xcd(&X);
  if (rc != ATTN_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(attn_bwd_pre_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(dout), lse,
                     ws, rows, d, N);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "attn_bwd preprocess launch");
  const double scale = 1.0 / std::sqrt((double)d);
  const int M_kv = (int)M_b;
  BwdArgs a{q, k, v, dout, ws, dq, dk, dv, B, H_Q, H_KV, N, d, M_kv, M_kv, mapping, X,
            (float)(1.4426950408889634 * scale), (float)scale};
  e = (d <= 64) ? launch_bwd<64>(a, causal, s) : launch_bwd<128>(a, causal, s);
  if (e != hipSuccess) return hip_fail(e, "attn_bwd launch");
  return ATTN_OK;
}

}  // extern "C"
