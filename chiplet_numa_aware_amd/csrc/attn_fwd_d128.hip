// Forward kernel instantiations for padded head dim 128 (causal x d == D),
// in a translation unit of their own so the two head dims compile in
// parallel.
#include <hip/hip_runtime.h>

#include "attn_fwd_kernel.hpp"
#include "fwd_launch.hpp"

namespace attn_numa {
namespace {

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


}  // namespace

hipError_t launch_fwd_d128(const FwdArgs& a, int causal, hipStream_t s) {
  return launch<128>(a, causal, s);
}

}  // namespace attn_numa
