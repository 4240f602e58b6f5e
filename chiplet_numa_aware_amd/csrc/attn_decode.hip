// Launch of the decode kernel (units of at most kDecodeMaxRows rows): picks
// the padded head dim, causal and d == D instantiations and sizes the grid,
// one 32-row workgroup per (unit, split, row block).
#include <hip/hip_runtime.h>

#include "decode_kernel.hpp"
#include "fwd_launch.hpp"

namespace attn_numa {
namespace {

template <int D, bool CAUSAL, bool FULL_D>
hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
  const int M = (a.N_rows + kDecRows - 1) / kDecRows;
  const unsigned W = (unsigned)a.B * (unsigned)a.H_U * (unsigned)M * (unsigned)a.num_splits;
  hipLaunchKernelGGL((attn_decode_kernel<D, CAUSAL, FULL_D>), dim3(W), dim3(64), 0, stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, a.B,
                     a.H_U, a.H_KV, a.N_rows, a.pos_mod, a.N_kv, a.d, M, a.kv_chunk,
                     a.num_splits, a.o_ws, a.lse_ws, a.mapping, a.X, a.scale_log2);
  return hipGetLastError();
}

template <int D>
hipError_t launch(const FwdArgs& a, int causal, hipStream_t s) {
  const bool full = (a.d == D);
  if (causal)
    return full ? launch_one<D, true, true>(a, s) : launch_one<D, true, false>(a, s);
  return full ? launch_one<D, false, true>(a, s) : launch_one<D, false, false>(a, s);
}

}  // namespace

hipError_t launch_decode(const FwdArgs& a, int causal, hipStream_t s) {
  return a.d <= 64 ? launch<64>(a, causal, s) : launch<128>(a, causal, s);
}

}  // namespace attn_numa
