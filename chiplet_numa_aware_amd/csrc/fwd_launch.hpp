// What one forward launch needs, and the per-head-dim launchers (each
// compiled in its own translation unit: attn_fwd_d64.hip, attn_fwd_d128.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace attn_numa {

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


// Launch the forward kernel of padded head dim 64 (d <= 64) or 128
// (64 < d <= 128): picks causal and d == D instantiations.
hipError_t launch_fwd_d64(const FwdArgs& a, int causal, hipStream_t s);
hipError_t launch_fwd_d128(const FwdArgs& a, int causal, hipStream_t s);

// Units of at most this many rows (decode; only one wave of an
// attn_fwd_kernel workgroup would have rows) run attn_decode_kernel instead:
// one-wave workgroups of 32 rows (attn_decode.hip).  a.W and a.M_q are
// ignored; the launcher sizes its own grid.
constexpr int kDecodeMaxRows = 64;
hipError_t launch_decode(const FwdArgs& a, int causal, hipStream_t s);

}  // namespace attn_numa
