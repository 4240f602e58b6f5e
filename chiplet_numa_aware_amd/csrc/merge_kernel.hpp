// Merge of split-KV partial attention results (the decode reduction of the
// "Fused Grouped-Query Attention" page: per-shard partial results are reduced
// into the final output), in (O, lse) form:
//   lse = ln sum_s exp(lse_s),   O = sum_s exp(lse_s - lse) O_s.
//
// One wave per output row (b, h, row); lane l owns columns 2l and 2l + 1
// (d <= 128).  Every part is read once: S * (d + 1) * 4 bytes per row, so the
// kernel is bound by memory bandwidth.  A row whose parts are all -inf (it saw
// no key) gets O = 0 and lse = -inf.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn_numa {

constexpr int kMergeWaves = 4;  // rows per workgroup

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) x = fmaxf(x, __shfl_xor(x, s, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) x += __shfl_xor(x, s, 64);
  return x;
}

// o_parts fp32 [S][rows][d], lse_parts fp32 [S][rows] -> o bf16 [rows][d],
// lse fp32 [rows] (lse may be NULL).
__global__ __launch_bounds__(64 * kMergeWaves) void attn_merge_kernel(
    const float* __restrict__ o_parts, const float* __restrict__ lse_parts, int S,
    uint64_t rows, int d, uint16_t* __restrict__ o, float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const uint64_t row = (uint64_t)blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  if (row >= rows) return;  // the whole wave
  float m = -INFINITY;
  for (int s = lane; s < S; s += 64) m = fmaxf(m, lse_parts[(uint64_t)s * rows + row]);
  m = wave_max(m);
  const bool seen = m != -INFINITY;
  float total = 0.f;
  if (seen)
    for (int s = lane; s < S; s += 64) total += expf(lse_parts[(uint64_t)s * rows + row] - m);
  total = wave_sum(total);
  const int c = 2 * lane;
  float a0 = 0.f, a1 = 0.f;
  if (seen && c < d) {
    for (int s = 0; s < S; ++s) {
      const float w = expf(lse_parts[(uint64_t)s * rows + row] - m);  // 0 for an empty part
      const float2 x = *reinterpret_cast<const float2*>(o_parts + ((uint64_t)s * rows + row) * d + c);
      a0 += w * x.x;
      a1 += w * x.y;
    }
  }
  const float inv = seen ? 1.f / total : 0.f;
  if (c < d) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 p;
    p.x = (__bf16)(a0 * inv);
    p.y = (__bf16)(a1 * inv);
    *reinterpret_cast<uint32_t*>(o + row * d + c) = __builtin_bit_cast(uint32_t, p);
  }
  if (lse != nullptr && lane == 0) lse[row] = seen ? m + logf(total) : -INFINITY;
}

}  // namespace attn_numa
