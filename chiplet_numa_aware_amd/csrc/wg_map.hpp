// Workgroup-ID remap: linear workgroup id -> (batch, query head, row block).
//
// Shared by the attention kernel (device) and attn_wg_map (host), so the
// table the host reports is the one the kernel runs.
//
// Source: "Optimizing Attention on GPUs by Exploiting GPU Architectural NUMA
// Effects" (digest page):
//   * §2 Q1: the dispatcher places linear workgroup id w on XCD (w mod X).
//   * §2 Q2, §3 Figure 10: an Attention Compute Cluster (ACC) is every
//     workgroup reading one K/V (one head for MHA, one KV group for GQA);
//     Swizzled Head-first keeps an ACC on one XCD, one ACC at a time.
//   * §3 before/after table and §7 Figures 3 and 11: the block-first and
//     head-first orders and the chiplet swizzle.
//
// The four modes are two independent bits:
//   bit 0  order    0 = block-first (heads fastest), 1 = head-first (row
//                   blocks fastest, so an ACC is a contiguous id range)
//   bit 1  swizzle  0 = logical id = w, 1 = XCD x = w mod X takes the x-th
//                   contiguous slice of the logical order, in order.
// Batch is the outermost index in both orders.  Slices are balanced (their
// lengths differ by at most one), which is also the fallback when X does not
// divide the number of ACCs: every XCD still walks its ACCs in one run and an
// ACC is split only where a slice boundary falls inside it.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define ATTN_HD __host__ __device__ __forceinline__
#else
#define ATTN_HD inline
#endif

namespace attn_numa {

enum Mapping : int {
  kNaiveBlockFirst = 0,
  kNaiveHeadFirst = 1,
  kSwizzledBlockFirst = 2,
  kSwizzledHeadFirst = 3,
};

constexpr int kBlockM = 256;  // query rows per workgroup (row-block height)

struct WgCoord {
  uint32_t b, h, m;
};

// Logical position of workgroup w when XCD (w mod X) owns a contiguous,
// balanced slice of [0, W).
ATTN_HD uint32_t chiplet_slice_index(uint32_t w, uint32_t W, uint32_t X) {
  const uint32_t x = w % X;
  const uint32_t base = W / X;
  const uint32_t extra = W % X;
  return x * base + (x < extra ? x : extra) + w / X;
}

// All arguments are assumed validated: W = B*H_Q*M < 2^31, X >= 1, w < W.
ATTN_HD WgCoord wg_map(int mapping, uint32_t w, uint32_t B, uint32_t H_Q,
                       uint32_t M, uint32_t X) {
  const uint32_t per_batch = H_Q * M;
  const uint32_t L =
      (mapping & 2) ? chiplet_slice_index(w, B * per_batch, X) : w;
  WgCoord c;
  c.b = L / per_batch;
  const uint32_t r = L - c.b * per_batch;
  if (mapping & 1) {  // head-first
    c.h = r / M;
    c.m = r - c.h * M;
  } else {  // block-first
    c.m = r / H_Q;
    c.h = r - c.m * H_Q;
  }
  return c;
}

}  // namespace attn_numa
