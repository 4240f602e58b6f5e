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
// The four modes of the pages are two independent bits:
//   bit 0  order    0 = block-first (heads fastest), 1 = head-first (row
//                   blocks fastest, so an ACC is a contiguous id range)
//   bit 1  swizzle  0 = logical id = w, 1 = XCD x = w mod X takes the x-th
//                   contiguous slice of the logical order, in order.
// A third bit, not on the pages, orders the work for causal attention:
//   bit 2  longest first: row blocks are taken from the last (the most keys
//                   under a causal mask) to the first, and in the head-first
//                   order the G query heads of an ACC that share a row block
//                   are adjacent (ACC, then row block, then head).
// Under a causal mask, row blocks differ in length; taken shortest first,
// the workgroups that share an XCD start at staggered times and drift apart
// in the K/V stream beyond what L2 holds.  Taken longest first, a workgroup
// that starts later is shorter, so concurrent workgroups stay close together.
// Batch is the outermost index in both orders.  Slices are balanced (their
// lengths differ by at most one), which is also the fallback when X does not
// divide the number of ACCs: every XCD still walks its ACCs in one run and an
// ACC is split only where a slice boundary falls inside it.  The pages leave
// that fallback open (digest §7, key implementation details, item 1; the
// commentary page's H_Q = 12 example).
// A fourth bit, not on the pages, balances the fallback's work:
//   bit 3  balanced split (swizzled head-first only; other modes ignore it):
//                   an ACC that a slice boundary splits takes its (row block,
//                   head) units in folded order, i.e. the longest-first list
//                   taken first, last, second, second-to-last, ...  Under a
//                   causal mask the work of row block m grows linearly with
//                   m, so consecutive units of the folded list pair up into
//                   equal work, and each XCD's piece of a split ACC carries
//                   work in proportion to its unit count.  Whole ACCs keep
//                   the order of bits 0-2.
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
  kLongestFirst = 4,  // bit, combined with any of the above
  kBalancedSplit = 8, // bit, acts on kSwizzledHeadFirst only
};
constexpr int kMaxMapping = 15;

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

// XCD slice holding logical position P < W (the inverse of the balanced
// slicing: the first W mod X slices hold one more position).
ATTN_HD uint32_t slice_of(uint32_t P, uint32_t W, uint32_t X) {
  const uint32_t base = W / X;
  const uint32_t big = (W % X) * (base + 1);  // positions in the longer slices
  return P < big ? P / (base + 1) : W % X + (P - big) / base;
}

// All arguments are assumed validated: W = B*H_Q*M < 2^31, X >= 1, w < W,
// G (query heads per ACC) >= 1 divides H_Q.
ATTN_HD WgCoord wg_map(int mapping, uint32_t w, uint32_t B, uint32_t H_Q,
                       uint32_t M, uint32_t X, uint32_t G) {
  const uint32_t per_batch = H_Q * M;
  const uint32_t W = B * per_batch;
  const uint32_t L = (mapping & 2) ? chiplet_slice_index(w, W, X) : w;
  WgCoord c;
  c.b = L / per_batch;
  const uint32_t r = L - c.b * per_batch;
  uint32_t m;
  if ((mapping & 3) == kSwizzledHeadFirst && (mapping & kBalancedSplit)) {
    const uint32_t U = G * M;  // units of one ACC; ACC a holds [a U, a U + U)
    const uint32_t a = L / U;
    if (slice_of(a * U, W, X) != slice_of(a * U + U - 1, W, X)) {
      const uint32_t s = L - a * U;
      // folded position s -> index u of the longest-first list (row block
      // M-1-u/G, head u mod G of the group)
      const uint32_t u = (s & 1u) ? U - 1u - (s >> 1) : (s >> 1);
      const uint32_t md = u / G;
      const uint32_t acc_in_batch = r / U;
      c.h = acc_in_batch * G + (u - md * G);
      c.m = M - 1u - md;
      return c;
    }
  }
  if ((mapping & 1) && (mapping & kLongestFirst)) {  // ACC, block, head
    const uint32_t acc = r / (G * M);
    const uint32_t s = r - acc * (G * M);
    m = s / G;
    c.h = acc * G + (s - m * G);
  } else if (mapping & 1) {  // head-first
    c.h = r / M;
    m = r - c.h * M;
  } else {  // block-first
    m = r / H_Q;
    c.h = r - m * H_Q;
  }
  c.m = (mapping & kLongestFirst) ? M - 1 - m : m;
  return c;
}

}  // namespace attn_numa
