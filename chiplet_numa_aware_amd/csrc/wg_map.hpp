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
//   bit 3  balanced split (swizzled head-first only; other modes ignore it).
//                   It acts only on XCDs whose slice holds part of an ACC
//                   that a slice boundary splits, and keeps every XCD's ACCs.
//                   (a) A split ACC's (row block, head) units are laid out in
//                   folded order (its longest-first list taken first, last,
//                   second, second-to-last, ...) before the slices cut it:
//                   under a causal mask row block m carries work linear in m,
//                   so consecutive folded units pair up into equal work and
//                   each XCD's piece carries work in proportion to its size.
//                   (b) On such an XCD a piece is merged with the adjacent
//                   whole ACC of the slice (a leading piece with the first
//                   whole ACC, a trailing one with the last; with fewer than
//                   two whole ACCs the whole slice is one group), and a merged
//                   group runs longest first (row block descending, then ACC,
//                   then head): the list-scheduling order that keeps the
//                   XCD's longest workgroups from starting last.  Groups run in
//                   slice order; a group of one whole ACC keeps the order of
//                   bits 0-2.
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

// Units of one ACC that an XCD's slice holds, as longest-first indices u
// (row block M-1-u/G, head u mod G of the group): [e0, e1) and [o0, o1).
// For a split ACC in folded order, positions [lo, hi) of the ACC hold the
// even positions s -> u = s/2 and the odd ones -> u = U-1-(s-1)/2.
struct AccPart {
  uint32_t acc, e0, e1, o0, o1;
};

ATTN_HD AccPart acc_part(uint32_t a, uint32_t lo, uint32_t hi, uint32_t U, bool split) {
  AccPart p;
  p.acc = a;
  if (split) {
    p.e0 = (lo + 1) / 2;
    p.e1 = (hi + 1) / 2;
    p.o0 = U - hi / 2;
    p.o1 = U - lo / 2;
  } else {  // a whole ACC: every unit, in longest-first order
    p.e0 = lo;
    p.e1 = hi;
    p.o0 = U;
    p.o1 = U;
  }
  return p;
}

// Elements of [a, b) below T.
ATTN_HD uint32_t below(uint32_t T, uint32_t a, uint32_t b) {
  return T <= a ? 0u : (T >= b ? b - a : T - a);
}

ATTN_HD uint32_t part_count_below(const AccPart& p, uint32_t T) {
  return below(T, p.e0, p.e1) + below(T, p.o0, p.o1);
}

ATTN_HD bool acc_split(uint32_t a, uint32_t U, uint32_t W, uint32_t X) {
  return slice_of(a * U, W, X) != slice_of(a * U + U - 1, W, X);
}

// Unit kk (in longest-first order: row block descending, then ACC, then
// head) of the group made of the parts of ACCs g_lo..g_hi (at most three)
// of the slice [s0, s1).  Returns (global ACC, longest-first index u).
ATTN_HD void merged_unit(uint32_t kk, uint32_t g_lo, uint32_t g_hi, uint32_t s0, uint32_t s1,
                         uint32_t U, uint32_t W, uint32_t X, uint32_t G, uint32_t M,
                         uint32_t* acc, uint32_t* u) {
  // At most three parts; the loops run over all three with a guard so that
  // every index is a constant and the parts stay in (scalar) registers.
  AccPart parts[3];
  const uint32_t np = g_hi - g_lo + 1;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const uint32_t a = g_lo + (uint32_t)i;
    const uint32_t lo = (s0 > a * U ? s0 : a * U) - a * U;
    const uint32_t hi = (s1 < a * U + U ? s1 : a * U + U) - a * U;
    parts[i] = (uint32_t)i < np ? acc_part(a, lo, hi, U, acc_split(a, U, W, X))
                                : AccPart{a, 0u, 0u, 0u, 0u};  // empty
  }
  auto count = [&](uint32_t md) {  // units of the group in row blocks above M-1-md
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 3; ++i) c += part_count_below(parts[i], md * G);
    return c;
  };
  // The largest md with count(md) <= kk (count(0) = 0, count(M) = group size).
  uint32_t lo_md = 0, hi_md = M;
  while (hi_md - lo_md > 1) {
    const uint32_t mid = (lo_md + hi_md) / 2;
    if (count(mid) <= kk) lo_md = mid; else hi_md = mid;
  }
  uint32_t r = kk - count(lo_md);
  const uint32_t bs = lo_md * G, be = bs + G;
  uint32_t found_acc = parts[0].acc, found_u = 0;
  bool found = false;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const AccPart& p = parts[i];
    const uint32_t ea = p.e0 > bs ? p.e0 : bs, eb = p.e1 < be ? p.e1 : be;
    const uint32_t ne = eb > ea ? eb - ea : 0u;
    const uint32_t oa = p.o0 > bs ? p.o0 : bs, ob = p.o1 < be ? p.o1 : be;
    const uint32_t no = ob > oa ? ob - oa : 0u;
    if (!found && r < ne) {
      found_acc = p.acc;
      found_u = ea + r;
      found = true;
    } else if (!found && r < ne + no) {
      found_acc = p.acc;
      found_u = oa + (r - ne);
      found = true;
    } else if (!found) {
      r -= ne + no;
    }
  }
  *acc = found_acc;  // found for every kk below the group size
  *u = found_u;
}

// (batch, query head, row block) at logical position L of the order that
// bits 0 and 2 give (batch outermost).
ATTN_HD WgCoord decode_logical(int mapping, uint32_t L, uint32_t H_Q, uint32_t M, uint32_t G) {
  const uint32_t per_batch = H_Q * M;
  WgCoord c;
  c.b = L / per_batch;
  const uint32_t r = L - c.b * per_batch;
  uint32_t m;
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


// All arguments are assumed validated: W = B*H_Q*M < 2^31, X >= 1, w < W,
// G (query heads per ACC) >= 1 divides H_Q.
ATTN_HD WgCoord wg_map(int mapping, uint32_t w, uint32_t B, uint32_t H_Q,
                       uint32_t M, uint32_t X, uint32_t G) {
  const uint32_t W = B * H_Q * M;
  if ((mapping & 3) == kSwizzledHeadFirst && (mapping & kBalancedSplit)) {
    const uint32_t U = G * M;  // units of one ACC; ACC a holds [a U, a U + U)
    const uint32_t x = w % X, k = w / X;
    const uint32_t s0 = x * (W / X) + (x < W % X ? x : W % X);
    const uint32_t s1 = s0 + W / X + (x < W % X ? 1u : 0u);
    const uint32_t a_lo = s0 / U, a_hi = (s1 - 1) / U;
    const uint32_t tail = acc_split(a_lo, U, W, X) ? 1u : 0u;
    const uint32_t head = (a_hi != a_lo && acc_split(a_hi, U, W, X)) ? 1u : 0u;
    if (tail + head > 0) {
      const uint32_t n_whole = a_hi - a_lo + 1 - tail - head;
      uint32_t g_lo = a_lo, g_hi = a_hi, kk = k;
      bool merged = true;
      if (n_whole >= 2) {
        // groups: {piece?, first whole}, each middle whole ACC, {last whole, piece?}
        const uint32_t first_end = (a_lo + tail + 1) * U;  // end of the first group
        const uint32_t size0 = first_end - s0;
        const uint32_t mid_units = (n_whole - 2) * U;
        if (k < size0) {
          g_hi = a_lo + tail;
          merged = tail != 0;
        } else if (k < size0 + mid_units) {
          g_lo = g_hi = a_lo + tail + 1 + (k - size0) / U;
          kk = (k - size0) % U;
          merged = false;
        } else {
          g_lo = a_hi - head;
          kk = k - size0 - mid_units;
          merged = head != 0;
        }
      }
      if (merged) {
        uint32_t acc = 0, u = 0;
        merged_unit(kk, g_lo, g_hi, s0, s1, U, W, X, G, M, &acc, &u);
        const uint32_t md = u / G;
        const uint32_t H_KV = H_Q / G;
        WgCoord c;
        c.b = acc / H_KV;
        c.h = (acc - c.b * H_KV) * G + (u - md * G);
        c.m = M - 1u - md;
        return c;
      }
      // A group of one whole ACC keeps the order of bits 0-2: fall through
      // with its logical position.
      return decode_logical(mapping, g_lo * U + kk, H_Q, M, G);
    }
  }
  const uint32_t L = (mapping & 2) ? chiplet_slice_index(w, W, X) : w;
  return decode_logical(mapping, L, H_Q, M, G);
}

}  // namespace attn_numa
