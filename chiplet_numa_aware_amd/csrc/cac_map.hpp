// Compute Affinity Cluster (CAC) tile map for a tiled GEMM: linear workgroup
// id -> (batch, tile row, tile column).
//
// "Optimizing Attention on GPUs by Exploiting GPU Architectural NUMA
// Effects" (commentary page, the paragraph generalising the ACC): the ACC
// becomes a Compute Affinity Cluster, the set of workgroups that share input
// data, so that other kernels such as GEMM get the same XCD placement.  In
// C = A B^T an output tile (i, j) reads row panel i of A and column panel j
// of B; a block of gm x gn tiles shares gm A panels and gn B panels, which is
// the cluster here.  The two bits mirror the attention remap (wg_map.hpp):
//   bit 0  order    0 = row-major tiles (columns fastest), 1 = cluster-major:
//                   gm x gn blocks of tiles (row-major over blocks, clipped at
//                   the grid's edges), tiles row-major inside a block
//   bit 1  swizzle  0 = logical id = w (the dispatcher's round robin spreads
//                   consecutive ids over the XCDs), 1 = XCD x = w mod X takes
//                   the x-th contiguous balanced slice of the logical order
//                   (chiplet_slice_index), so one XCD walks whole clusters.
// Batch is outermost in both orders.
#pragma once

#include <stdint.h>

#include "wg_map.hpp"

namespace attn_numa {

struct TileCoord {
  uint32_t l, tm, tn;
};

// All arguments are assumed validated: W = L*Mt*Nt < 2^31, w < W, X >= 1,
// 1 <= gm, 1 <= gn.
ATTN_HD TileCoord cac_tile_map(int mapping, uint32_t w, uint32_t L, uint32_t Mt,
                               uint32_t Nt, uint32_t gm, uint32_t gn, uint32_t X) {
  const uint32_t per_batch = Mt * Nt;
  const uint32_t r0 = (mapping & 2) ? chiplet_slice_index(w, L * per_batch, X) : w;
  TileCoord c;
  c.l = r0 / per_batch;
  const uint32_t r = r0 - c.l * per_batch;
  if (mapping & 1) {
    // Every cluster row but the last is gm tall, and the last one comes last,
    // so the cluster row is a plain division.
    const uint32_t cm = r / (gm * Nt);
    const uint32_t r1 = r - cm * gm * Nt;
    const uint32_t h = (Mt - cm * gm < gm) ? Mt - cm * gm : gm;
    const uint32_t cn = r1 / (h * gn);
    const uint32_t r2 = r1 - cn * h * gn;
    const uint32_t wd = (Nt - cn * gn < gn) ? Nt - cn * gn : gn;
    const uint32_t i = r2 / wd;
    c.tm = cm * gm + i;
    c.tn = cn * gn + (r2 - i * wd);
  } else {
    c.tm = r / Nt;
    c.tn = r - c.tm * Nt;
  }
  return c;
}

}  // namespace attn_numa
