"""Reuse-lag model of the L2 hit rate of the attention forward pass.

"Optimizing Attention on GPUs by Exploiting GPU Architectural NUMA Effects"
(digest page, "What formal guarantee would be desirable", and the commentary
page) notes that the method has no model that predicts the L2 hit rate from
(H_Q, N, d, L2 size, NUM_XCD), so practitioners cannot tell when Swizzled
Head-first matters.  This module is such a model, for this kernel's tiling.

Model (host only; the remap table comes from the library, attn_wg_map, so it
is the order the kernel runs):

* Dispatch: workgroup w runs on XCD w mod X (digest §2 Q1), in increasing w.
  Each XCD runs ``slots`` workgroups at once (its CUs times workgroups per
  CU) and starts the next one in order when one finishes (list scheduling).
* A workgroup streams the K/V tiles of its key range (causal: the keys its
  rows see) in order, one tile per unit of time.
* The XCD's L2 holds ``cap = l2_bytes / tile_bytes`` K/V tiles.  Each running
  workgroup brings at most one new tile per unit of time, so a tile stays at
  least cap / slots units.  A read hits when another workgroup of the same
  ACC (same K/V) on the same XCD started at most cap / slots units earlier
  and reads that tile too.

Predicted hit rate = hits / K/V tile reads.  The model ignores Q, O and lse
traffic, the set associativity of L2 and the Infinity Cache behind it; the
design notes compare it with the measured TCC hit rates per mode.
"""
from __future__ import annotations

import heapq
from collections import defaultdict, deque

import numpy as np

BLOCK_N = 32           # keys per K/V tile of the kernel
L2_BYTES = 4 << 20     # per XCD on MI355X
CUS_PER_XCD = 32


def workgroups_per_cu(d: int) -> int:
    """Forward workgroups resident per CU: one with head dim > 64 (one
    256-thread workgroup fills the CU's registers), two with head dim <= 64
    (padded to 64, two waves per SIMD)."""
    return 2 if d <= 64 else 1


def predict_hit(B: int, H_Q: int, H_KV: int, N: int, d: int, causal: bool,
                mapping: int, num_xcd: int = 8, slots: int | None = None,
                l2_bytes: int = L2_BYTES) -> float:
    """Predicted fraction of K/V tile reads that hit in L2.  ``slots``:
    workgroups an XCD runs at once (default: its CUs x workgroups_per_cu)."""
    if slots is None:
        slots = CUS_PER_XCD * workgroups_per_cu(d)
    from . import attn_block_m, attn_wg_map  # the library's host table
    G = H_Q // H_KV
    block_m = attn_block_m()
    table = attn_wg_map(mapping, B, H_Q, H_KV, N, num_xcd)
    acc = table[:, 0].astype(np.int64) * H_KV + table[:, 1] // G
    if causal:
        keys = np.minimum(N, (table[:, 2].astype(np.int64) + 1) * block_m)
    else:
        keys = np.full(table.shape[0], N, dtype=np.int64)
    tiles = -(-keys // BLOCK_N)
    cap = l2_bytes / (2 * BLOCK_N * d * 2)
    lag_max = cap / slots
    hits = 0
    for x in range(num_xcd):
        running = [0.0] * min(slots, (table.shape[0] - x + num_xcd - 1) // num_xcd)
        heapq.heapify(running)
        recent = defaultdict(deque)  # ACC -> (start, tiles) of its recent workgroups
        for w in range(x, table.shape[0], num_xcd):
            start = heapq.heappop(running)
            length = int(tiles[w])
            heapq.heappush(running, start + length)
            window = recent[int(acc[w])]
            while window and window[0][0] < start - lag_max:
                window.popleft()
            shared = max((n for _, n in window), default=0)
            hits += min(length, shared)
            window.append((start, length))
    return hits / float(tiles.sum())


def best_mapping(B: int, H_Q: int, H_KV: int, N: int, d: int, causal: bool,
                 candidates=(3, 7, 15, 1, 2, 0), **kw) -> int:
    """The candidate mapping with the highest predicted hit rate (ties go to
    the earlier candidate)."""
    scores = [(predict_hit(B, H_Q, H_KV, N, d, causal, m, **kw), -i, m)
              for i, m in enumerate(candidates)]
    return max(scores)[2]
