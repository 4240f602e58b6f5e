"""CPU oracle for the Compute Affinity Cluster (CAC) scheduled GEMM.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no
code with the HIP kernels.

Source: "Optimizing Attention on GPUs by Exploiting GPU Architectural NUMA
Effects", commentary page, the paragraph that generalises the Attention
Compute Cluster to a "Compute Affinity Cluster": the workgroups that share
input data, placed together on one XCD.  For C = A B^T tiled into 256 x 256
output tiles, tile (i, j) reads row panel i of A and column panel j of B; a
block of gm x gn tiles shares gm A panels and gn B panels and is the cluster.
The placement reuses the digest's dispatch rule (§2 Q1: workgroup w runs on
XCD w mod X) and its chiplet swizzle (§7: XCD x takes the x-th contiguous
slice of the logical order), read as balanced slices, as for attention.

* ``gemm(a, b)``: C[l] = A[l] B[l]^T in float64 (the definition; numpy
  matmul).  Parity status: pinned (tests/test_gemm_oracle.py: brute-force
  loops, exact small integers, identity and permutation matrices).
* ``cac_tile_table(mode, L, Mt, Nt, gm, gn, X)``: the (l, tile row, tile
  column) of each workgroup id, built by listing the logical order
  explicitly and cutting it into per-XCD slices.  Parity status: pinned
  (bijection, cluster contiguity, per-XCD contiguity, a hand-worked order).
"""
from __future__ import annotations

import numpy as np


def gemm(a, b) -> np.ndarray:
    """C[l] = A[l] B[l]^T, float64.  a [L, M, K] (or [M, K]), b [L, N, K]
    (or [N, K])."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return a @ np.swapaxes(b, -1, -2)


def _logical_order(mode: int, Mt: int, Nt: int, gm: int, gn: int):
    """Tiles of one batch in the logical order of the mode's bit 0."""
    if not (mode & 1):
        return [(i, j) for i in range(Mt) for j in range(Nt)]
    order = []
    for ci in range(0, Mt, gm):            # cluster rows, top to bottom
        for cj in range(0, Nt, gn):        # clusters of the row, left to right
            for i in range(ci, min(Mt, ci + gm)):      # tiles inside: row-major
                for j in range(cj, min(Nt, cj + gn)):
                    order.append((i, j))
    return order


def cac_tile_table(mode: int, L: int, Mt: int, Nt: int, gm: int, gn: int,
                   X: int) -> np.ndarray:
    """int64 [W, 3]: row w = (l, tile row, tile column) of workgroup id w."""
    per = _logical_order(mode, Mt, Nt, gm, gn)
    logical = [(l, i, j) for l in range(L) for (i, j) in per]
    W = len(logical)
    if not (mode & 2):
        return np.array(logical, dtype=np.int64).reshape(W, 3)
    # XCD x receives ids x, x + X, x + 2X, ... in that order; it works through
    # the x-th slice of the logical order.  Slices are as equal as possible,
    # the first W mod X one longer.
    base, extra = divmod(W, X)
    starts, pos = [], 0
    for x in range(X):
        starts.append(pos)
        pos += base + (1 if x < extra else 0)
    out = np.empty((W, 3), dtype=np.int64)
    for w in range(W):
        x, k = w % X, w // X
        out[w] = logical[starts[x] + k]
    return out
