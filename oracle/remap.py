"""Integer oracle for the workgroup-ID -> (batch, head, row block) remap.

TEST INFRASTRUCTURE ONLY (same rule as oracle/sdpa.py): only tests/,
``__graft_entry__.smoke()`` and bench.py's cpu_baseline leg may use it.  It is
pure Python and shares no code with the C++ header the kernel uses.

Source: "Optimizing Attention on GPUs by Exploiting GPU Architectural NUMA
Effects" (digest page).

* §2 Q1: the hardware dispatcher hands linear workgroup id w to XCD
  ``w mod X`` (chunked round-robin with chunk 1).
* §2 Q2 and §3 Figure 10: an Attention Compute Cluster (ACC) is the set of
  workgroups that read the same K/V, i.e. one head for MHA and one KV group for
  GQA; Swizzled Head-first puts every workgroup of one ACC on one XCD and lets
  each XCD work on one ACC at a time.
* §3 "Method as before/after diff" and §5: the baselines are Naive
  Block-first (all heads of a row block before the next block), Naive
  Head-first (all blocks of a head before the next head, no swizzle) and
  Swizzled Block-first (block-first order behind the chiplet swizzle of §7,
  Figure 3).
* §7 Figure 11 gives Swizzled Head-first for one batch with H_Q a multiple of
  X; §7 "key implementation details" says the pages define no fallback.

Readings (the pages are silent or their printed form is not a bijection):

* Batch is the outermost index of the logical order: L = b·(H_Q·M) + r.
* Block-first decode of r: m = r // H_Q, h = r mod H_Q (heads fastest).
* Head-first decode of r: h = r // M, m = r mod M (blocks fastest).  With
  contiguous GQA groups this order is ACC-major: ACC (b, kv) owns the
  contiguous range [(b·H_Q + kv·G)·M, +G·M).
* Chiplet swizzle: XCD x = w mod X receives the w's congruent to x in
  increasing order, and gets the x-th contiguous slice of the logical order.
  Slices differ in length by at most one when X does not divide W (the
  printed swizzle divides W by X and is a bijection only when X | W):
  sigma(w) = x·floor(W/X) + min(x, W mod X) + floor(w/X).
  This balanced split is the fallback when the number of ACCs is not a
  multiple of X: every XCD still takes the ACCs in one contiguous run, and
  an ACC is split between neighbouring XCDs only where a slice boundary falls
  inside it.

Added (not on the pages): LONGEST_FIRST, a causal-aware order.  Row blocks
are taken last to first (the most visible keys first under a causal mask)
and, head-first, the G query heads of an ACC sharing a row block are
adjacent.  Pinned by properties (bijection; the ACC-per-XCD structure of the
base mode is kept; within each ACC the row blocks run in non-increasing
order with a row block's heads adjacent; with G = 1 it is the base mode with
m reversed).

Added (not on the pages): BALANCED_SPLIT, the fallback made work-balanced
for causal attention (the digest's §7 implementation notes leave the
fallback open; the commentary page raises H_Q = 12 over 8 XCDs without a
remedy).  It changes Swizzled Head-first only (other modes ignore it), and
only on XCDs whose slice holds part of an ACC that a slice boundary splits.
The slices stay as they are, so every XCD keeps the same ACCs; two things
change:
* which units of a split ACC each XCD gets: the ACC's (row block, head)
  units are laid out in folded order (its longest-first list taken first,
  last, second, second-to-last, ...) before the slices cut it, so under a
  causal mask, where row block m carries work linear in m, each XCD's piece
  carries work in proportion to its unit count;
* the order in which such an XCD runs its units: a piece is merged with the
  adjacent whole ACC of the slice (a leading piece with the first whole ACC,
  a trailing piece with the last; with fewer than two whole ACCs everything
  in the slice is one group) and each merged group runs longest first
  (row block descending, then ACC, then head), the list-scheduling order
  that keeps the XCD's longest workgroups from starting last.  Groups run in
  slice order; a group of one whole ACC keeps the order of the other bits.
Pinned by properties (bijection; identical to the mode without the bit on
every XCD without a piece and for every other base mode; each XCD keeps its
ACCs; per-XCD causal work within one row block's work of the mean, where the
plain slices are off by up to 16% at H_Q = 12; merged groups non-increasing
in row block).

Parity status: pinned.  On the domain where the pages print formulas (one
batch, X dividing H_Q, X dividing W) tests/test_remap_oracle.py checks
the dispatch order those formulas produce, and the invariants the
pages state (one ACC per XCD, 16 heads per XCD for Naive Block-first at
H_Q=128, Figure 10's 8-head / 4-XCD example) everywhere else.
"""
from __future__ import annotations

import functools

NBF, NHF, SBF, SHF = 0, 1, 2, 3
MODE_NAMES = {NBF: "naive_block_first", NHF: "naive_head_first",
              SBF: "swizzled_block_first", SHF: "swizzled_head_first"}


def row_blocks(N: int, block_m: int = 128) -> int:
    """Row blocks per head, M = ceil(N / BLOCK_M) (BLOCK_M = 128, §4)."""
    return -(-N // block_m)


def num_workgroups(B: int, H_Q: int, N: int, block_m: int = 128) -> int:
    return B * H_Q * row_blocks(N, block_m)


def xcd_of(w: int, X: int) -> int:
    """XCD that the chunk-1 round-robin dispatcher gives workgroup w."""
    return w % X


def chiplet_swizzle(w: int, W: int, X: int) -> int:
    """Logical index of workgroup w: XCD x owns the x-th contiguous slice."""
    x = w % X
    return x * (W // X) + min(x, W % X) + w // X


def _decode(L: int, H_Q: int, M: int, head_first: bool):
    per_batch = H_Q * M
    b, r = divmod(L, per_batch)
    if head_first:
        h, m = divmod(r, M)
    else:
        m, h = divmod(r, H_Q)
    return b, h, m


# Added to a mode: causal-aware order (not on the pages).  Row blocks are
# taken last to first, i.e. longest first under a causal mask, and in the
# head-first order an ACC's G query heads that share a row block are adjacent
# (ACC, then row block, then head within the KV group).
LONGEST_FIRST = 4


# Added to a mode: work-balanced fallback for Swizzled Head-first (not on
# the pages): an ACC split between XCDs takes its units in folded order.
BALANCED_SPLIT = 8


def slice_starts(W: int, X: int):
    """First logical index of each XCD's slice (and W at the end)."""
    starts = [0]
    for x in range(X):
        starts.append(starts[-1] + W // X + (1 if x < W % X else 0))
    return starts


def _slice_of(P: int, starts) -> int:
    x = 0
    while starts[x + 1] <= P:
        x += 1
    return x


def acc_is_split(a: int, G: int, M: int, W: int, X: int) -> bool:
    """Whether ACC a (logical range [a*G*M, (a+1)*G*M)) meets two slices."""
    starts = slice_starts(W, X)
    return _slice_of(a * G * M, starts) != _slice_of((a + 1) * G * M - 1, starts)


def folded(units):
    """First, last, second, second-to-last, ... of a list."""
    out, i, j = [], 0, len(units) - 1
    while i <= j:
        out.append(units[i])
        if i != j:
            out.append(units[j])
        i, j = i + 1, j - 1
    return out


@functools.lru_cache(maxsize=16)
def _balanced_table(B: int, H_Q: int, M: int, X: int, G: int, longest_first: bool):
    """(b, h, m) of every workgroup id under SHF + BALANCED_SPLIT, built by
    listing: the ACC-major order with split ACCs folded, cut into the XCD
    slices, each slice's ACC parts grouped and the groups with a piece sorted
    longest first, the k-th unit of XCD x going to id x + k X."""
    H_KV = H_Q // G
    U = G * M
    W = B * H_Q * M
    starts = slice_starts(W, X)
    seq = []
    for a in range(B * H_KV):
        b, kv = divmod(a, H_KV)
        if longest_first:
            units = [(M - 1 - md, kv * G + hg) for md in range(M) for hg in range(G)]
        else:
            units = [(m, kv * G + hg) for hg in range(G) for m in range(M)]
        if acc_is_split(a, G, M, W, X):
            units = folded([(M - 1 - md, kv * G + hg) for md in range(M) for hg in range(G)])
        seq += [(a, b, h, m) for m, h in units]
    table = [None] * W
    for x in range(X):
        part_list = []                       # runs of one ACC inside the slice
        for item in seq[starts[x]:starts[x + 1]]:
            if part_list and part_list[-1][0][0] == item[0]:
                part_list[-1].append(item)
            else:
                part_list.append([item])
        whole = [i for i, p in enumerate(part_list) if len(p) == U]
        has_piece = len(whole) < len(part_list)
        if not has_piece:
            groups = [[i] for i in range(len(part_list))]
        elif len(whole) <= 1:
            groups = [list(range(len(part_list)))]
        else:
            first, last = whole[0], whole[-1]
            groups = ([list(range(0, first + 1))] + [[i] for i in range(first + 1, last)]
                      + [list(range(last, len(part_list)))])
        order = []
        for g in groups:
            items = [it for i in g for it in part_list[i]]
            if any(len(part_list[i]) < U for i in g):
                items = sorted(items, key=lambda it: (-it[3], it[0], it[2]))
            order += items
        for k, (_, b, h, m) in enumerate(order):
            table[x + k * X] = (b, h, m)
    return tuple(table)


def wg_map(mode: int, w: int, B: int, H_Q: int, N: int, X: int,
           block_m: int = 128, G: int = 1):
    """(b, h_q, m) computed by linear workgroup id ``w`` under ``mode``
    (0..3, optionally + LONGEST_FIRST and/or BALANCED_SPLIT); G = query heads
    per KV group."""
    M = row_blocks(N, block_m)
    W = B * H_Q * M
    if not 0 <= w < W:
        raise ValueError("workgroup id out of range")
    if not 0 <= mode <= 15 or H_Q % G:
        raise ValueError("unknown mapping mode or G")
    base, longest_first = mode & 3, bool(mode & LONGEST_FIRST)
    L = chiplet_swizzle(w, W, X) if base in (SBF, SHF) else w
    head_first = base in (NHF, SHF)
    if base == SHF and mode & BALANCED_SPLIT:
        return _balanced_table(B, H_Q, M, X, G, longest_first)[w]
    if longest_first and head_first:
        b, r = divmod(L, H_Q * M)
        acc, s = divmod(r, G * M)
        m, hg = divmod(s, G)
        h = acc * G + hg
    else:
        b, h, m = _decode(L, H_Q, M, head_first)
    if longest_first:
        m = M - 1 - m
    return b, h, m


def wg_table(mode: int, B: int, H_Q: int, N: int, X: int, block_m: int = 128,
             G: int = 1):
    """List of (b, h, m) for w = 0..W-1."""
    W = num_workgroups(B, H_Q, N, block_m)
    return [wg_map(mode, w, B, H_Q, N, X, block_m, G) for w in range(W)]
