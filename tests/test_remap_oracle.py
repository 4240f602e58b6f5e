"""The integer remap oracle against what the pages state and show (CPU).

"Optimizing Attention on GPUs by Exploiting GPU Architectural NUMA Effects"
(digest page):
* §2 Q1: the dispatcher hands workgroup w to XCD w mod X.
* §2 Q2 and §6 step 5: Swizzled Head-first gives one XCD a whole ACC (every
  row block of one head) before it moves to the next, and gives each XCD its
  own run of consecutive heads; §3 Figure 10 shows it for 8 heads, 128 row
  blocks and 4 XCDs (golden fixture).
* §7 Figure 3: the chiplet swizzle hands each XCD one contiguous run of the
  logical workgroup order.
* §4 "6 minimum checks" item 3: Naive Block-first puts 16 heads on each XCD
  at H_Q = 128 (golden fixture).
These are checked as properties of the dispatch order (what the k-th
workgroup each XCD receives computes), not by re-typing the printed code.
"""
import os
import random
from collections import defaultdict

import pytest

import oracle
from oracle import NBF, NHF, SBF, SHF

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# (B, H_Q, H_KV, N) of every workload the forward pass is measured on.
CONFIGS = [
    (1, 8, 8, 1024),
    (1, 128, 128, 8192), (1, 128, 128, 32768), (1, 128, 128, 131072),
    (1, 64, 8, 8192), (1, 64, 8, 32768), (1, 64, 8, 131072),
    (2, 32, 4, 32768), (2, 12, 12, 32768), (1, 12, 12, 32768),
]


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    return rows


def _random_shapes(n, seed=0):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        H_KV = rng.randint(1, 10)
        G = rng.randint(1, 4)
        B = rng.randint(1, 4)
        M = rng.randint(1, 20)
        N = M * 128 - rng.choice([0, 0, 1, 64, 127])
        X = rng.choice([1, 2, 4, 8])
        out.append((B, H_KV * G, H_KV, max(N, 1), X))
    return out


@pytest.mark.parametrize("mode", [NBF, NHF, SBF, SHF])
def test_every_mode_is_a_bijection(mode):
    shapes = [(B, H_Q, H_KV, N, 8) for B, H_Q, H_KV, N in CONFIGS]
    shapes += _random_shapes(200)
    for B, H_Q, H_KV, N, X in shapes:
        M = oracle.row_blocks(N)
        tab = oracle.wg_table(mode, B, H_Q, N, X)
        assert len(tab) == B * H_Q * M
        assert len(set(tab)) == len(tab), (mode, B, H_Q, N, X)
        for b, h, m in tab:
            assert 0 <= b < B and 0 <= h < H_Q and 0 <= m < M


def _per_xcd_sequence(mode, B, H_Q, N, X, G=1):
    """Per XCD, what its k-th workgroup (ids x, x + X, x + 2X, ...) computes."""
    W = oracle.num_workgroups(B, H_Q, N)
    seq = defaultdict(list)
    for w in range(W):
        seq[oracle.xcd_of(w, X)].append(oracle.wg_map(mode, w, B, H_Q, N, X, G=G))
    return seq


def test_shf_dispatch_order_single_batch():
    """One batch, X | H_Q: XCD x receives heads x*H_Q/X .. (x+1)*H_Q/X - 1,
    one head at a time (a whole ACC before the next), each head's row blocks
    in order, and no other XCD receives any of them."""
    for H_Q, M, X in [(128, 64, 8), (16, 8, 8), (64, 3, 8), (8, 128, 4),
                      (128, 1024, 8), (24, 5, 4), (6, 7, 2), (5, 9, 1)]:
        seq = _per_xcd_sequence(SHF, 1, H_Q, M * 128, X)
        hpx = H_Q // X
        for x in range(X):
            expect = [(0, h, m) for h in range(x * hpx, (x + 1) * hpx) for m in range(M)]
            assert seq[x] == expect, (H_Q, M, X, x)


def test_sbf_dispatch_order_is_contiguous_runs_of_block_first():
    """X | W: XCD x receives the x-th contiguous run of W/X workgroups of the
    block-first order (batch outermost, then row block, heads fastest)."""
    for B, H_Q, M, X in [(1, 128, 64, 8), (2, 16, 8, 8), (1, 12, 2, 8),
                         (3, 4, 2, 4), (1, 8, 128, 4)]:
        W = B * H_Q * M
        assert W % X == 0
        order = [(b, h, m) for b in range(B) for m in range(M) for h in range(H_Q)]
        seq = _per_xcd_sequence(SBF, B, H_Q, M * 128, X)
        n = W // X
        for x in range(X):
            assert seq[x] == order[x * n:(x + 1) * n], (B, H_Q, M, X, x)


def _acc(b, h, H_Q, H_KV):
    return b * H_KV + h // (H_Q // H_KV)


def _xcd_runs(mode, B, H_Q, H_KV, N, X):
    """Per XCD: the ACC of each workgroup in dispatch order."""
    W = oracle.num_workgroups(B, H_Q, N)
    per = defaultdict(list)
    for w in range(W):
        b, h, _ = oracle.wg_map(mode, w, B, H_Q, N, X)
        per[oracle.xcd_of(w, X)].append(_acc(b, h, H_Q, H_KV))
    return per


def test_shf_puts_each_acc_on_one_xcd_one_at_a_time():
    shapes = [(B, H_Q, H_KV, N, 8) for B, H_Q, H_KV, N in CONFIGS]
    shapes += [s for s in _random_shapes(300, seed=1)]
    checked = 0
    for B, H_Q, H_KV, N, X in shapes:
        if (B * H_KV) % X:
            continue
        checked += 1
        per = _xcd_runs(SHF, B, H_Q, H_KV, N, X)
        owner = {}
        for x, accs in per.items():
            assert accs == sorted(accs), "an XCD must finish one ACC before the next"
            assert len(set(accs)) == B * H_KV // X
            for a in set(accs):
                assert owner.setdefault(a, x) == x, "ACC split over XCDs"
        assert len(owner) == B * H_KV
    assert checked > 30


def test_fallback_is_balanced_and_contiguous():
    shapes = [(1, 12, 12, 32768, 8), (1, 32, 4, 32768, 8), (1, 8, 1, 8192, 8),
              (3, 5, 5, 1000, 8), (1, 2, 1, 300, 8)]
    shapes += [s for s in _random_shapes(300, seed=2)]
    checked = 0
    for B, H_Q, H_KV, N, X in shapes:
        if (B * H_KV) % X == 0:
            continue
        checked += 1
        W = oracle.num_workgroups(B, H_Q, N)
        per = _xcd_runs(SHF, B, H_Q, H_KV, N, X)
        sizes = [len(per.get(x, [])) for x in range(X)]
        assert max(sizes) - min(sizes) <= 1
        U = (H_Q // H_KV) * oracle.row_blocks(N)
        slice_len = W // X
        spans = defaultdict(set)
        for x, accs in per.items():
            assert accs == sorted(accs)
            for a in accs:
                spans[a].add(x)
        for a, xs in spans.items():
            xs = sorted(xs)
            assert xs == list(range(xs[0], xs[-1] + 1)), "ACC on non-adjacent XCDs"
            if slice_len:
                assert len(xs) <= -(-U // slice_len) + 1
    assert checked > 30


def test_fallback_c4_prime_split():
    """B=1, H=12, X=8: 12 ACCs of 256 blocks over 8 slices of 384 blocks:
    8 ACCs stay whole and 4 are split over two XCDs."""
    per = _xcd_runs(SHF, 1, 12, 12, 32768, 8)
    spans = defaultdict(set)
    for x, accs in per.items():
        for a in accs:
            spans[a].add(x)
    n_split = sum(1 for xs in spans.values() if len(xs) == 2)
    assert n_split == 4 and all(len(xs) <= 2 for xs in spans.values())


def test_naive_block_first_16_heads_per_xcd_golden():
    golden = _read_golden("nbf_h128_heads_per_xcd.txt")
    for N in (128, 1024, 131072):
        per = _xcd_runs(NBF, 1, 128, 128, N, 8)
        got = sorted((x, len(set(a))) for x, a in per.items())
        assert [list(t) for t in got] == golden


def test_naive_head_first_stripes_a_head_over_xcds():
    for B, H_Q, N, X in [(1, 128, 131072, 8), (1, 8, 1024, 8), (1, 4, 384, 8),
                         (2, 3, 640, 4)]:
        M = oracle.row_blocks(N)
        W = B * H_Q * M
        seen = defaultdict(set)
        for w in range(W):
            b, h, _ = oracle.wg_map(NHF, w, B, H_Q, N, X)
            seen[(b, h)].add(oracle.xcd_of(w, X))
        assert all(len(s) == min(X, M) for s in seen.values())


def test_figure10_worked_example_golden():
    golden = _read_golden("fig10_shf_x4_h8_m128.txt")
    N = 128 * 128
    count = defaultdict(lambda: defaultdict(int))
    for w in range(8 * 128):
        b, h, m = oracle.wg_map(SHF, w, 1, 8, N, 4)
        count[h][oracle.xcd_of(w, 4)] += 1
    got = []
    for h in range(8):
        (x, c), = count[h].items()
        got.append([h, x, c])
    assert got == golden


def test_batch_outer_reading_keeps_each_batch_whole_per_xcd_run():
    """With B > 1 the oracle puts the batch outermost (the printed per-batch
    id is not a bijection for B = 2); under SHF with X | H_Q every XCD then
    serves batch 0's heads before batch 1's, and each (batch, head) whole."""
    B, H_Q, M, X = 2, 16, 8, 8
    seq = _per_xcd_sequence(SHF, B, H_Q, M * 128, X)
    for x, items in seq.items():
        assert [b for b, _, _ in items] == sorted(b for b, _, _ in items)
        heads = defaultdict(set)
        for b, h, m in items:
            heads[(b, h)].add(m)
        assert all(ms == set(range(M)) for ms in heads.values())


# ---- LONGEST_FIRST (causal-aware order; not on the pages) -------------------
def _lf_shapes():
    shapes = [(1, 8, 8, 1024 * 8, 8), (1, 64, 8, 16384, 8), (2, 32, 4, 8192, 8),
              (1, 12, 12, 8192, 8), (1, 8, 1, 4096, 8), (3, 6, 2, 1000, 4)]
    return shapes + list(_random_shapes(60, seed=7))


@pytest.mark.parametrize("base", [NBF, NHF, SBF, SHF])
def test_longest_first_is_a_bijection(base):
    for B, H_Q, H_KV, N, X in _lf_shapes():
        G = H_Q // H_KV
        tab = oracle.wg_table(base | oracle.LONGEST_FIRST, B, H_Q, N, X, G=G)
        assert len(set(tab)) == len(tab) == oracle.num_workgroups(B, H_Q, N)


@pytest.mark.parametrize("base", [NBF, NHF, SBF, SHF])
def test_longest_first_with_one_head_per_acc_reverses_row_blocks(base):
    for B, H_Q, H_KV, N, X in _lf_shapes():
        M = oracle.row_blocks(N)
        a = oracle.wg_table(base, B, H_Q, N, X, G=1)
        b = oracle.wg_table(base | oracle.LONGEST_FIRST, B, H_Q, N, X, G=1)
        assert b == [(bb, h, M - 1 - m) for bb, h, m in a]


def test_longest_first_keeps_acc_per_xcd_and_orders_each_acc():
    """SHF + LONGEST_FIRST: the XCD that owns each workgroup is the one SHF
    gives it (same ACC slices); within an ACC the workgroups an XCD runs go
    from the last row block to the first, each row block's G heads adjacent."""
    for B, H_Q, H_KV, N, X in _lf_shapes():
        G = H_Q // H_KV
        M = oracle.row_blocks(N)
        W = oracle.num_workgroups(B, H_Q, N)
        lf = SHF | oracle.LONGEST_FIRST
        acc_of = lambda b, h: b * H_KV + h // G
        owner_shf = defaultdict(set)
        for w in range(W):
            b, h, m = oracle.wg_map(SHF, w, B, H_Q, N, X)
            owner_shf[acc_of(b, h)].add(w % X)
        seq = defaultdict(list)                   # per XCD, in dispatch order
        for w in range(W):
            b, h, m = oracle.wg_map(lf, w, B, H_Q, N, X, G=G)
            seq[w % X].append((acc_of(b, h), m, h))
        owner_lf = defaultdict(set)
        for x, items in seq.items():
            for a, m, h in items:
                owner_lf[a].add(x)
            by_acc = defaultdict(list)
            for a, m, h in items:
                by_acc[a].append((m, h))
            for a, ms in by_acc.items():
                assert all(ms[i][0] >= ms[i + 1][0] for i in range(len(ms) - 1)), (a, x)
                # a row block's heads are adjacent within the ACC's run
                seen = set()
                for i, (m, h) in enumerate(ms):
                    if i and ms[i - 1][0] != m:
                        assert m not in seen
                        seen.add(ms[i - 1][0])
        if (B * H_KV) % X == 0:
            assert all(len(s) == 1 for s in owner_lf.values())
        assert {a: len(s) for a, s in owner_lf.items()} == {a: len(s) for a, s in owner_shf.items()}


def test_longest_first_rejects_bad_mode():
    with pytest.raises(ValueError):
        oracle.wg_map(-1, 0, 1, 8, 1024, 8)


# ---- BALANCED_SPLIT (work-balanced fallback; not on the pages) -------------
BAL = oracle.BALANCED_SPLIT


def _causal_unit_work(m, N, bm):
    """(query, key) pairs of row block m under a top-left causal mask."""
    lo, hi = m * bm, min((m + 1) * bm, N)
    return (hi * (hi + 1) - lo * (lo + 1)) // 2


def _bal_shapes(n=150, seed=11):
    rng = random.Random(seed)
    out = [(1, 12, 12, 32768, 8, 256), (2, 12, 12, 32768, 8, 256), (1, 32, 4, 32768, 8, 256),
           (1, 6, 2, 4096, 8, 256), (3, 5, 5, 1000, 8, 128), (1, 8, 1, 8192, 8, 256)]
    for _ in range(n):
        H_KV, G, B, M = rng.randint(1, 12), rng.randint(1, 4), rng.randint(1, 3), rng.randint(1, 30)
        bm = rng.choice([128, 256])
        N = max(M * bm - rng.choice([0, 0, 1, 77]), 1)
        out.append((B, H_KV * G, H_KV, N, rng.choice([2, 4, 8]), bm))
    return out


def test_balanced_split_is_a_bijection_in_every_mode():
    for B, H_Q, H_KV, N, X, bm in _bal_shapes(60):
        G = H_Q // H_KV
        for mode in range(8, 16):
            tab = oracle.wg_table(mode, B, H_Q, N, X, block_m=bm, G=G)
            assert len(set(tab)) == len(tab) == oracle.num_workgroups(B, H_Q, N, bm), mode


def _xcd_has_piece(B, H_Q, H_KV, N, X, bm, x):
    """Whether XCD x's slice holds part of an ACC that a slice boundary splits."""
    G = H_Q // H_KV
    M = oracle.row_blocks(N, bm)
    U = G * M
    W = B * H_Q * M
    starts = oracle.slice_starts(W, X)
    lo, hi = starts[x], starts[x + 1]
    return any(oracle.acc_is_split(a, G, M, W, X) for a in range(lo // U, (hi - 1) // U + 1)) if hi > lo else False


def test_balanced_split_changes_only_xcds_holding_a_split_piece():
    """Other base modes ignore the bit; under SHF every XCD whose slice holds
    no piece of a split ACC runs exactly what it runs without the bit."""
    for B, H_Q, H_KV, N, X, bm in _bal_shapes(80, seed=12):
        G = H_Q // H_KV
        for base in (0, 1, 2, 4, 5, 6):
            assert (oracle.wg_table(base | BAL, B, H_Q, N, X, bm, G)
                    == oracle.wg_table(base, B, H_Q, N, X, bm, G))
        for lf in (0, oracle.LONGEST_FIRST):
            plain = oracle.wg_table(SHF | lf, B, H_Q, N, X, bm, G)
            bal = oracle.wg_table(SHF | lf | BAL, B, H_Q, N, X, bm, G)
            for w in range(len(plain)):
                if not _xcd_has_piece(B, H_Q, H_KV, N, X, bm, w % X):
                    assert bal[w] == plain[w]


def test_balanced_split_keeps_each_acc_on_its_xcds():
    """Every XCD keeps the ACCs (and unit counts per ACC) it has under plain
    SHF; an ACC spans at most 2 XCDs when there are at least X ACCs."""
    for B, H_Q, H_KV, N, X, bm in _bal_shapes(80, seed=13):
        G = H_Q // H_KV
        per_plain, per_bal = defaultdict(list), defaultdict(list)
        for w, ((b, h, _), (b2, h2, _)) in enumerate(zip(
                oracle.wg_table(SHF | 4, B, H_Q, N, X, bm, G),
                oracle.wg_table(SHF | 4 | BAL, B, H_Q, N, X, bm, G))):
            per_plain[w % X].append(_acc(b, h, H_Q, H_KV))
            per_bal[w % X].append(_acc(b2, h2, H_Q, H_KV))
        for x in per_plain:
            assert sorted(per_bal[x]) == sorted(per_plain[x])
        if B * H_KV >= X:
            spans = defaultdict(set)
            for x, accs in per_bal.items():
                for a in accs:
                    spans[a].add(x)
            assert all(len(s) <= 2 for s in spans.values())


def test_balanced_split_runs_merged_groups_longest_first():
    """On an XCD that holds a piece, the units run in non-increasing row
    block within each merged group, and at most two ACCs are interleaved at
    any point (a piece only merges with its neighbouring whole ACC)."""
    for B, H_Q, H_KV, N, X, bm in _bal_shapes(80, seed=15):
        G = H_Q // H_KV
        M = oracle.row_blocks(N, bm)
        tab = oracle.wg_table(SHF | 4 | BAL, B, H_Q, N, X, bm, G)
        for x in range(X):
            if not _xcd_has_piece(B, H_Q, H_KV, N, X, bm, x):
                continue
            seq = [tab[w] for w in range(x, len(tab), X)]
            accs = sorted({_acc(b, h, H_Q, H_KV) for b, h, _ in seq})
            # count how many ACCs have started but not finished at each point
            first = {a: min(i for i, (b, h, _) in enumerate(seq) if _acc(b, h, H_Q, H_KV) == a) for a in accs}
            last = {a: max(i for i, (b, h, _) in enumerate(seq) if _acc(b, h, H_Q, H_KV) == a) for a in accs}
            whole = sum(1 for a in accs if sum(1 for b, h, _ in seq if _acc(b, h, H_Q, H_KV) == a) == G * M)
            live = max(sum(1 for a in accs if first[a] <= i <= last[a]) for i in range(len(seq)))
            assert live <= (3 if whole <= 1 else 2), (B, H_Q, H_KV, N, X, x)
            # longest first inside every run where ACCs interleave
            for i in range(1, len(seq)):
                a0, a1 = _acc(*seq[i - 1][:2], H_Q, H_KV), _acc(*seq[i][:2], H_Q, H_KV)
                together = first[a1] < last[a0] and first[a0] < last[a1]
                if together:
                    assert seq[i][2] <= seq[i - 1][2], (x, i)


def test_balanced_split_c4_prime_makespan():
    """B=1, H=12, N=32K, 256-row blocks, 8 XCDs of 32 CUs: list scheduling
    of each XCD's workgroups in dispatch order (lengths = visible key tiles)
    finishes within 5% of the ideal (the XCD's work over its CUs) with the
    balanced split; longest first alone leaves 16.5% (the heavy half of a
    split ACC on one XCD)."""
    import heapq
    N, bm = 32768, 256

    def makespan(mode):
        tab = oracle.wg_table(mode, 1, 12, N, 8, bm, 1)
        worst, total = 0, 0
        for x in range(8):
            lengths = [min(N, (m + 1) * bm) // 32 for (_, _, m) in tab[x::8]]
            total += sum(lengths)
            cus = [0] * 32
            for ln in lengths:
                t = heapq.heappop(cus)
                heapq.heappush(cus, t + ln)
            worst = max(worst, max(cus))
        return worst / (total / 8 / 32)
    assert round(makespan(SHF | 4), 3) == 1.165
    assert makespan(SHF | 4 | BAL) <= 1.05


def test_balanced_split_per_xcd_causal_work_within_a_row_block_of_the_mean():
    """Per-XCD causal work (query-key pairs) is within one row block's work
    of the mean when N is a multiple of the row-block height, and within two
    for ragged N (the last row block breaks the linear work of the fold)."""
    worst_exact = worst_ragged = 0.0
    for B, H_Q, H_KV, N, X, bm in _bal_shapes(150, seed=14):
        G = H_Q // H_KV
        M = oracle.row_blocks(N, bm)
        unit_max = max(_causal_unit_work(m, N, bm) for m in range(M))
        work = [0] * X
        for w, (b, h, m) in enumerate(oracle.wg_table(SHF | 4 | BAL, B, H_Q, N, X, bm, G)):
            work[w % X] += _causal_unit_work(m, N, bm)
        mean = sum(work) / X
        dev = max(abs(x - mean) for x in work) / unit_max
        if N % bm == 0:
            worst_exact = max(worst_exact, dev)
        else:
            worst_ragged = max(worst_ragged, dev)
    assert worst_exact <= 1.0 and worst_ragged <= 2.0, (worst_exact, worst_ragged)


def test_balanced_split_c4_prime_numbers():
    """B=1, H=12, N=32K, 256-row blocks, 8 XCDs: plain slices leave the
    heaviest XCD 16.7% above the mean causal work (the piece holding the
    long row blocks of a split ACC); the folded pieces balance it exactly."""
    N, bm = 32768, 256
    for mode, expect in ((SHF | 4, 1.1667), (SHF, 1.1667), (SHF | 4 | BAL, 1.0), (SHF | BAL, 1.0)):
        work = [0] * 8
        for w, (b, h, m) in enumerate(oracle.wg_table(mode, 1, 12, N, 8, bm, 1)):
            work[w % 8] += _causal_unit_work(m, N, bm)
        assert round(max(work) / (sum(work) / 8), 4) == expect, mode


def test_folded_order_small_example():
    assert oracle.folded([0, 1, 2, 3, 4]) == [0, 4, 1, 3, 2]
    assert oracle.folded([0, 1, 2, 3]) == [0, 3, 1, 2]
    assert oracle.folded([]) == []


def test_balanced_split_rejects_bad_mode():
    with pytest.raises(ValueError):
        oracle.wg_map(16, 0, 1, 8, 1024, 8)
