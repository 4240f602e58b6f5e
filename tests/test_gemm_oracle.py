"""Pins of oracle/gemm.py against what the mathematics fixes, and planted
mistakes that the pins must catch."""
import itertools

import numpy as np
import pytest

from oracle.gemm import cac_tile_table, gemm


# ---- gemm -------------------------------------------------------------------
def test_gemm_brute_force_loops():
    rng = np.random.default_rng(1)
    a = rng.standard_normal((2, 3, 5))
    b = rng.standard_normal((2, 4, 5))
    c = gemm(a, b)
    for l, i, j in itertools.product(range(2), range(3), range(4)):
        assert abs(c[l, i, j] - sum(a[l, i, k] * b[l, j, k] for k in range(5))) < 1e-12


def test_gemm_exact_integers():
    rng = np.random.default_rng(2)
    a = rng.integers(-50, 50, (7, 33))
    b = rng.integers(-50, 50, (9, 33))
    c = gemm(a, b)
    ref = [[sum(int(a[i, k]) * int(b[j, k]) for k in range(33)) for j in range(9)] for i in range(7)]
    assert np.array_equal(c, np.array(ref, dtype=np.float64))


def test_gemm_identity_and_permutation():
    rng = np.random.default_rng(3)
    a = rng.standard_normal((6, 6))
    assert np.array_equal(gemm(a, np.eye(6)), a)       # A I^T = A
    perm = rng.permutation(6)
    p = np.eye(6)[perm]
    assert np.array_equal(gemm(a, p), a[:, perm])      # B = P picks columns


# ---- cac_tile_table -----------------------------------------------------------
SHAPES = [(1, 3, 5, 2, 2, 8), (2, 7, 3, 4, 3, 8), (1, 16, 8, 4, 8, 8), (3, 5, 5, 2, 3, 3),
          (1, 1, 1, 1, 1, 8), (2, 9, 11, 4, 8, 8)]


def pin_bijection(table_fn):
    for mode in range(4):
        for L, Mt, Nt, g1, g2, X in SHAPES:
            t = table_fn(mode, L, Mt, Nt, g1, g2, X)
            seen = {tuple(r) for r in t.tolist()}
            assert len(t) == L * Mt * Nt and len(seen) == len(t), (mode, L, Mt, Nt)
            assert seen == set(itertools.product(range(L), range(Mt), range(Nt)))


def pin_hand_worked_order(table_fn):
    """3 x 5 tiles, 2 x 2 clusters, cluster-major (mode 1, no swizzle): the
    top cluster row is 2 tiles tall (clusters of columns {0,1}, {2,3}, {4}),
    the bottom one 1 tile tall, tiles row-major inside a cluster."""
    want = [(0, 0), (0, 1), (1, 0), (1, 1), (0, 2), (0, 3), (1, 2), (1, 3), (0, 4), (1, 4),
            (2, 0), (2, 1), (2, 2), (2, 3), (2, 4)]
    t = table_fn(1, 1, 3, 5, 2, 2, 8)
    assert [tuple(r[1:]) for r in t.tolist()] == want
    # mode 0: plain row-major
    t0 = table_fn(0, 1, 3, 5, 2, 2, 8)
    assert [tuple(r[1:]) for r in t0.tolist()] == [(i, j) for i in range(3) for j in range(5)]


def pin_clusters_contiguous(table_fn):
    """Cluster-major: the tiles of one cluster are consecutive ids."""
    for L, Mt, Nt, g1, g2, X in SHAPES:
        t = table_fn(1, L, Mt, Nt, g1, g2, X)
        cl = [(l, i // g1, j // g2) for l, i, j in t.tolist()]
        changes = sum(1 for a, b in zip(cl, cl[1:]) if a != b)
        assert changes == len(set(cl)) - 1, (L, Mt, Nt, g1, g2)


def pin_xcd_slices(table_fn):
    """Swizzled modes: XCD x = w mod X receives, in id order, a contiguous
    run of the unswizzled order, and the runs differ in length by at most
    one (a balanced cut), for any X."""
    for base in (0, 1):
        for L, Mt, Nt, g1, g2, X in SHAPES:
            logical = [tuple(r) for r in table_fn(base, L, Mt, Nt, g1, g2, X).tolist()]
            pos = {r: k for k, r in enumerate(logical)}
            t = [tuple(r) for r in table_fn(base | 2, L, Mt, Nt, g1, g2, X).tolist()]
            lengths = []
            for x in range(X):
                idx = [pos[t[w]] for w in range(x, len(t), X)]
                assert idx == list(range(idx[0], idx[0] + len(idx))) if idx else True
                lengths.append(len(idx))
            assert max(lengths) - min(lengths) <= 1


def pin_one_cluster_per_xcd(table_fn):
    """With 32-tile clusters and 32 workgroups in flight per XCD (one per
    CU), the swizzled cluster order gives each XCD whole clusters: tiles
    w, w + X, ... of XCD x fall into ceil(n_x / 32) clusters."""
    L, Mt, Nt, X = 1, 64, 8, 8
    t = table_fn(3, L, Mt, Nt, 4, 8, X)
    for x in range(X):
        ids = list(range(x, len(t), X))
        clusters = {(int(t[w][1]) // 4, int(t[w][2]) // 8) for w in ids}
        assert len(clusters) == -(-len(ids) // 32)


PINS = [pin_bijection, pin_hand_worked_order, pin_clusters_contiguous, pin_xcd_slices,
        pin_one_cluster_per_xcd]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_tile_table_pinned(pin):
    pin(cac_tile_table)


# ---- planted mistakes ------------------------------------------------------------
def _col_major_inside(mode, L, Mt, Nt, g1, g2, X):
    t = cac_tile_table(mode, L, Mt, Nt, g1, g2, X)
    if not (mode & 1):
        return t
    out = t.copy()
    # re-order each cluster's tiles column-major (same set, wrong order)
    i = 0
    while i < len(t):
        key = (t[i][0], t[i][1] // g1, t[i][2] // g2)
        j = i
        while j < len(t) and (t[j][0], t[j][1] // g1, t[j][2] // g2) == key:
            j += 1
        blk = sorted(t[i:j].tolist(), key=lambda r: (r[2], r[1]))
        out[i:j] = blk
        i = j
    return out


def _floor_slices(mode, L, Mt, Nt, g1, g2, X):
    if not (mode & 2):
        return cac_tile_table(mode, L, Mt, Nt, g1, g2, X)
    logical = cac_tile_table(mode & 1, L, Mt, Nt, g1, g2, X)
    W = len(logical)
    per = W // X
    out = np.empty_like(logical)
    for w in range(W):
        x, k = w % X, w // X
        out[w] = logical[min(W - 1, x * per + k)]       # slices of floor(W / X): overlap
    return out


def _no_swizzle(mode, L, Mt, Nt, g1, g2, X):
    return cac_tile_table(mode & 1, L, Mt, Nt, g1, g2, X)


def _transposed_clusters(mode, L, Mt, Nt, g1, g2, X):
    return cac_tile_table(mode, L, Mt, Nt, g2 if g2 <= Mt else g1, g1 if g1 <= Nt else g2, X)


MUTANTS = {
    "tiles column-major inside a cluster": _col_major_inside,
    "slices of floor(W/X) (not a bijection)": _floor_slices,
    "swizzle bit ignored": _no_swizzle,
    "cluster shape transposed": _transposed_clusters,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_tile_table_pins_catch_mutant(name):
    caught = 0
    for pin in PINS:
        try:
            pin(MUTANTS[name])
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin catches: {name}"
