"""Pins of the split-KV oracle (oracle/split.py) to facts fixed outside it.

* The merge of partial results over ANY partition of the keys equals the
  full attention: the definition (oracle.attention, N_q == N_kv) or a
  brute-force loop evaluation (N_q != N_kv, causal bottom-right aligned).
* Brute force with Python loops and math.fsum on tiny shapes, per split.
* Closed forms: Q = 0 gives O_s = mean of the visible V rows of the split
  and lse_s = ln(their count); a split a row cannot see gives (0, -inf).
* Merge identities: one part is returned unchanged; two identical parts
  give the same O and lse + ln 2; -inf parts carry no weight.
* Decode (N_q = 1): causal equals non-causal (the row sees every key).
Each check also runs against planted mistakes (tests below) to show it
catches them.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from oracle import split as split_mod


def brute_partial(q, k, v, causal, kv_begin, kv_end):
    """Loops, no max subtraction, math.fsum; bottom-right causal."""
    B, H_Q, N_q, d = q.shape
    H_KV, N_kv = k.shape[1], k.shape[2]
    G = H_Q // H_KV
    o = np.zeros(q.shape)
    lse = np.full((B, H_Q, N_q), -np.inf)
    for b in range(B):
        for h in range(H_Q):
            g = h // G
            for i in range(N_q):
                keys = [j for j in range(kv_begin, kv_end)
                        if not causal or j <= i + N_kv - N_q]
                if not keys:
                    continue
                s = [math.fsum(float(q[b, h, i, t]) * float(k[b, g, j, t]) for t in range(d))
                     / math.sqrt(d) for j in keys]
                e = [math.exp(x) for x in s]
                z = math.fsum(e)
                for t in range(d):
                    o[b, h, i, t] = math.fsum(e[n] * float(v[b, g, j, t])
                                              for n, j in enumerate(keys)) / z
                lse[b, h, i] = math.log(z)
    return o, lse


def _qkv(rng, B, H_Q, H_KV, N_q, N_kv, d):
    return (rng.standard_normal((B, H_Q, N_q, d)), rng.standard_normal((B, H_KV, N_kv, d)),
            rng.standard_normal((B, H_KV, N_kv, d)))


def _random_partition(rng, N_kv, S):
    """S contiguous ranges covering [0, N_kv); some may be empty."""
    cuts = np.sort(rng.integers(0, N_kv + 1, S - 1))
    bounds = [0, *cuts.tolist(), N_kv]
    return list(zip(bounds[:-1], bounds[1:]))


def _split_then_merge(mod, q, k, v, causal, parts):
    outs = [mod.partial_attention(q, k, v, causal, a, b) for a, b in parts]
    return mod.merge(np.stack([o for o, _ in outs]), np.stack([l for _, l in outs]))


def pin_merge_equals_definition(mod, seed=0):
    rng = np.random.default_rng(seed)
    for B, H_Q, H_KV, N, d, S in [(1, 2, 2, 37, 8, 3), (2, 4, 2, 64, 16, 5), (1, 3, 1, 20, 4, 20)]:
        q, k, v = _qkv(rng, B, H_Q, H_KV, N, N, d)
        for causal in (False, True):
            o_ref, lse_ref = oracle.attention(q, k, v, causal)
            o, lse = _split_then_merge(mod, q, k, v, causal, _random_partition(rng, N, S))
            np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def pin_merge_equals_brute_force_rectangular(mod, seed=1):
    rng = np.random.default_rng(seed)
    for B, H_Q, H_KV, N_q, N_kv, d, S in [(1, 2, 1, 3, 11, 4, 3), (2, 2, 2, 1, 9, 3, 4),
                                           (1, 1, 1, 6, 6, 5, 2), (1, 2, 2, 4, 13, 2, 5)]:
        q, k, v = _qkv(rng, B, H_Q, H_KV, N_q, N_kv, d)
        for causal in (False, True):
            o_ref, lse_ref = brute_partial(q, k, v, causal, 0, N_kv)
            o, lse = _split_then_merge(mod, q, k, v, causal, _random_partition(rng, N_kv, S))
            np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def pin_partial_brute_force(mod, seed=2):
    rng = np.random.default_rng(seed)
    for B, H_Q, H_KV, N_q, N_kv, d in [(1, 2, 1, 5, 9, 3), (2, 2, 2, 7, 7, 4), (1, 1, 1, 1, 12, 2)]:
        q, k, v = _qkv(rng, B, H_Q, H_KV, N_q, N_kv, d)
        for causal in (False, True):
            for a, b in [(0, N_kv), (2, 6), (N_kv - 3, N_kv), (4, 4)]:
                o, lse = mod.partial_attention(q, k, v, causal, a, b)
                o_ref, lse_ref = brute_partial(q, k, v, causal, a, b)
                np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
                assert np.array_equal(np.isinf(lse), np.isinf(lse_ref))
                fin = np.isfinite(lse_ref)
                np.testing.assert_allclose(lse[fin], lse_ref[fin], rtol=0, atol=1e-12)


def pin_closed_forms(mod, seed=3):
    rng = np.random.default_rng(seed)
    N_q, N_kv, d = 4, 10, 3
    q = np.zeros((1, 1, N_q, d))
    k = rng.standard_normal((1, 1, N_kv, d))
    v = rng.standard_normal((1, 1, N_kv, d))
    a, b = 3, 8
    o, lse = mod.partial_attention(q, k, v, True, a, b)
    for i in range(N_q):
        vis = [j for j in range(a, b) if j <= i + N_kv - N_q]
        if vis:
            np.testing.assert_allclose(o[0, 0, i], v[0, 0, vis].mean(axis=0), atol=1e-14)
            assert abs(lse[0, 0, i] - math.log(len(vis))) < 1e-14
        else:
            assert np.all(o[0, 0, i] == 0) and lse[0, 0, i] == -np.inf
    # Decode: the single row sees every key, causal or not.
    q1, k1, v1 = _qkv(rng, 2, 4, 2, 1, 17, 5)
    oc, lc = mod.partial_attention(q1, k1, v1, True, 0, 17)
    on, ln_ = mod.partial_attention(q1, k1, v1, False, 0, 17)
    np.testing.assert_array_equal(oc, on)
    np.testing.assert_array_equal(lc, ln_)


def pin_merge_identities(mod, seed=4):
    rng = np.random.default_rng(seed)
    o1 = rng.standard_normal((2, 3, 5))
    l1 = rng.standard_normal((2, 3))
    o, lse = mod.merge(o1[None], l1[None])
    np.testing.assert_allclose(o, o1, atol=1e-15)
    np.testing.assert_allclose(lse, l1, atol=1e-15)
    o, lse = mod.merge(np.stack([o1, o1]), np.stack([l1, l1]))
    np.testing.assert_allclose(o, o1, atol=1e-14)
    np.testing.assert_allclose(lse, l1 + math.log(2), atol=1e-14)
    o2 = rng.standard_normal((2, 3, 5))
    o, lse = mod.merge(np.stack([o1, o2]), np.stack([l1, np.full((2, 3), -np.inf)]))
    np.testing.assert_allclose(o, o1, atol=1e-15)
    np.testing.assert_allclose(lse, l1, atol=1e-15)
    # Two parts with lse a, b: weights e^a / (e^a + e^b).
    a, b = 0.3, -1.2
    o, lse = mod.merge(np.array([[[1.0]], [[3.0]]]), np.array([[a], [b]]))
    wa = math.exp(a) / (math.exp(a) + math.exp(b))
    assert abs(o[0, 0] - (wa * 1.0 + (1 - wa) * 3.0)) < 1e-15
    assert abs(lse[0] - math.log(math.exp(a) + math.exp(b))) < 1e-15
    o, lse = mod.merge(np.zeros((3, 1, 2)), np.full((3, 1), -np.inf))
    assert np.all(o == 0) and lse[0] == -np.inf


PINS = [pin_merge_equals_definition, pin_merge_equals_brute_force_rectangular,
        pin_partial_brute_force, pin_closed_forms, pin_merge_identities]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_split_oracle_pinned(pin):
    pin(split_mod)


# ---- planted mistakes: each must be caught by at least one pin -------------
class _Mutant:
    """A copy of the split oracle with one function replaced."""

    def __init__(self, **over):
        self.partial_attention = split_mod.partial_attention
        self.merge = split_mod.merge
        self.__dict__.update(over)


def _merge_no_weights(o_parts, lse_parts):          # plain average of the parts
    o, lse = split_mod.merge(o_parts, lse_parts)
    return np.asarray(o_parts).mean(axis=0), lse


def _merge_max_not_logsumexp(o_parts, lse_parts):   # lse = max lse_s
    o, _ = split_mod.merge(o_parts, lse_parts)
    return o, np.asarray(lse_parts).max(axis=0)


def _partial_top_left(q, k, v, causal, a, b):        # causal offset dropped
    N_q = q.shape[2]
    kk, vv = k[:, :, :N_q], v[:, :, :N_q]
    if k.shape[2] == N_q or not causal:
        return split_mod.partial_attention(q, k, v, causal, a, b)
    o, lse = split_mod.partial_attention(q, kk, vv, causal, min(a, N_q), min(b, N_q))
    return o, lse


def _partial_inclusive_end(q, k, v, causal, a, b):   # one key too many
    return split_mod.partial_attention(q, k, v, causal, a, min(b + 1, k.shape[2]))


def _partial_unnormalised(q, k, v, causal, a, b):    # O_s not divided by l_s
    o, lse = split_mod.partial_attention(q, k, v, causal, a, b)
    fin = np.isfinite(lse)
    scale = np.where(fin, np.exp(np.where(fin, lse, 0.0)), 0.0)
    return o * scale[..., None], lse


MUTANTS = {
    "merge without exp weights": _Mutant(merge=_merge_no_weights),
    "merge lse as max": _Mutant(merge=_merge_max_not_logsumexp),
    "causal top-left for N_q != N_kv": _Mutant(partial_attention=_partial_top_left),
    "split end inclusive": _Mutant(partial_attention=_partial_inclusive_end),
    "partial O unnormalised": _Mutant(partial_attention=_partial_unnormalised),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_split_pins_catch_mutant(name):
    mod = MUTANTS[name]
    caught = 0
    for pin in PINS:
        try:
            pin(mod)
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin catches: {name}"
