"""Pins of the backward oracle (oracle/backward.py) to facts fixed outside it.

* Central finite differences of the forward oracle: for L = sum(dO * O),
  dL/dx for sampled elements x of Q, K and V (float64, h = 1e-6).
* torch's float64 autograd through the math-backend SDPA (a library routine),
  with and without is_causal, with GQA by repeating K/V.
* Closed forms: every V row equal makes O independent of P, so dQ = dK = 0
  and dV = Pᵀ dO sums dO over the queries that see each key; dO = 0 gives
  zero gradients.
* GQA: a KV head's dK, dV equal the sums of the MHA gradients of its query
  heads with K/V repeated.
Planted mistakes in copies of the oracle are each caught (tests below).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch
from torch.nn.attention import SDPBackend, sdpa_kernel

import oracle
from oracle import backward as bwd_mod


def _rand(seed, *shapes):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(s) for s in shapes]


def pin_finite_differences(fn, seed=0):
    for B, H_Q, H_KV, N, d, causal in [(1, 2, 1, 5, 3, True), (1, 1, 1, 6, 4, False),
                                       (2, 2, 2, 4, 2, True)]:
        q, k, v, do = _rand(seed, (B, H_Q, N, d), (B, H_KV, N, d), (B, H_KV, N, d), (B, H_Q, N, d))
        dq, dk, dv = fn(q, k, v, do, causal)
        loss = lambda q_, k_, v_: float((oracle.attention(q_, k_, v_, causal)[0] * do).sum())
        rng = np.random.default_rng(seed + 1)
        h = 1e-6
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            for _ in range(6):
                idx = tuple(int(rng.integers(n)) for n in x.shape)
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
                args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
                num = (loss(*args_p) - loss(*args_m)) / (2 * h)
                assert abs(num - g[idx]) < 1e-6, (name, idx, num, g[idx])


def pin_torch_autograd(fn, seed=1):
    for B, H_Q, H_KV, N, d, causal in [(1, 4, 2, 17, 8, True), (2, 2, 2, 9, 5, False)]:
        q, k, v, do = _rand(seed, (B, H_Q, N, d), (B, H_KV, N, d), (B, H_KV, N, d), (B, H_Q, N, d))
        G = H_Q // H_KV
        tq = torch.tensor(q, requires_grad=True)
        tk = torch.tensor(k, requires_grad=True)
        tv = torch.tensor(v, requires_grad=True)
        with sdpa_kernel(SDPBackend.MATH):
            o = torch.nn.functional.scaled_dot_product_attention(
                tq, tk.repeat_interleave(G, 1), tv.repeat_interleave(G, 1), is_causal=causal)
        (o * torch.tensor(do)).sum().backward()
        dq, dk, dv = fn(q, k, v, do, causal)
        np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11, rtol=0)
        np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11, rtol=0)
        np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11, rtol=0)


def pin_closed_forms(fn, seed=2):
    B, H, N, d = 1, 2, 7, 4
    q, k, do = _rand(seed, (B, H, N, d), (B, H, N, d), (B, H, N, d))
    row = np.random.default_rng(seed).standard_normal(d)
    v = np.broadcast_to(row, (B, H, N, d)).copy()
    for causal in (False, True):
        dq, dk, dv = fn(q, k, v, do, causal)
        assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
        # column sums: sum_j dV[j] = sum_i dO[i] (the rows of P sum to 1)
        np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)
    # Q = 0: causal row i is uniform over keys 0..i, so dV[j] = sum_{i>=j} dO[i] / (i+1)
    # (non-causal: every row uniform over all N keys, dV[j] = sum_i dO[i] / N).
    for causal in (False, True):
        _, _, dv0 = fn(np.zeros_like(q), k, v, do, causal)
        for j in range(N):
            rows = range(j, N) if causal else range(N)
            want = sum(do[:, :, i] / ((i + 1) if causal else N) for i in rows)
            np.testing.assert_allclose(dv0[:, :, j], want, atol=1e-12)
    zq, zk, zv = fn(q, k, v, np.zeros_like(do), True)
    assert not zq.any() and not zk.any() and not zv.any()


def pin_gqa_is_summed_mha(fn, seed=3):
    B, H_Q, H_KV, N, d = 1, 6, 2, 8, 3
    q, k, v, do = _rand(seed, (B, H_Q, N, d), (B, H_KV, N, d), (B, H_KV, N, d), (B, H_Q, N, d))
    G = H_Q // H_KV
    dq, dk, dv = fn(q, k, v, do, True)
    mq, mk, mv = fn(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), do, True)
    np.testing.assert_allclose(dq, mq, atol=1e-13)
    np.testing.assert_allclose(dk, mk.reshape(B, H_KV, G, N, d).sum(axis=2), atol=1e-13)
    np.testing.assert_allclose(dv, mv.reshape(B, H_KV, G, N, d).sum(axis=2), atol=1e-13)


PINS = [pin_finite_differences, pin_torch_autograd, pin_closed_forms, pin_gqa_is_summed_mha]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pinned(pin):
    pin(bwd_mod.attention_backward)


# ---- planted mistakes ------------------------------------------------------
def _wrap(transform):
    def fn(q, k, v, do, causal):
        return transform(*bwd_mod.attention_backward(q, k, v, do, causal), q, k, v, do, causal)
    return fn


def _no_softmax_jacobian(q, k, v, do, causal):          # dS = P * dP (D term dropped)
    B, H_Q, N, d = q.shape
    H_KV = k.shape[1]
    G = H_Q // H_KV
    dq = np.zeros_like(q)
    for b in range(B):
        for h in range(H_Q):
            g = h // G
            s = q[b, h] @ k[b, g].T / np.sqrt(d)
            if causal:
                s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
            p = np.exp(s - s.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            dq[b, h] = (p * (do[b, h] @ v[b, g].T)) @ k[b, g] / np.sqrt(d)
    _, dk, dv = bwd_mod.attention_backward(q, k, v, do, causal)
    return dq, dk, dv


MUTANTS = {
    "dQ without the 1/sqrt(d) scale": _wrap(lambda dq, dk, dv, q, k, v, do, c: (dq * np.sqrt(q.shape[3]), dk, dv)),
    "dK transposed roles (uses dV)": _wrap(lambda dq, dk, dv, *a: (dq, dv, dv)),
    "dV not summed over the GQA group (last head only)": None,
    "softmax Jacobian term dropped": _no_softmax_jacobian,
    "causal mask ignored": lambda q, k, v, do, causal: bwd_mod.attention_backward(q, k, v, do, False),
}


def _gqa_last_head_only(q, k, v, do, causal):
    B, H_Q, N, d = q.shape
    H_KV = k.shape[1]
    G = H_Q // H_KV
    dq, dk, dv = bwd_mod.attention_backward(q, k, v, do, causal)
    sel = [g * G + G - 1 for g in range(H_KV)]
    _, mk, mv = bwd_mod.attention_backward(q[:, sel], k, v, do[:, sel], causal)
    return dq, mk, mv


MUTANTS["dV not summed over the GQA group (last head only)"] = _gqa_last_head_only


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_pins_catch_mutant(name):
    caught = 0
    for pin in PINS:
        try:
            pin(MUTANTS[name])
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin catches: {name}"


# ---- sampled forms (long sequences) against the full oracle -----------------
@pytest.mark.parametrize("causal", [False, True])
def test_sampled_forms_equal_full_backward(causal):
    """dQ of chosen rows and dK/dV of chosen keys, computed one row or key
    at a time, equal the full oracle on a GQA shape (2 query heads per KV
    head), whatever the row chunk."""
    rng = np.random.default_rng(11)
    B, H_Q, H_KV, N, d = 1, 4, 2, 70, 16
    q = rng.standard_normal((B, H_Q, N, d))
    k = rng.standard_normal((B, H_KV, N, d))
    v = rng.standard_normal((B, H_KV, N, d))
    do = rng.standard_normal((B, H_Q, N, d))
    dq, dk, dv = bwd_mod.attention_backward(q, k, v, do, causal)
    rows = np.array([0, 1, 17, 68, 69])
    for h in range(H_Q):
        g = h // (H_Q // H_KV)
        got = bwd_mod.backward_query_rows(q[0, h, rows], k[0, g], v[0, g], do[0, h, rows], rows, causal)
        np.testing.assert_allclose(got, dq[0, h, rows], rtol=1e-12, atol=1e-12)
    keys = np.array([0, 5, 33, 69])
    for g in range(H_KV):
        heads = [g * 2, g * 2 + 1]
        for chunk in (7, 512):
            gk, gv = bwd_mod.backward_key_rows(q[0, heads], k[0, g], v[0, g], do[0, heads], keys,
                                               causal, row_chunk=chunk)
            np.testing.assert_allclose(gk, dk[0, g, keys], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(gv, dv[0, g, keys], rtol=1e-12, atol=1e-12)


# ---- K = 0 closed form (full sequence lengths) against the full oracle ------
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 2, 300, 16), (4, 2, 257, 8), (1, 1, 1, 8), (2, 1, 513, 32)],
                         ids=str)
def test_zero_key_closed_form_equals_full_backward(shape, causal):
    """backward_zero_keys (uniform attention over the visible keys, suffix
    sums taken block by block) equals the general oracle with K = 0 on every
    key, for ragged lengths and GQA, whatever the block; dQ is then zero."""
    H_Q, H_KV, N, d = shape
    rng = np.random.default_rng(N + d)
    q = rng.standard_normal((1, H_Q, N, d))
    v = rng.standard_normal((1, H_KV, N, d))
    do = rng.standard_normal((1, H_Q, N, d))
    k = np.zeros((1, H_KV, N, d))
    dq, dk, dv = bwd_mod.attention_backward(q, k, v, do, causal)
    assert np.all(dq == 0.0)
    G = H_Q // H_KV
    for g in range(H_KV):
        heads = slice(g * G, (g + 1) * G)
        for block in (1, 64, 256):
            gk, gv = bwd_mod.backward_zero_keys(q[0, heads], v[0, g], do[0, heads], causal, block=block)
            np.testing.assert_allclose(gk, dk[0, g], rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(gv, dv[0, g], rtol=1e-10, atol=1e-12)


def test_zero_key_closed_form_is_sensitive():
    """The comparison above discriminates: the causal closed form differs from
    the non-causal oracle, and dK depends on V through the rows' D term (with
    K = 0, V enters dK only through dO_i . V_j and D_i)."""
    rng = np.random.default_rng(5)
    H, N, d = 2, 130, 8
    q = rng.standard_normal((1, H, N, d))
    v = rng.standard_normal((1, H, N, d))
    do = rng.standard_normal((1, H, N, d))
    k = np.zeros((1, H, N, d))
    _, dk, dv = bwd_mod.attention_backward(q, k, v, do, False)
    gk, gv = bwd_mod.backward_zero_keys(q[0, :1], v[0, 0], do[0, :1], True)
    assert not np.allclose(gk, dk[0, 0]) and not np.allclose(gv, dv[0, 0])
    gk0, _ = bwd_mod.backward_zero_keys(q[0, :1], np.zeros_like(v[0, 0]), do[0, :1], False)
    gk1, _ = bwd_mod.backward_zero_keys(q[0, :1], v[0, 0], do[0, :1], False)
    assert not np.allclose(gk0, gk1)
