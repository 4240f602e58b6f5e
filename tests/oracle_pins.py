"""Checks that pin an attention implementation to facts fixed outside it.

Each ``pin_*`` takes ``attn(q, k, v, causal) -> (O, lse)`` (numpy in, numpy
float64 out, layouts [B,H_Q,N,d] / [B,H_KV,N,d] / [B,H_Q,N]) and raises
AssertionError when the implementation disagrees with:

* a brute-force evaluation of the definition with Python loops
  (``math.fsum``/``math.exp``), on tiny inputs;
* closed forms (all-equal scores, causal row 0, one-hot rows);
* identities every correct result satisfies (probabilities sum to one,
  lse bounds, causal prefix independence, GQA = repeated MHA);
* torch's float64 math-backend scaled_dot_product_attention.

The definition pinned: "Optimizing Attention on GPUs by Exploiting GPU
Architectural NUMA Effects", §4 equation (S = Q Kᵀ, P = softmax(S/√d),
O = P V), with causal = top-left lower triangle and lse = ln Σ exp(S/√d).
The same checks run against deliberately broken copies of the oracle in
test_oracle_mutants.py to show that they catch plausible mistakes.
"""
from __future__ import annotations

import math

import numpy as np
import torch
from torch.nn.attention import SDPBackend, sdpa_kernel


def _rand(rng, shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def brute_force(q, k, v, causal):
    """The definition with explicit loops, no max subtraction, math.fsum."""
    B, H_Q, N, d = q.shape
    H_KV = k.shape[1]
    G = H_Q // H_KV
    o = np.zeros(q.shape)
    lse = np.zeros((B, H_Q, N))
    for b in range(B):
        for h in range(H_Q):
            g = h // G
            for i in range(N):
                keys = range(i + 1) if causal else range(N)
                s = [math.fsum(float(q[b, h, i, t]) * float(k[b, g, j, t])
                               for t in range(d)) / math.sqrt(d) for j in keys]
                e = [math.exp(x) for x in s]
                z = math.fsum(e)
                for t in range(d):
                    o[b, h, i, t] = math.fsum(
                        e[jj] * float(v[b, g, j, t])
                        for jj, j in enumerate(keys)) / z
                lse[b, h, i] = math.log(z)
    return o, lse


def pin_brute_force(attn, seed=0):
    rng = np.random.default_rng(seed)
    shapes = [(1, 1, 1, 1, 1), (1, 2, 2, 5, 3), (2, 4, 2, 7, 8),
              (1, 4, 1, 16, 4), (2, 3, 3, 9, 5)]
    for B, H_Q, H_KV, N, d in shapes:
        q = _rand(rng, (B, H_Q, N, d))
        k = _rand(rng, (B, H_KV, N, d))
        v = _rand(rng, (B, H_KV, N, d))
        for causal in (False, True):
            o, lse = attn(q, k, v, causal)
            ob, lb = brute_force(q, k, v, causal)
            assert np.max(np.abs(o - ob)) <= 1e-12, (B, H_Q, H_KV, N, d, causal)
            assert np.max(np.abs(lse - lb)) <= 1e-12, (B, H_Q, H_KV, N, d, causal)


def _scores(q, k, b, h, G):
    d = q.shape[-1]
    return (q[b, h] @ k[b, h // G].T) / math.sqrt(d)


def pin_lse_identities(attn, seed=1):
    """Σ_j exp(s_j - lse) = 1, Σ_j exp(s_j - lse) v_j = o, lse bounds."""
    rng = np.random.default_rng(seed)
    B, H_Q, H_KV, N, d = 2, 4, 2, 40, 16
    q = _rand(rng, (B, H_Q, N, d), 2.0)
    k = _rand(rng, (B, H_KV, N, d))
    v = _rand(rng, (B, H_KV, N, d))
    G = H_Q // H_KV
    for causal in (False, True):
        o, lse = attn(q, k, v, causal)
        for b in range(B):
            for h in range(H_Q):
                s = _scores(q, k, b, h, G)
                for i in range(N):
                    n_allowed = i + 1 if causal else N
                    si = s[i, :n_allowed]
                    p = np.exp(si - lse[b, h, i])
                    assert abs(p.sum() - 1.0) <= 1e-12
                    ref_o = p @ v[b, h // G, :n_allowed]
                    assert np.max(np.abs(ref_o - o[b, h, i])) <= 1e-12
                    mx = si.max()
                    assert mx - 1e-12 <= lse[b, h, i] <= mx + math.log(n_allowed) + 1e-12


def pin_all_equal_scores(attn, seed=2):
    """Q = 0: every score is 0, so O_i = mean(V_J) and lse_i = ln |J|."""
    rng = np.random.default_rng(seed)
    B, H_Q, H_KV, N, d = 1, 2, 1, 33, 8
    q = np.zeros((B, H_Q, N, d))
    k = _rand(rng, (B, H_KV, N, d))
    v = _rand(rng, (B, H_KV, N, d))
    o, lse = attn(q, k, v, False)
    for h in range(H_Q):
        assert np.max(np.abs(o[0, h] - v[0, 0].mean(axis=0)[None, :])) <= 1e-12
        assert np.max(np.abs(lse[0, h] - math.log(N))) <= 1e-12
    o, lse = attn(q, k, v, True)
    csum = np.cumsum(v[0, 0], axis=0) / np.arange(1, N + 1)[:, None]
    for h in range(H_Q):
        assert np.max(np.abs(o[0, h] - csum)) <= 1e-12
        assert np.max(np.abs(lse[0, h] - np.log(np.arange(1, N + 1)))) <= 1e-12


def pin_causal(attn, seed=3):
    """Causal row i = full attention over the prefix; later keys are ignored;
    row 0 gives O_0 = V_0 and lse_0 = q_0·k_0/√d."""
    rng = np.random.default_rng(seed)
    B, H, N, d = 1, 2, 24, 8
    q = _rand(rng, (B, H, N, d))
    k = _rand(rng, (B, H, N, d))
    v = _rand(rng, (B, H, N, d))
    o, lse = attn(q, k, v, True)
    for i in (0, 1, 7, N - 1):
        op, lp = attn(q[:, :, :i + 1], k[:, :, :i + 1], v[:, :, :i + 1], False)
        assert np.max(np.abs(op[:, :, i] - o[:, :, i])) <= 1e-12
        assert np.max(np.abs(lp[:, :, i] - lse[:, :, i])) <= 1e-12
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 10:] = _rand(rng, k2[:, :, 10:].shape, 5.0)
    v2[:, :, 10:] = _rand(rng, v2[:, :, 10:].shape, 5.0)
    o2, lse2 = attn(q, k2, v2, True)
    assert np.array_equal(o2[:, :, :10], o[:, :, :10])
    assert np.array_equal(lse2[:, :, :10], lse[:, :, :10])
    assert np.max(np.abs(o[:, :, 0] - v[:, :, 0])) <= 1e-12
    s00 = np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]) / math.sqrt(d)
    assert np.max(np.abs(lse[:, :, 0] - s00)) <= 1e-12


def pin_gqa_equals_repeated_mha(attn, seed=4):
    rng = np.random.default_rng(seed)
    B, H_Q, H_KV, N, d = 2, 6, 2, 20, 8
    q = _rand(rng, (B, H_Q, N, d))
    k = _rand(rng, (B, H_KV, N, d))
    v = _rand(rng, (B, H_KV, N, d))
    G = H_Q // H_KV
    kr = np.repeat(k, G, axis=1)
    vr = np.repeat(v, G, axis=1)
    for causal in (False, True):
        o, lse = attn(q, k, v, causal)
        om, lm = attn(q, kr, vr, causal)
        assert np.max(np.abs(o - om)) <= 1e-13
        assert np.max(np.abs(lse - lm)) <= 1e-13


def pin_one_hot(attn, seed=5):
    """K[j*] = c·Q[i] with a score margin of at least 40: O_i = V[j*]."""
    rng = np.random.default_rng(seed)
    N, d = 32, 16
    q = _rand(rng, (1, 1, N, d), 0.1)
    k = _rand(rng, (1, 1, N, d), 0.1)
    v = _rand(rng, (1, 1, N, d))
    i, js = 20, 13
    qi = q[0, 0, i]
    c = 60.0 * math.sqrt(d) / float(qi @ qi)
    k[0, 0, js] = c * qi
    for causal in (False, True):
        o, lse = attn(q, k, v, causal)
        assert np.max(np.abs(o[0, 0, i] - v[0, 0, js])) <= 1e-12
        s = float(qi @ k[0, 0, js]) / math.sqrt(d)
        assert abs(lse[0, 0, i] - s) <= 1e-12


def pin_torch_sdpa(attn, seed=6):
    """torch's float64 math SDPA on the CPU (a library routine)."""
    rng = np.random.default_rng(seed)
    for B, H_Q, H_KV, N, d in [(2, 4, 4, 65, 32), (1, 8, 2, 50, 24)]:
        q = _rand(rng, (B, H_Q, N, d))
        k = _rand(rng, (B, H_KV, N, d))
        v = _rand(rng, (B, H_KV, N, d))
        G = H_Q // H_KV
        tq = torch.from_numpy(q)
        tk = torch.from_numpy(np.repeat(k, G, axis=1))
        tv = torch.from_numpy(np.repeat(v, G, axis=1))
        for causal in (False, True):
            with sdpa_kernel(SDPBackend.MATH):
                ref = torch.nn.functional.scaled_dot_product_attention(
                    tq, tk, tv, is_causal=causal).numpy()
            o, _ = attn(q, k, v, causal)
            assert np.max(np.abs(o - ref)) <= 1e-12, (B, H_Q, H_KV, causal)


ALL_PINS = [pin_brute_force, pin_lse_identities, pin_all_equal_scores,
            pin_causal, pin_gqa_equals_repeated_mha, pin_one_hot,
            pin_torch_sdpa]
