"""fp64 CPU oracle for the attention backward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP kernels.

What it computes: the gradients of the attention forward pass of "Optimizing
Attention on GPUs by Exploiting GPU Architectural NUMA Effects", §4 equation
(S = Q Kᵀ / √d, P = softmax(S) row-wise, O = P V), given the upstream
gradient dO (the pages run FlashAttention-2's backward with the same
workgroup remaps, digest page "Backward pass" and §5; they do not restate
its equations, so this is the gradient of the forward definition, written
out by the chain rule):

    dV = Pᵀ dO
    dP = dO Vᵀ
    dS = P ⊙ (dP - rowsum(dP ⊙ P))      (softmax Jacobian, row by row)
    dQ = dS K / √d,   dK = dSᵀ Q / √d

per head; with GQA a KV head's dK and dV are the sums over its query heads.
Causal masking as in sdpa.py (masked scores have P = 0).  No tiling, no
recomputation trick: P is formed from S directly.

Parity status: pinned (central finite differences of oracle.attention on
tiny shapes, torch float64 autograd of the math-backend SDPA, the closed
form dQ = dK = 0 when every V row is equal, dO = 0, GQA = summed MHA; see
tests/test_backward_oracle.py).  The sampled forms below (dQ of chosen query
rows, dK and dV of chosen keys, for long sequences) are pinned against
attention_backward on small shapes in the same file.
"""
from __future__ import annotations

import numpy as np

from .sdpa import kv_head


def _as_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def attention_backward(q, k, v, dout, causal: bool):
    """Gradients (dQ [B,H_Q,N,d], dK [B,H_KV,N,d], dV [B,H_KV,N,d]) of
    sum(dout * O) with O = attention(q, k, v), float64."""
    q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    B, H_Q, N, d = q.shape
    H_KV = k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    scale = 1.0 / np.sqrt(d)
    mask = np.tril(np.ones((N, N), dtype=bool)) if causal else None
    for b in range(B):
        for h in range(H_Q):
            g = kv_head(h, H_Q, H_KV)
            s = (q[b, h] @ k[b, g].T) * scale
            if causal:
                s = np.where(mask, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            p = e / e.sum(axis=1, keepdims=True)
            dv[b, g] += p.T @ dout[b, h]
            dp = dout[b, h] @ v[b, g].T
            ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
            dq[b, h] = (ds @ k[b, g]) * scale
            dk[b, g] += (ds.T @ q[b, h]) * scale
    return dq, dk, dv


def _softmax_rows(q_rows, k_head, rows, causal):
    """P (the softmax of the scaled, masked scores) of some query rows of one
    head, float64 [R, N]; also returns the scale 1/sqrt(d)."""
    d = q_rows.shape[1]
    scale = 1.0 / np.sqrt(d)
    s = (q_rows @ k_head.T) * scale
    if causal:
        s = np.where(np.arange(k_head.shape[0])[None, :] <= rows[:, None], s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=1, keepdims=True), scale


def backward_query_rows(q_rows, k_head, v_head, dout_rows, rows, causal: bool):
    """dQ of some query rows of one head, float64 [R, d].

    q_rows, dout_rows: [R, d], the rows' queries and upstream gradients;
    k_head, v_head: [N, d] (the head's KV head); rows: [R] their positions
    (causal mask).  dQ_i needs row i alone: dS_i = P_i * (dP_i - <dP_i, P_i>)
    with dP_i = dO_i V^T, and dQ_i = dS_i K / sqrt(d).
    """
    q_rows, k_head, v_head, dout_rows = (_as_f64(x) for x in (q_rows, k_head, v_head, dout_rows))
    rows = np.asarray(rows, dtype=np.int64)
    p, scale = _softmax_rows(q_rows, k_head, rows, causal)
    dp = dout_rows @ v_head.T
    ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
    return (ds @ k_head) * scale


def backward_key_rows(q_heads, k_head, v_head, dout_heads, keys, causal: bool,
                      row_chunk: int = 512):
    """dK and dV of some keys of one KV head, float64 ([K, d], [K, d]).

    q_heads, dout_heads: [G, N, d], the query heads that read this KV head
    (their contributions are summed); k_head, v_head: [N, d]; keys: [K] key
    indices.  dV_j = sum over heads and rows i of P[i, j] dO_i, and
    dK_j = sum of dS[i, j] Q_i / sqrt(d): every row's P and dS need that row's
    whole score row (its normalisation), so all rows are formed; they are
    taken ``row_chunk`` at a time only to bound memory.
    """
    q_heads, k_head, v_head, dout_heads = (_as_f64(x) for x in (q_heads, k_head, v_head, dout_heads))
    keys = np.asarray(keys, dtype=np.int64)
    G, N, d = q_heads.shape
    dk = np.zeros((len(keys), d))
    dv = np.zeros((len(keys), d))
    for h in range(G):
        for r0 in range(0, N, row_chunk):
            rows = np.arange(r0, min(N, r0 + row_chunk))
            p, scale = _softmax_rows(q_heads[h, rows], k_head, rows, causal)
            dp = dout_heads[h, rows] @ v_head.T
            ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
            dv += p[:, keys].T @ dout_heads[h, rows]
            dk += (ds[:, keys].T @ q_heads[h, rows]) * scale
    return dk, dv


def backward_zero_keys(q_heads, v_head, dout_heads, causal: bool, block: int = 256):
    """dK and dV of every key of one KV head whose keys K are all zero,
    float64 ([N, d], [N, d]); dQ is then exactly zero.

    With K = 0 every score is 0, so row i attends uniformly to its visible
    keys: P[i, j] = c_i = 1 / |J_i| (|J_i| = i + 1 causal, N otherwise).  The
    chain rule of the module docstring then gives, with I_j the rows that
    see key j (i >= j causal, all rows otherwise), O_i = c_i sum_{j in J_i}
    V_j and D_i = dO_i . O_i:

        dV_j = sum_{i in I_j} c_i dO_i
        dS[i, j] = c_i (dO_i . V_j - D_i)
        dK_j = (A_j V_j - b_j) / sqrt(d),
            A_j = sum_{i in I_j} c_i Q_i dO_iᵀ,  b_j = sum_{i in I_j} c_i D_i Q_i

    (summed over the G query heads in q_heads, dout_heads: [G, N, d]).  The
    sums over I_j are suffix sums when causal, taken ``block`` rows at a time
    from the last block down: O(N d^2) per head instead of the O(N^2 d) of
    the general form, so it runs at the full sequence lengths.
    """
    q_heads, v_head, dout_heads = (_as_f64(x) for x in (q_heads, v_head, dout_heads))
    G, N, d = q_heads.shape
    scale = 1.0 / np.sqrt(d)
    count = np.arange(1, N + 1, dtype=np.float64) if causal else np.full(N, float(N))
    c = 1.0 / count
    if causal:
        o = np.cumsum(v_head, axis=0) * c[:, None]
    else:
        o = np.broadcast_to(v_head.sum(axis=0) * c[0], (N, d))
    dk = np.zeros((N, d))
    dv = np.zeros((N, d))
    for h in range(G):
        qh, doh = q_heads[h], dout_heads[h]
        D = (doh * o).sum(axis=1)
        cdo = doh * c[:, None]
        if not causal:
            A = qh.T @ cdo                       # sum_i c_i Q_i dO_iᵀ
            b = qh.T @ (c * D)
            dv += cdo.sum(axis=0)[None, :]
            dk += (v_head @ A.T - b[None, :]) * scale
            continue
        dv += np.cumsum(cdo[::-1], axis=0)[::-1]
        A = np.zeros((d, d))
        b = np.zeros(d)
        for j0 in range((N - 1) // block * block, -1, -block):
            j1 = min(N, j0 + block)
            rows = slice(j0, j1)
            vb, qb, cdb = v_head[rows], qh[rows], cdo[rows]
            # in-block rows i >= j: W[i, j] = c_i (dO_i . V_j - D_i)
            w = cdb @ vb.T - (c[rows] * D[rows])[:, None]
            w = np.tril(w)
            dk[rows] += (vb @ A.T - b[None, :] + w.T @ qb) * scale
            A += qb.T @ cdb
            b += qb.T @ (c[rows] * D[rows])
    return dk, dv
