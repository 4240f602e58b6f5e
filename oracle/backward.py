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
