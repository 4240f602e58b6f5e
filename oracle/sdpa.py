"""fp64 CPU oracle for the attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP kernels behind the C ABI and their Python binding) never calls it,
and it shares no code with them.

What it computes: plain scaled dot-product attention, as written in
"Optimizing Attention on GPUs by Exploiting GPU Architectural NUMA Effects",
§4 (notation table and the equation S = Q Kᵀ, P = softmax(S / √d), O = P V),
per head, with Q, K, V ∈ R^{N×d}.  The FlashAttention-2 kernel of that page
(§3, Figure 4: every row-block workgroup reads all of Kᵀ and V with an online
softmax) is an exact reordering of this definition, and the workgroup remap
changes only which workgroup computes which rows (§4, check 6: no change to
the algorithm), so the oracle is the definition itself: no tiling, no online
softmax, one dense score row per query, a library matmul for the sums.

Readings where the pages are silent (each is listed with the others in the
design notes):

* GQA: query head h reads KV head ``h // (H_Q // H_KV)`` (contiguous groups;
  the digest's §2 Q2 defines the cluster for GQA as one KV group, and the
  "Fused Grouped-Query Attention" page groups 8 query heads on 1 KV head).
* Causal: top-left aligned lower triangle; query row i sees keys 0..i.
* Scale: 1/√d with the real head dimension d.
* lse: natural-log logsumexp of the scaled, masked scores of each row.

Parity status: pinned (brute force on tiny inputs, closed forms for
all-equal scores and causal row 0, lse identities, GQA/MHA equivalence,
one-hot rows and torch's fp64 math SDPA; see tests/test_oracle.py).
"""
from __future__ import annotations

import numpy as np


def kv_head(h: int, H_Q: int, H_KV: int) -> int:
    """KV head read by query head ``h`` (contiguous query-head groups)."""
    return h // (H_Q // H_KV)


def _as_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def attention_head_rows(q_rows, k_head, v_head, rows, causal: bool):
    """O and lse for some query rows of one head.

    q_rows: [R, d] queries; k_head, v_head: [N, d]; rows: [R] the query
    positions (they decide the causal mask).  Returns (O [R, d], lse [R]),
    float64.
    """
    q_rows = _as_f64(q_rows)
    k_head = _as_f64(k_head)
    v_head = _as_f64(v_head)
    rows = np.asarray(rows, dtype=np.int64)
    d = q_rows.shape[1]
    n_keys = k_head.shape[0]
    # S = Q Kᵀ / √d for the selected rows (one full score row per query).
    s = (q_rows @ k_head.T) / np.sqrt(d)
    if causal:
        keys = np.arange(n_keys)[None, :]
        s = np.where(keys <= rows[:, None], s, -np.inf)
    # softmax along the keys, written out: subtract the row max, exponentiate,
    # normalise by the row sum.
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    ell = e.sum(axis=1, keepdims=True)
    p = e / ell
    o = p @ v_head
    lse = (m + np.log(ell))[:, 0]
    return o, lse


def attention(q, k, v, causal: bool, row_chunk: int = 1024):
    """Full attention forward: (O [B,H_Q,N,d], lse [B,H_Q,N]) in float64.

    q: [B,H_Q,N,d]; k, v: [B,H_KV,N,d].  Rows are processed in chunks of
    ``row_chunk`` only to bound memory; every row still sees its whole key
    range at once.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, H_Q, N, d = q.shape
    H_KV = k.shape[1]
    if H_Q % H_KV:
        raise ValueError("H_Q must be a multiple of H_KV")
    o = np.empty((B, H_Q, N, d), dtype=np.float64)
    lse = np.empty((B, H_Q, N), dtype=np.float64)
    for b in range(B):
        for h in range(H_Q):
            g = kv_head(h, H_Q, H_KV)
            for r0 in range(0, N, row_chunk):
                rows = np.arange(r0, min(N, r0 + row_chunk))
                o[b, h, rows], lse[b, h, rows] = attention_head_rows(
                    q[b, h, rows], k[b, g], v[b, g], rows, causal)
    return o, lse


def attention_sampled(q, k, v, causal: bool, samples):
    """Oracle on sampled rows only.

    ``samples``: iterable of (b, h, rows).  q, k, v: arrays indexable as
    [b, h] -> [N, d] (numpy arrays of any float dtype).
    Returns a list of (b, h, rows, O [R,d], lse [R]).
    """
    out = []
    H_Q = q.shape[1]
    H_KV = k.shape[1]
    for b, h, rows in samples:
        g = kv_head(h, H_Q, H_KV)
        rows = np.asarray(rows, dtype=np.int64)
        o_r, lse_r = attention_head_rows(_as_f64(q[b, h])[rows],
                                         k[b, g], v[b, g], rows, causal)
        out.append((b, h, rows, o_r, lse_r))
    return out

