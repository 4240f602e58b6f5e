"""fp64 CPU oracle for split-KV partial attention and the (O, lse) merge.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
never calls it, and it shares no code with the HIP kernels.

What it computes.  Attention of N_q query rows over N_kv keys, restricted to a
contiguous key range [kv_begin, kv_end) (one split of the keys), returned as a
partial result: the output normalised over that range, O_s, and its natural-log
logsumexp, lse_s.  Partial results over the splits of a partition of the keys
are combined by the merge

    lse = ln sum_s exp(lse_s),    O = sum_s exp(lse_s - lse) O_s,

the (m, l, O) reduction of the "Fused Grouped-Query Attention" page (decode
and sequence-parallel strategies: each device computes attention over its KV
shard, the partial results are reduced into the final output), written here
in (O, lse) form, since lse_s = m_s + ln l_s and O_s = (unnormalised O_s) / l_s.
The per-split attention is the definition of "Optimizing Attention on GPUs by
Exploiting GPU Architectural NUMA Effects", §4 (S = Q Kᵀ, P = softmax(S/√d),
O = P V) over the keys of the split.

Readings where the pages are silent:

* Causal with N_q != N_kv: bottom-right aligned, so query row i (0-based)
  sees key j iff j <= i + (N_kv - N_q).  With N_q == N_kv this is the
  top-left lower triangle of the full oracle; with N_q = 1 (decode) the one
  row sees every key.
* A row that sees no key of a split has O_s = 0 and lse_s = -inf; it then
  carries weight exp(-inf) = 0 in the merge.
* GQA, scale and lse as in sdpa.py.

Parity status: pinned (the merge of partials over random key partitions
equals the full definition; brute force with Python loops on tiny shapes;
closed forms for Q = 0 and empty splits; merge identities; see
tests/test_split_oracle.py).
"""
from __future__ import annotations

import numpy as np

from .sdpa import kv_head


def _as_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def causal_offset(N_q: int, N_kv: int) -> int:
    """Row i sees keys 0 .. i + causal_offset under the causal mask."""
    return N_kv - N_q


def partial_head_rows(q_rows, k_head, v_head, rows, N_q: int, causal: bool,
                      kv_begin: int, kv_end: int):
    """(O_s [R, d], lse_s [R]) of some query rows of one head over the keys
    kv_begin .. kv_end - 1.  ``rows`` are the query positions (0 .. N_q - 1);
    k_head, v_head: [N_kv, d]."""
    q_rows = _as_f64(q_rows)
    k_head = _as_f64(k_head)
    v_head = _as_f64(v_head)
    rows = np.asarray(rows, dtype=np.int64)
    n_kv, d = k_head.shape
    R = q_rows.shape[0]
    o = np.zeros((R, d))
    lse = np.full(R, -np.inf)
    if kv_end <= kv_begin:
        return o, lse
    keys = np.arange(kv_begin, kv_end)
    s = (q_rows @ k_head[keys].T) / np.sqrt(d)
    if causal:
        last = rows + causal_offset(N_q, n_kv)
        s = np.where(keys[None, :] <= last[:, None], s, -np.inf)
    seen = np.isfinite(s).any(axis=1)
    if not seen.any():
        return o, lse
    s = s[seen]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    ell = e.sum(axis=1, keepdims=True)
    o[seen] = (e / ell) @ v_head[keys]
    lse[seen] = (m + np.log(ell))[:, 0]
    return o, lse


def partial_attention(q, k, v, causal: bool, kv_begin: int, kv_end: int):
    """Partial attention of every row over keys [kv_begin, kv_end):
    q [B,H_Q,N_q,d], k and v [B,H_KV,N_kv,d] -> (O_s [B,H_Q,N_q,d],
    lse_s [B,H_Q,N_q]), float64."""
    q = _as_f64(q)
    B, H_Q, N_q, d = q.shape
    H_KV = k.shape[1]
    o = np.zeros((B, H_Q, N_q, d))
    lse = np.full((B, H_Q, N_q), -np.inf)
    rows = np.arange(N_q)
    for b in range(B):
        for h in range(H_Q):
            g = kv_head(h, H_Q, H_KV)
            o[b, h], lse[b, h] = partial_head_rows(
                q[b, h], k[b, g], v[b, g], rows, N_q, causal, kv_begin, kv_end)
    return o, lse


def merge(o_parts, lse_parts):
    """Merge S partial results: o_parts [S, ..., d], lse_parts [S, ...] ->
    (O [..., d], lse [...]).  A row whose every part is -inf gets O = 0 and
    lse = -inf."""
    o_parts = _as_f64(o_parts)
    lse_parts = _as_f64(lse_parts)
    top = lse_parts.max(axis=0)
    finite = np.isfinite(top)
    shift = np.where(finite, top, 0.0)
    w = np.exp(lse_parts - shift[None])        # exp(-inf) = 0 for empty parts
    total = w.sum(axis=0)
    lse = np.where(finite, shift + np.log(np.where(finite, total, 1.0)), -np.inf)
    o = (w[..., None] * o_parts).sum(axis=0)
    o = np.where(finite[..., None], o / np.where(finite, total, 1.0)[..., None], 0.0)
    return o, lse
