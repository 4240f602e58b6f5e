"""Seeded synthetic inputs for the attention forward pass.

This module only draws numbers: it holds none of the attention arithmetic, so
both the HIP path and the fp64 CPU oracle can take their inputs from it.

Recipe (the workloads are synthetic attention shapes; no dataset is involved):

* Q, K and V are i.i.d. standard normal, drawn in float32 with
  ``torch.Generator`` and rounded to bfloat16 (round-to-nearest-even).
  Q uses ``seed``, K ``seed + 1`` and V ``seed + 2``.
* Layout is [B, H, N, d] contiguous: Q (and O) have H = H_Q heads, K and V
  have H = H_KV heads.
* Sampled rows for long sequences: a fixed-seed choice of (batch, head)
  pairs and query rows, so that the oracle can check a subset of outputs one
  row at a time.
"""
from __future__ import annotations

import numpy as np
import torch


def normal_bf16(shape, seed: int, device="cpu") -> torch.Tensor:
    """i.i.d. N(0, 1) drawn in float32 from ``seed`` and rounded to bf16."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    flat = out.view(-1)
    # Draw in slices so a 4 GiB bf16 tensor never needs a 16 GiB fp32 twin.
    step = 1 << 28
    for s in range(0, flat.numel(), step):
        e = min(flat.numel(), s + step)
        flat[s:e] = torch.randn(e - s, generator=gen, device=dev,
                                dtype=torch.float32).to(torch.bfloat16)
    return out


def make_qkv(B: int, H_Q: int, H_KV: int, N: int, d: int, seed: int,
             device="cpu"):
    """Q [B,H_Q,N,d], K and V [B,H_KV,N,d], bf16, contiguous."""
    q = normal_bf16((B, H_Q, N, d), seed, device)
    k = normal_bf16((B, H_KV, N, d), seed + 1, device)
    v = normal_bf16((B, H_KV, N, d), seed + 2, device)
    return q, k, v


def sample_rows(B: int, H_Q: int, H_KV: int, N: int, n_pairs: int = 16,
                n_rows: int = 32, seed: int = 1234):
    """Seeded (b, h, rows) selection for checking long sequences by sampling.

    Always contains (0, 0) and (B-1, H_Q-1), and one head of every KV group
    when there are at most ``n_pairs`` of them; the rest are uniform draws.
    Each pair gets ``n_rows`` distinct rows: 0, 1, 127, 128, N/2, N-2 and
    N-1 (those that exist) plus uniform draws.  Returns a list of
    ``(b, h, np.ndarray[int64])`` sorted by (b, h).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    G = H_Q // H_KV
    total = B * H_Q
    want = min(n_pairs, total)
    pairs: list[tuple[int, int]] = []

    def add(p):
        if p not in pairs and len(pairs) < want:
            pairs.append(p)

    add((0, 0))
    add((B - 1, H_Q - 1))
    if B * H_KV <= n_pairs:
        for b in range(B):
            for g in range(H_KV):
                add((b, g * G + int(rng.integers(G))))
    while len(pairs) < want:
        idx = int(rng.integers(total))
        add((idx // H_Q, idx % H_Q))
    forced = [r for r in (0, 1, 127, 128, N // 2, N - 2, N - 1) if 0 <= r < N]
    out = []
    for b, h in sorted(pairs):
        rows = list(dict.fromkeys(forced))
        k = min(n_rows, N)
        while len(rows) < k:
            r = int(rng.integers(N))
            if r not in rows:
                rows.append(r)
        out.append((b, h, np.array(sorted(rows), dtype=np.int64)))
    return out
