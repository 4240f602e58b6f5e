"""Split-KV decode at the benchmark's full sizes, in the launch configuration
``bench.py --pass decode`` times (same shapes, splits, seeds and mapping),
checked on seeded sampled (batch, query head) rows against the fp64 oracle
(oracle.partial_head_rows over every key), plus bit-identity across mapping
modes at the largest shape.

Shapes (bf16 N(0,1), d=128, one query row, causal = every key):
  B=16 GQA 64/8 with 128K keys in 16 splits; B=64 GQA 64/8 with 32K keys in
  8 splits; B=8 MHA 32 heads with 32K keys in 16 splits.
"""
from collections import defaultdict

import numpy as np
import pytest
import torch

import bench
import chiplet_numa_aware_amd as attn
import oracle
from chiplet_numa_aware_amd import inputs
from tests.gpu_util import assert_close, f64, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", sorted(bench.SPLIT_WORKLOADS))
def test_decode_bench_shape_sampled_parity(name):
    B, H_Q, H_KV, N_q, N_kv, d, causal, S = bench.SPLIT_WORKLOADS[name]
    say(f"case {name}: B={B} H_Q={H_Q} H_KV={H_KV} N_q={N_q} N_kv={N_kv} splits={S}")
    q = inputs.normal_bf16((B, H_Q, N_q, d), 1000, "cuda")
    k = inputs.normal_bf16((B, H_KV, N_kv, d), 1001, "cuda")
    v = inputs.normal_bf16((B, H_KV, N_kv, d), 1002, "cuda")
    o, lse = attn.attn_fwd_split(q, k, v, causal=causal, num_splits=S, mapping=3)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(lse).all())
    by_kv = defaultdict(list)
    for b, h, rows in inputs.sample_rows(B, H_Q, H_KV, N_q, n_pairs=48, n_rows=N_q):
        by_kv[(b, oracle.kv_head(h, H_Q, H_KV))].append((h, rows))
    o_got, o_ref, l_got, l_ref = [], [], [], []
    for (b, g), heads in sorted(by_kv.items()):
        kh, vh = f64(k[b, g]), f64(v[b, g])
        for h, rows in heads:
            o_r, l_r = oracle.partial_head_rows(f64(q[b, h])[rows], kh, vh, rows, N_q,
                                                causal, 0, N_kv)
            o_got.append(f64(o[b, h])[rows])
            l_got.append(f64(lse[b, h])[rows])
            o_ref.append(o_r)
            l_ref.append(l_r)
    assert_close(np.concatenate(o_got), np.concatenate(l_got), np.concatenate(o_ref),
                 np.concatenate(l_ref), f"{name} sampled rows")
    if name == "decode_gqa64x8_b16_128k":
        for m in (0, 7, 15):
            o2, l2 = attn.attn_fwd_split(q, k, v, causal=causal, num_splits=S, mapping=m)
            torch.cuda.synchronize()
            assert torch.equal(o2, o) and torch.equal(l2, lse), m
    del q, k, v, o, lse
    torch.cuda.empty_cache()
