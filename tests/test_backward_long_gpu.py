"""Full-size backward (attn_bwd) in the launch configuration the benchmark's
backward pass times, checked on seeded samples against the fp64 oracle:

* dQ of sampled (batch, head, row) sets, one row at a time
  (oracle.backward_query_rows; cheap at any N);
* dK and dV of sampled keys of a few KV heads (oracle.backward_key_rows,
  which forms every score row of the heads that read them, so it is run
  where that takes seconds: N <= 32K).

Workloads (bf16 N(0,1) inputs, d=128 unless stated): MHA B=1 H=128 N=32768
causal; MHA B=1 H=128 N=131072 non-causal (dQ rows only); GQA B=1 64/8
N=8192 causal (a whole KV group for dK/dV); MHA B=1 H=128 d=56 N=32768 causal.

At N=131072, dK and dV of every key of a few KV heads are checked in the
degenerate case K = 0 (every score 0, uniform attention over the visible
keys), where the oracle has an O(N d^2) closed form
(oracle.backward_zero_keys) and dQ must be exactly zero.  The gradient
kernels have no data-dependent branches, so the case runs the same code in
the same launch configuration as random inputs.
"""
import numpy as np
import pytest
import torch

import chiplet_numa_aware_amd as attn
import oracle
from chiplet_numa_aware_amd import inputs
from tests.gpu_util import check_grad, f64, grad_inputs, say

pytestmark = pytest.mark.gpu

LONG_BWD = [
    # name, B, H_Q, H_KV, N, d, causal, seed, mapping, KV heads checked for dK/dV
    ("mha_32k_causal", 1, 128, 128, 32768, 128, True, 611, 7, (127,)),
    ("mha_128k", 1, 128, 128, 131072, 128, False, 620, 3, ()),
    ("gqa64x8_8k_causal", 1, 64, 8, 8192, 128, True, 630, 7, (5,)),
    ("dsv3_d56_32k_causal", 1, 128, 128, 32768, 56, True, 640, 7, (0,)),
]


def _sample_keys(N, n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    forced = [j for j in (0, 1, 127, 128, N // 2, N - 2, N - 1) if 0 <= j < N]
    rest = rng.choice(N, size=n, replace=False)
    return np.unique(np.concatenate([forced, rest]))


@pytest.mark.parametrize("cfg", LONG_BWD, ids=lambda c: c[0])
def test_long_backward_sampled(cfg):
    name, B, H_Q, H_KV, N, d, causal, seed, mapping, kv_heads = cfg
    say(f"case bwd long {name} mapping {mapping}")
    q, k, v, dout = grad_inputs(B, H_Q, H_KV, N, d, seed)
    o, lse = attn.attn_fwd(q, k, v, causal=causal, mapping=mapping)
    dq, dk, dv = attn.attn_bwd(q, k, v, o, dout, lse, causal=causal, mapping=mapping)
    torch.cuda.synchronize()
    G = H_Q // H_KV

    got, ref = [], []
    for b, h, rows in inputs.sample_rows(B, H_Q, H_KV, N, n_pairs=8, n_rows=16, seed=1234):
        g = oracle.kv_head(h, H_Q, H_KV)
        ridx = torch.as_tensor(rows, device=q.device)
        ref.append(oracle.backward_query_rows(
            f64(q[b, h].index_select(0, ridx)), f64(k[b, g]), f64(v[b, g]),
            f64(dout[b, h].index_select(0, ridx)), rows, causal))
        got.append(f64(dq[b, h].index_select(0, ridx)))
    check_grad(np.concatenate(got), np.concatenate(ref), f"{name} dQ sampled rows")

    for g in kv_heads:
        keys = _sample_keys(N, 16, seed + g)
        kidx = torch.as_tensor(keys, device=q.device)
        heads = list(range(g * G, (g + 1) * G))
        rk, rv = oracle.backward_key_rows(f64(q[0, heads]), f64(k[0, g]), f64(v[0, g]),
                                          f64(dout[0, heads]), keys, causal)
        check_grad(f64(dk[0, g].index_select(0, kidx)), rk, f"{name} dK keys of KV head {g}")
        check_grad(f64(dv[0, g].index_select(0, kidx)), rv, f"{name} dV keys of KV head {g}")


ZERO_KEYS = [
    # name, B, H_Q, H_KV, N, d, causal, seed, mapping, KV heads checked
    ("mha_128k", 1, 128, 128, 131072, 128, False, 650, 3, (0, 127)),
    ("mha_128k_causal", 1, 128, 128, 131072, 128, True, 651, 15, (64,)),
    ("gqa64x8_128k_causal", 1, 64, 8, 131072, 128, True, 652, 15, (3,)),
]


@pytest.mark.parametrize("cfg", ZERO_KEYS, ids=lambda c: c[0])
def test_long_backward_zero_keys_every_key(cfg):
    name, B, H_Q, H_KV, N, d, causal, seed, mapping, kv_heads = cfg
    say(f"case bwd zero keys {name} mapping {mapping}")
    q, k, v, dout = grad_inputs(B, H_Q, H_KV, N, d, seed)
    k.zero_()
    o, lse = attn.attn_fwd(q, k, v, causal=causal, mapping=mapping)
    dq, dk, dv = attn.attn_bwd(q, k, v, o, dout, lse, causal=causal, mapping=mapping)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(dq)) == 0, f"{name}: dQ not zero with K = 0"
    G = H_Q // H_KV
    for g in kv_heads:
        heads = slice(g * G, (g + 1) * G)
        rk, rv = oracle.backward_zero_keys(f64(q[0, heads]), f64(v[0, g]), f64(dout[0, heads]), causal)
        check_grad(f64(dk[0, g]), rk, f"{name} dK every key, KV head {g}")
        check_grad(f64(dv[0, g]), rv, f"{name} dV every key, KV head {g}")
    del q, k, v, dout, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
