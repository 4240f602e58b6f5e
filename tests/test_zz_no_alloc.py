"""attn_fwd_split_noalloc: the split-KV attention whose split partials live
in the library's fixed device scratch instead of a caller workspace (for
callers that cannot allocate).  Through the C ABI, on two calls in a row (the
second with a smaller input), against attn_fwd_split with a caller workspace
(bit-identical: same kernels) and against the fp64 oracle at the forward
bar; a call whose partials would not fit the scratch is rejected."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import chiplet_numa_aware_amd as attn
import oracle
from chiplet_numa_aware_amd import inputs
from tests.gpu_util import assert_close, f64, say

pytestmark = pytest.mark.gpu

CASES = [
    # B, H_Q, H_KV, N_q, N_kv, d, causal, S: a decode batch, then a smaller one
    (4, 16, 4, 1, 8192, 128, True, 8),
    (2, 8, 2, 1, 3000, 128, True, 4),
    # and a prefill chunk with a ragged tail and d = 56, then a smaller one
    (1, 4, 2, 300, 2000, 56, True, 5),
    (1, 2, 2, 70, 500, 56, False, 3),
]


def _qkv(B, H_Q, H_KV, N_q, N_kv, d, seed):
    q = inputs.normal_bf16((B, H_Q, N_q, d), seed, "cuda")
    k = inputs.normal_bf16((B, H_KV, N_kv, d), seed + 1, "cuda")
    v = inputs.normal_bf16((B, H_KV, N_kv, d), seed + 2, "cuda")
    return q, k, v


@pytest.mark.parametrize("pair", [(0, 1), (2, 3)], ids=["decode", "prefill"])
def test_noalloc_equals_workspace_entry_point(pair):
    for i in pair:
        B, H_Q, H_KV, N_q, N_kv, d, causal, S = case = CASES[i]
        say(f"case noalloc {case}")
        q, k, v = _qkv(B, H_Q, H_KV, N_q, N_kv, d, seed=900 + i)
        o_ref, lse_ref = attn.attn_fwd_split(q, k, v, causal=causal, num_splits=S)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, H_Q, N_q), float("nan"), device="cuda")
        attn.attn_fwd_split_noalloc(q, k, v, o, lse, causal=causal, num_splits=S)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), case
        qh, kh, vh = f64(q), f64(k), f64(v)
        o_or, lse_or = oracle.partial_attention(qh, kh, vh, causal, 0, N_kv)
        fin = np.isfinite(lse_or)
        assert_close(f64(o)[fin], f64(lse)[fin], o_or[fin], lse_or[fin], f"noalloc {case}")


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    # 64 splits x 64 rows x (128 + 1) fp32 of 4 x 32 heads: above 32 MiB
    B, H_Q, H_KV, N_q, N_kv, d, S = 4, 32, 8, 64, 4096, 128, 64
    need = S * B * H_Q * N_q * (d + 1) * 4
    assert need > attn.SCRATCH_BYTES
    q, k, v = _qkv(B, H_Q, H_KV, N_q, N_kv, d, seed=950)
    o = torch.empty_like(q)
    with pytest.raises(attn.AttnError) as err:
        attn.attn_fwd_split_noalloc(q, k, v, o, None, causal=True, num_splits=S)
    assert err.value.code == -8
