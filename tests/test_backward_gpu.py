"""Attention backward (attn_bwd) on the GPU against the fp64 oracle
(oracle/backward.py), through the C ABI.

The GPU gradients use the GPU forward's bf16 O and fp32 lse, as a training
step would; the oracle differentiates the exact attention.  Bar per tensor
(dQ, dK, dV), from the rounding steps of the kernels (bf16 P and dS before
their products, D from the bf16 O, bf16 outputs; see the design notes):
relative L2 error <= BWD_REL_L2 and max|err| <= BWD_MAX_REL * max|ref|.
"""
from __future__ import annotations

import pytest
import torch

import chiplet_numa_aware_amd as attn
import oracle
from tests.gpu_util import check_grad, f64, grad_inputs, say

pytestmark = pytest.mark.gpu


CASES = [
    # B, H_Q, H_KV, N, d, causal
    (1, 2, 2, 300, 128, False),
    (1, 2, 2, 300, 128, True),
    (2, 4, 2, 257, 64, True),      # GQA, ragged tail, d = 64
    (1, 4, 1, 200, 56, False),     # d = 56 runs the 64-wide tile
    (1, 2, 1, 333, 96, True),      # d = 96 runs the 128-wide tile
    (1, 2, 2, 32, 128, True),      # one tile
    (1, 3, 3, 1, 128, False),      # one row
    (1, 2, 2, 129, 64, True),      # one key past a 128-key block
    (1, 8, 2, 700, 128, True),     # GQA 4 heads per KV head, several blocks
    (1, 1, 1, 1030, 128, False),
    (2, 6, 2, 301, 128, True),     # GQA, 3 query heads per KV head
    (1, 3, 1, 190, 64, False),
]


@pytest.mark.parametrize("case", CASES, ids=str)
def test_backward_matches_oracle(case):
    B, H_Q, H_KV, N, d, causal = case
    say(f"case bwd {case}")
    q, k, v, dout = grad_inputs(B, H_Q, H_KV, N, d, seed=900 + N + d)
    o, lse = attn.attn_fwd(q, k, v, causal=causal)
    dq, dk, dv = attn.attn_bwd(q, k, v, o, dout, lse, causal=causal)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(f64(q), f64(k), f64(v), f64(dout), causal)
    check_grad(f64(dq), rq, f"dQ {case}")
    check_grad(f64(dk), rk, f"dK {case}")
    check_grad(f64(dv), rv, f"dV {case}")


@pytest.mark.parametrize("causal", [False, True])
def test_backward_bitwise_identical_across_mappings(causal):
    q, k, v, dout = grad_inputs(2, 8, 2, 1000, 128, seed=910)
    o, lse = attn.attn_fwd(q, k, v, causal=causal)
    ref = None
    for mapping in range(16):
        dq, dk, dv = attn.attn_bwd(q, k, v, o, dout, lse, causal=causal, mapping=mapping)
        torch.cuda.synchronize()
        if ref is None:
            ref = (dq.clone(), dk.clone(), dv.clone())
        else:
            for a, b, name in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
                assert torch.equal(a, b), (mapping, name)


def test_backward_workspace_layout_is_checked():
    """The workspace is [B, H_Q, 2, N] (each head's lse2 rows, then its D
    rows); a buffer of another shape, or on the host, is rejected before
    any launch."""
    B, H_Q, H_KV, N, d = 2, 4, 2, 64, 64
    q, k, v, dout = grad_inputs(B, H_Q, H_KV, N, d, seed=925)
    o, lse = attn.attn_fwd(q, k, v)
    for bad in (torch.empty((2, B, H_Q, N), device="cuda"),
                torch.empty((B, H_Q, 2, N)),
                torch.empty((B, H_Q, 2, N), device="cuda", dtype=torch.float64)):
        with pytest.raises(ValueError):
            attn.attn_bwd(q, k, v, o, dout, lse, ws=bad)
    dq, dk, dv = attn.attn_bwd(q, k, v, o, dout, lse, ws=torch.empty((B, H_Q, 2, N), device="cuda"))
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(f64(q), f64(k), f64(v), f64(dout), False)
    check_grad(f64(dk), rk, "dK with a caller workspace")


def test_backward_writes_every_element():
    """Outputs prefilled with NaN come back finite (every element written)."""
    B, H_Q, H_KV, N, d = 1, 4, 2, 390, 120
    q, k, v, dout = grad_inputs(B, H_Q, H_KV, N, d, seed=920)
    o, lse = attn.attn_fwd(q, k, v, causal=True)
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    ws = torch.full((B, H_Q, 2, N), float("nan"), device="cuda")
    attn.attn_bwd(q, k, v, o, dout, lse, causal=True, dq=dq, dk=dk, dv=dv, ws=ws)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    rq, rk, rv = oracle.attention_backward(f64(q), f64(k), f64(v), f64(dout), True)
    check_grad(f64(dq), rq, "dQ d=120")
    check_grad(f64(dk), rk, "dK d=120")
    check_grad(f64(dv), rv, "dV d=120")
