"""Split-KV attention and the (O, lse) merge on the GPU against the oracle
(oracle/split.py), through the C ABI (attn_fwd_split, attn_merge).

Every split's partial result in the workspace is compared with
oracle.partial_attention over that split's key range, and the merged output
with the full attention; N_q != N_kv uses the bottom-right causal reading.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import chiplet_numa_aware_amd as attn
import oracle
from chiplet_numa_aware_amd import inputs
from tests.gpu_util import (LSE_MAX_ABS, O_MAX_ABS, O_REL_L2, assert_close, f64, lse_bar, say)

pytestmark = pytest.mark.gpu


def _qkv(B, H_Q, H_KV, N_q, N_kv, d, seed):
    q = inputs.normal_bf16((B, H_Q, N_q, d), seed, "cuda")
    k = inputs.normal_bf16((B, H_KV, N_kv, d), seed + 1, "cuda")
    v = inputs.normal_bf16((B, H_KV, N_kv, d), seed + 2, "cuda")
    return q, k, v


def _check_lse_inf_pattern(got, ref, what, bar=LSE_MAX_ABS):
    got = np.asarray(got, np.float64)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{what}: -inf rows differ"
    fin = np.isfinite(ref)
    err = float(np.abs(got[fin] - ref[fin]).max()) if fin.any() else 0.0
    assert err <= bar, f"{what}: lse max|err| {err}"


def _check_partial(o_gpu, lse_gpu, o_ref, lse_ref, what):
    """fp32 partial O (no output rounding): the bar of the bf16 output."""
    o_gpu = np.asarray(o_gpu, np.float64)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite partial O"
    err = np.abs(o_gpu - o_ref)
    denom = float(np.linalg.norm(o_ref))
    rel = float(np.linalg.norm(o_gpu - o_ref)) / denom if denom > 0 else float(err.max())
    say(f"  {what}: partial O max|err|={err.max():.3e} relL2={rel:.3e}")
    assert float(err.max()) <= O_MAX_ABS and rel <= O_REL_L2, what
    _check_lse_inf_pattern(lse_gpu, lse_ref, what, lse_bar(o_gpu.shape[-1]))


SPLIT_CASES = [
    # B, H_Q, H_KV, N_q, N_kv, d, causal, S
    (1, 4, 2, 300, 1000, 128, True, 1),
    (1, 4, 2, 300, 1000, 128, False, 3),
    (1, 4, 2, 300, 1000, 128, True, 5),
    (2, 2, 2, 64, 64, 64, True, 2),
    (1, 2, 1, 513, 777, 56, True, 4),
    (1, 2, 2, 40, 40, 128, False, 4),       # chunk 32: splits 2 and 3 are empty
    (1, 2, 2, 200, 100, 128, True, 2),      # N_q > N_kv: early rows see no key
    (2, 8, 2, 1, 3000, 128, True, 8),       # decode, GQA (packed: 4 heads per unit)
    (1, 4, 4, 7, 4096, 64, True, 16),
    # GQA with N_q < 256: the heads of a KV group share the rows of a workgroup
    (1, 8, 2, 37, 1000, 128, True, 3),      # units of 148 rows
    (2, 16, 2, 100, 700, 64, True, 2),      # units of 800 rows: heads wrap inside blocks
    (1, 8, 1, 255, 255, 128, True, 1),      # one unit of 2040 rows, N_q == N_kv
    (1, 6, 3, 90, 2500, 56, False, 5),
    # units of at most 64 rows run the one-wave decode kernel; the rest the
    # 256-row kernel: both sides of the boundary
    (1, 8, 1, 8, 500, 128, True, 3),        # packed unit of 64 rows: decode kernel
    (1, 8, 1, 9, 500, 128, True, 3),        # packed unit of 72 rows
    (1, 2, 2, 64, 64, 128, True, 1),        # 64 rows, one split
    (1, 2, 2, 65, 65, 64, False, 1),        # 65 rows
    (1, 4, 2, 3, 1000, 56, True, 4),        # decode kernel with d = 56 (padded columns)
    (2, 3, 3, 33, 2000, 96, True, 7),       # two 32-row blocks of the decode kernel
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=str)
def test_split_partials_and_merge_match_oracle(case):
    B, H_Q, H_KV, N_q, N_kv, d, causal, S = case
    say(f"case split {case}")
    q, k, v = _qkv(B, H_Q, H_KV, N_q, N_kv, d, seed=500 + N_q + S)
    o_ws = torch.full((S, B, H_Q, N_q, d), float("nan"), device="cuda") if S > 1 else None
    lse_ws = torch.full((S, B, H_Q, N_q), float("nan"), device="cuda") if S > 1 else None
    o, lse = attn.attn_fwd_split(q, k, v, causal=causal, num_splits=S, o_ws=o_ws, lse_ws=lse_ws)
    torch.cuda.synchronize()
    qh, kh, vh = f64(q), f64(k), f64(v)
    o_ref, lse_ref = oracle.partial_attention(qh, kh, vh, causal, 0, N_kv)
    fin = np.isfinite(lse_ref)
    assert_close(f64(o)[fin], f64(lse)[fin], o_ref[fin], lse_ref[fin], what=f"merged {case}")
    assert np.all(f64(o)[~fin] == 0), "rows with no visible key must be 0"
    _check_lse_inf_pattern(f64(lse), lse_ref, f"merged lse {case}", lse_bar(d))
    if S > 1:
        chunk = attn.attn_split_chunk(N_kv, S)
        for s in range(S):
            a, b = min(s * chunk, N_kv), min((s + 1) * chunk, N_kv)
            po, pl = oracle.partial_attention(qh, kh, vh, causal, a, b)
            _check_partial(f64(o_ws[s]), f64(lse_ws[s]), po, pl, f"split {s} [{a},{b}) of {case}")


@pytest.mark.parametrize("causal", [False, True])
def test_single_split_equals_attn_fwd_bitwise(causal):
    q, k, v = _qkv(1, 8, 2, 1100, 1100, 128, seed=77)
    for mapping in (0, 3):
        o1, l1 = attn.attn_fwd(q, k, v, causal=causal, mapping=mapping)
        o2, l2 = attn.attn_fwd_split(q, k, v, causal=causal, num_splits=1, mapping=mapping)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("N_q", [300, 60])   # 60: packed rows
def test_split_bitwise_identical_across_mappings(N_q):
    q, k, v = _qkv(2, 8, 4, N_q, 2000, 128, seed=78)
    ref = None
    for mapping in range(16):
        o, l = attn.attn_fwd_split(q, k, v, causal=True, num_splits=6, mapping=mapping)
        torch.cuda.synchronize()
        if ref is None:
            ref = (o.clone(), l.clone())
        else:
            assert torch.equal(o, ref[0]) and torch.equal(l, ref[1]), mapping


def test_decode_long_kv_every_head():
    """Decode at 64K keys, GQA 64/8, 32 splits: every row checked in full."""
    B, H_Q, H_KV, N_kv, d, S = 2, 64, 8, 65536, 128, 32
    q, k, v = _qkv(B, H_Q, H_KV, 1, N_kv, d, seed=79)
    o, lse = attn.attn_fwd_split(q, k, v, causal=True, num_splits=S)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.partial_attention(f64(q), f64(k), f64(v), True, 0, N_kv)
    assert_close(f64(o), f64(lse), o_ref, lse_ref, what="decode 64K x 32 splits")


def test_merge_kernel_matches_oracle():
    rng = np.random.default_rng(5)
    S, B, H_Q, N_q, d = 5, 2, 3, 33, 64
    o_parts = rng.standard_normal((S, B, H_Q, N_q, d)).astype(np.float32)
    lse_parts = (rng.standard_normal((S, B, H_Q, N_q)) * 3).astype(np.float32)
    lse_parts[1, 0, 0, :] = -np.inf          # one empty part
    lse_parts[:, 1, 2, 7] = -np.inf          # a row with no keys at all
    o_parts[:, 1, 2, 7] = 0.0
    op = torch.from_numpy(o_parts).cuda()
    lp = torch.from_numpy(lse_parts).cuda()
    o, lse = attn.attn_merge(op, lp)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.merge(o_parts.astype(np.float64), lse_parts.astype(np.float64))
    fin = np.isfinite(lse_ref)
    assert_close(f64(o)[fin], f64(lse)[fin], o_ref[fin], lse_ref[fin], what="merge")
    assert np.all(f64(o)[~fin] == 0)
    _check_lse_inf_pattern(f64(lse), lse_ref, "merge lse")


@pytest.mark.parametrize("causal", [False, True])
def test_packed_rows_agree_with_attn_fwd(causal):
    """N_q == N_kv < 256 with GQA: attn_fwd_split groups the heads of a KV
    group into one row space; the result matches attn_fwd (which does not)
    within the bar, and the oracle."""
    q, k, v = _qkv(1, 16, 2, 200, 200, 128, seed=80)
    o1, l1 = attn.attn_fwd(q, k, v, causal=causal)
    o2, l2 = attn.attn_fwd_split(q, k, v, causal=causal, num_splits=1)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(f64(q), f64(k), f64(v), causal)
    assert_close(f64(o2), f64(l2), o_ref, lse_ref, what="packed split")
    assert_close(f64(o1), f64(l1), o_ref, lse_ref, what="attn_fwd")
