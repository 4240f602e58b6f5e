"""The fp64 oracle against facts fixed outside it (CPU only)."""
import numpy as np
import pytest
import torch

import oracle
from chiplet_numa_aware_amd import inputs
from tests import oracle_pins


def _attn(q, k, v, causal):
    return oracle.attention(q, k, v, causal)


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(_attn)


def test_row_chunking_does_not_change_rows():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 2, 50, 8))
    k = rng.standard_normal((1, 1, 50, 8))
    v = rng.standard_normal((1, 1, 50, 8))
    for causal in (False, True):
        o1, l1 = oracle.attention(q, k, v, causal, row_chunk=7)
        o2, l2 = oracle.attention(q, k, v, causal, row_chunk=64)
        assert np.max(np.abs(o1 - o2)) <= 1e-14
        assert np.max(np.abs(l1 - l2)) <= 1e-14


def test_sampled_rows_match_full():
    q, k, v = inputs.make_qkv(2, 4, 2, 300, 16, seed=11)
    qf, kf, vf = (t.double().numpy() for t in (q, k, v))
    samples = inputs.sample_rows(2, 4, 2, 300, n_pairs=5, n_rows=9, seed=3)
    for causal in (False, True):
        o, lse = oracle.attention(qf, kf, vf, causal)
        for b, h, rows, o_r, l_r in oracle.attention_sampled(qf, kf, vf, causal, samples):
            assert np.max(np.abs(o[b, h, rows] - o_r)) <= 1e-13
            assert np.max(np.abs(lse[b, h, rows] - l_r)) <= 1e-13


def test_inputs_are_bf16_normal_and_seeded():
    a = inputs.normal_bf16((4, 1000), seed=5)
    b = inputs.normal_bf16((4, 1000), seed=5)
    c = inputs.normal_bf16((4, 1000), seed=6)
    assert a.dtype == torch.bfloat16
    assert torch.equal(a, b) and not torch.equal(a, c)
    x = a.double()
    assert abs(x.mean().item()) < 0.05 and abs(x.std().item() - 1.0) < 0.05
    # bf16 -> fp64 is exact: the low 16 bits of the fp32 image are zero.
    bits = a.float().view(torch.int32)
    assert torch.all((bits & 0xFFFF) == 0)


def test_sample_rows_contract():
    for B, H_Q, H_KV, N in [(1, 128, 128, 131072), (1, 64, 8, 8192),
                            (2, 32, 4, 32768), (1, 8, 8, 1024), (1, 2, 1, 5)]:
        s = inputs.sample_rows(B, H_Q, H_KV, N)
        pairs = [(b, h) for b, h, _ in s]
        assert len(pairs) == len(set(pairs)) == min(16, B * H_Q)
        assert (0, 0) in pairs and (B - 1, H_Q - 1) in pairs
        if B * H_KV <= 16:
            G = H_Q // H_KV
            assert {(b, h // G) for b, h in pairs} >= {(b, g) for b in range(B) for g in range(H_KV)}
        for _, _, rows in s:
            assert len(rows) == min(32, N) and len(set(rows.tolist())) == len(rows)
            assert rows.min() >= 0 and rows.max() < N
            for r in (0, 1, 127, 128, N // 2, N - 2, N - 1):
                if 0 <= r < N:
                    assert r in rows
        assert inputs.sample_rows(B, H_Q, H_KV, N)[0][2].tolist() == s[0][2].tolist()
