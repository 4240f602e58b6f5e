"""Where the hardware runs each workgroup (XCC id register), against the
dispatch model the remap relies on: linear workgroup id w goes to XCD
(w mod X) in chunks of one ("Optimizing Attention on GPUs by Exploiting GPU
Architectural NUMA Effects", digest page §2 Q1), so Swizzled Head-first keeps
each ACC on one XCD when X divides the number of ACCs."""
from collections import defaultdict

import numpy as np
import pytest
import torch

import chiplet_numa_aware_amd as attn
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

SHAPES = [(1, 128, 128, 131072), (1, 64, 8, 32768), (2, 32, 4, 32768),
          (1, 12, 12, 32768), (1, 8, 8, 1024)]


def test_num_xcd_reports_device_and_override(monkeypatch):
    X = attn.attn_num_xcd()
    say(f"attn_num_xcd() = {X}")
    assert X >= 1
    monkeypatch.setenv("ATTN_NUM_XCD", "4")
    assert attn.attn_num_xcd() == 4
    monkeypatch.setenv("ATTN_NUM_XCD", "junk")
    assert attn.attn_num_xcd() == X


@pytest.mark.parametrize("shape", SHAPES, ids=str)
def test_probe_matches_host_table_and_dispatch_model(shape):
    B, H_Q, H_KV, N = shape
    X = attn.attn_num_xcd()
    say(f"case probe {shape} X={X}")
    for mode in range(16):
        out = attn.attn_probe_placement(mode, B, H_Q, H_KV, N)
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        table = attn.attn_wg_map(mode, B, H_Q, H_KV, N, X)
        assert np.array_equal(out[:, 1:], table)
        xcc = out[:, 0]
        w = np.arange(out.shape[0])
        # The same residue class w mod X always lands on the same XCC.
        for r in range(X):
            assert np.unique(xcc[w % X == r]).size == 1, (mode, r)
        assert np.unique(xcc).size == min(X, out.shape[0])
        if mode & 3 == 3 and (B * H_KV) % X == 0:
            acc = out[:, 1] * H_KV + out[:, 2] // (H_Q // H_KV)
            per = defaultdict(set)
            for a, x in zip(acc, xcc):
                per[int(a)].add(int(x))
            assert all(len(s) == 1 for s in per.values())
