"""The reuse-lag L2 model (chiplet_numa_aware_amd/l2model.py) against closed
forms and against the L2 hit rates rocprofv3 measured on MI355X
(profiles/counters_attn_fwd_<workload>.json, TCC_HIT / (TCC_HIT + TCC_MISS)).

The model covers the swizzled modes, whose XCDs each stream their own ACCs;
those are checked within 6 percentage points.  The collapse of swizzled
head-first under a causal mask at N = 128K with one workgroup per CU (head
dim 128: predicted 1-4%, measured 7-12%, varying between runs) is checked as
a collapse: both below 20%.  With two workgroups per CU (head dim <= 64) the
measured rate of that case is 38% against 6% predicted: the model misses
the reuse between the two workgroups of a CU there, so it is reported, not
checked.  It does not model the naive
modes' traffic across XCDs (measured naive head-first under a causal mask
keeps ~70% where the model predicts 12-52%); those are reported, not checked.
"""
import glob
import json
import os

import pytest

import bench
from chiplet_numa_aware_amd import l2model

PROFILES = os.path.join(os.path.dirname(os.path.dirname(__file__)), "profiles")
MODE_IDS = {"swizzled_block_first": 2, "swizzled_head_first": 3,
            "swizzled_head_first_longest_first": 7, "naive_head_first": 1,
            "naive_block_first": 0}


def _measured():
    out = []
    for path in sorted(glob.glob(os.path.join(PROFILES, "counters_attn_fwd_*.json"))):
        with open(path) as f:
            data = json.load(f)
        if data["workload"] in bench.WORKLOADS:
            out.append((data["workload"], data["modes"]))
    return out


def test_shf_non_causal_closed_form():
    """One ACC per XCD, equal workgroups started 32 at a time: each tile is
    fetched once per batch of 32, so the hit rate is exactly 1 - 1/32."""
    for B, H_Q, H_KV, N in [(1, 128, 128, 131072), (1, 64, 8, 32768), (2, 16, 16, 16384)]:
        assert l2model.predict_hit(B, H_Q, H_KV, N, 128, False, 3) == pytest.approx(1 - 1 / 32)


def test_sbf_mha_has_no_reuse():
    """Swizzled block-first gives each XCD 32 consecutive heads of one row
    block: no two concurrent workgroups share K/V."""
    assert l2model.predict_hit(1, 128, 128, 32768, 128, False, 2) == 0.0


def test_model_matches_measured_where_it_claims():
    rows = _measured()
    checked = 0
    for workload, modes in rows:
        B, H_Q, H_KV, N, d, causal = bench.WORKLOADS[workload]
        for name, mode in MODE_IDS.items():
            if name not in modes:
                continue
            pred = 100 * l2model.predict_hit(B, H_Q, H_KV, N, d, causal, mode)
            meas = modes[name]["l2_hit_pct"]
            # within 6 points: longest first, SHF non-causal, SBF at N >= 32K
            # with one workgroup per CU; SBF with two workgroups per CU
            # (d <= 64): no reuse between workgroups predicted, and the
            # measured rate stays below 10% (a floor of up to 7% from traffic
            # the model leaves out); the collapse of SHF under a causal mask
            # at N = 128K with one workgroup per CU: both < 20%
            if mode == 2 and N >= 32768 and l2model.workgroups_per_cu(d) == 2:
                assert pred == 0.0 and meas < 10.0, (workload, name, pred, meas)
            elif mode == 7 or (mode == 3 and not causal) or (mode == 2 and N >= 32768):
                assert abs(pred - meas) <= 6.0, (workload, name, pred, meas)
            elif mode == 3 and causal and N >= 131072 and l2model.workgroups_per_cu(d) == 1:
                assert pred < 20.0 and meas < 20.0, (workload, name, pred, meas)
            else:
                continue
            checked += 1
    assert checked >= 10


def test_longest_first_is_best_under_causal_in_model_and_measurement():
    checked = 0
    for workload, modes in _measured():
        B, H_Q, H_KV, N, d, causal = bench.WORKLOADS[workload]
        name_lf = "swizzled_head_first_longest_first"
        if not causal or name_lf not in modes or N < 32768:
            continue
        meas = {n: modes[n]["l2_hit_pct"] for n in MODE_IDS if n in modes}
        assert max(meas, key=meas.get) == name_lf, (workload, meas)
        checked += 1
        if l2model.workgroups_per_cu(d) > 1:
            # two workgroups per CU: not modelled (see the module notes); the
            # measured ranking above is still checked
            continue
        pred = {n: l2model.predict_hit(B, H_Q, H_KV, N, d, causal, m) for n, m in MODE_IDS.items()}
        assert max(pred, key=pred.get) == name_lf, (workload, pred)
    assert checked >= 4


def test_best_mapping():
    assert l2model.best_mapping(1, 128, 128, 131072, 128, True) == 7
    assert l2model.best_mapping(1, 64, 8, 32768, 128, True) == 7
    assert l2model.best_mapping(1, 128, 128, 131072, 128, False) == 3
