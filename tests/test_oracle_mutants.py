"""Plant plausible mistakes in the oracle (CPU only) and check that the pins
of tests/oracle_pins.py catch every one of them."""
import numpy as np
import pytest

import oracle
import oracle.sdpa as oa
from tests import oracle_pins


def _mutant_rows(bug):
    def rows_fn(q_rows, k_head, v_head, rows, causal):
        q_rows = np.asarray(q_rows, dtype=np.float64)
        k_head = np.asarray(k_head, dtype=np.float64)
        v_head = np.asarray(v_head, dtype=np.float64)
        rows = np.asarray(rows, dtype=np.int64)
        d = q_rows.shape[1]
        n = k_head.shape[0]
        scale = 1.0 / d if bug == "scale_1_over_d" else 1.0 / np.sqrt(d)
        s = (q_rows @ k_head.T) * scale
        if bug == "scores_transposed" and s.shape[0] == s.shape[1]:
            s = s.T
        if causal:
            keys = np.arange(n)[None, :]
            if bug == "mask_off_by_one":
                s = np.where(keys <= rows[:, None] + 1, s, -np.inf)
            elif bug == "mask_upper":
                s = np.where(keys >= rows[:, None], s, -np.inf)
            else:
                s = np.where(keys <= rows[:, None], s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        ell = e.sum(axis=1, keepdims=True)
        p = e / ell
        o = p @ (k_head if bug == "pv_uses_k" else v_head)
        if bug == "lse_without_max":
            lse = np.log(ell)[:, 0]
        elif bug == "lse_log2":
            lse = ((m + np.log(ell)) / np.log(2.0))[:, 0]
        else:
            lse = (m + np.log(ell))[:, 0]
        if bug == "o_not_normalised":
            o = e @ v_head
        return o, lse
    return rows_fn


BUGS = ["scale_1_over_d", "scores_transposed", "mask_off_by_one", "mask_upper",
        "pv_uses_k", "lse_without_max", "lse_log2", "o_not_normalised",
        "gqa_modulo_heads"]


@pytest.mark.parametrize("bug", BUGS)
def test_pins_catch_planted_mistake(bug, monkeypatch):
    if bug == "gqa_modulo_heads":
        monkeypatch.setattr(oa, "kv_head", lambda h, H_Q, H_KV: h % H_KV)
    else:
        monkeypatch.setattr(oa, "attention_head_rows", _mutant_rows(bug))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(lambda q, k, v, c: oa.attention(q, k, v, c))
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {bug}"


def test_unmutated_oracle_passes_every_pin():
    for pin in oracle_pins.ALL_PINS:
        pin(lambda q, k, v, c: oracle.attention(q, k, v, c))
