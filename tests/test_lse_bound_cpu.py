"""The lse bar for head dims below the padded width rests on a bound: the
row sum l is accumulated from the bf16-rounded P (the P V MFMA sums the row
through a 1 in V's padding), each term within a relative 2^-8 of the fp32
value (an 8-bit significand rounded to nearest even), so

    |ln(sum bf16(p_i)) - ln(sum p_i)| <= ln(1 + 2^-8) ~= 3.9e-3,

under the test bar of 4e-3.  This checks the bound numerically with torch's
round-to-nearest-even bf16 conversion, including the worst case (p values
whose significands sit just above a power of two, as a stale running max
produces) and the exact cases (p = 1 and powers of two).
"""
import math

import numpy as np
import torch

from tests.gpu_util import LSE_MAX_ABS_PADDED

BOUND = math.log1p(2.0 ** -8)


def _lse_gap(p: np.ndarray) -> float:
    p32 = torch.from_numpy(p.astype(np.float32))
    pb = p32.to(torch.bfloat16).to(torch.float64)
    return abs(math.log(float(pb.sum())) - math.log(float(p32.to(torch.float64).sum())))


def test_bound_is_under_the_bar():
    assert BOUND < LSE_MAX_ABS_PADDED


def test_random_rows_with_a_stale_max():
    rng = np.random.default_rng(17)
    worst = 0.0
    for n in (1, 2, 3, 8, 32, 100, 4096):
        for _ in range(200):
            s = rng.standard_normal(n) * rng.uniform(0.1, 8.0)
            stale = rng.uniform(0.0, 8.0)  # the running max lags the row max
            p = np.exp2(s - (s.max() - stale))
            worst = max(worst, _lse_gap(p))
    assert worst <= BOUND, worst


def test_worst_case_rounding_reaches_but_does_not_pass_the_bound():
    # One dominant term 1 + 2^-8 + tiny (rounds to 1, relative error just
    # under 2^-8): the gap approaches ln(1 + 2^-8) from below.
    p = np.array([1.0 + 2.0 ** -8 + 2.0 ** -20], dtype=np.float64)
    gap = _lse_gap(p)
    assert 0.99 * BOUND < gap <= BOUND, gap
    # Many such terms: the relative errors share a sign but cannot exceed it.
    p = np.full(1000, 3.0 * (1.0 + 2.0 ** -8 + 2.0 ** -20))
    assert _lse_gap(p) <= BOUND


def test_exact_when_p_is_a_power_of_two():
    p = np.array([1.0, 0.5, 0.25, 2.0 ** -10])
    assert _lse_gap(p) == 0.0
