"""The CAC-scheduled GEMM (cac_gemm) on the GPU against the fp64 oracle
(oracle/gemm.py), through the C ABI.  Every element must lie within the
rounding bound of bf16 inputs, fp32 accumulation and a bf16 result
(tests/gpu_util.check_gemm); integer inputs whose sums bf16 holds exactly
must come back bit-exact; the tile map must not change any bit of C."""
import numpy as np
import pytest
import torch

import chiplet_numa_aware_amd as attn
import oracle
from chiplet_numa_aware_amd import inputs
from tests.gpu_util import check_gemm, f64, say

pytestmark = pytest.mark.gpu


def _ab(L, M, N, K, seed):
    a = inputs.normal_bf16((L, M, K), seed, "cuda")
    b = inputs.normal_bf16((L, N, K), seed + 1, "cuda")
    return a, b


CASES = [
    # L, M, N, K
    (1, 256, 256, 32),        # one tile, one K step
    (1, 300, 136, 72),        # ragged M, N, K (K tail of 8)
    (2, 513, 264, 1000),      # batches, one row past a tile, K not a multiple of 32
    (1, 1, 8, 8),             # smallest shape
    (3, 700, 520, 256),
    (1, 1024, 2048, 96),      # 4 x 8 tiles: one default cluster
]


@pytest.mark.parametrize("case", CASES, ids=str)
def test_gemm_matches_oracle(case):
    L, M, N, K = case
    say(f"case gemm {case}")
    a, b = _ab(L, M, N, K, seed=700 + M + K)
    for mapping in (0, 3):
        c = attn.cac_gemm(a, b, mapping=mapping)
        torch.cuda.synchronize()
        check_gemm(f64(c), f64(a), f64(b), f"gemm {case} mapping {mapping}")


def test_gemm_exact_on_integers():
    """Entries in {-1, 0, 1} and K = 96: every partial sum is an integer of
    magnitude <= 96, exact in fp32 and in bf16, so C is bit-exact."""
    g = torch.Generator(device="cuda").manual_seed(5)
    L, M, N, K = 2, 333, 264, 96
    a = torch.randint(-1, 2, (L, M, K), generator=g, device="cuda").to(torch.bfloat16)
    b = torch.randint(-1, 2, (L, N, K), generator=g, device="cuda").to(torch.bfloat16)
    c = attn.cac_gemm(a, b, mapping=3)
    torch.cuda.synchronize()
    assert np.array_equal(f64(c), oracle.gemm(f64(a), f64(b)))


def test_gemm_bitwise_identical_across_maps():
    a, b = _ab(2, 1100, 1800, 200, seed=710)
    ref = None
    for mapping in range(4):
        for gm, gn in ((0, 0), (1, 1), (3, 5), (2, 8)):
            c = attn.cac_gemm(a, b, mapping=mapping, group_m=gm, group_n=gn)
            torch.cuda.synchronize()
            if ref is None:
                ref = c.clone()
            else:
                assert torch.equal(c, ref), (mapping, gm, gn)


def test_gemm_2d_and_prefilled_output():
    a = inputs.normal_bf16((520, 264), 720, "cuda")
    b = inputs.normal_bf16((392, 264), 721, "cuda")
    c = torch.full((520, 392), float("nan"), dtype=torch.bfloat16, device="cuda")
    attn.cac_gemm(a, b, c=c)
    torch.cuda.synchronize()
    assert torch.isfinite(c.float()).all()
    check_gemm(f64(c), f64(a), f64(b), "2-D, NaN-prefilled C")


@pytest.mark.parametrize("mapping", [0, 3])
def test_gemm_full_size_sampled_rows(mapping):
    """The benchmark's tall shape (M=65536, N=2048, K=8192) in its launch
    configuration; 64 seeded rows of C against the oracle, row by row."""
    L, M, N, K = 1, 65536, 2048, 8192
    a, b = _ab(L, M, N, K, seed=1000)
    c = attn.cac_gemm(a, b, mapping=mapping)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(1234))
    rows = np.unique(np.concatenate([[0, 255, 256, M // 2, M - 1], rng.choice(M, 59, replace=False)]))
    ridx = torch.as_tensor(rows, device="cuda")
    check_gemm(f64(c[0].index_select(0, ridx)), f64(a[0].index_select(0, ridx)), f64(b[0]),
               f"tall GEMM sampled rows, mapping {mapping}")


@pytest.mark.parametrize("shape", [(8, 16384, 1024, 4096), (1, 16384, 16384, 16384)],
                         ids=["batched_L8_16k_1k_4k", "square_16k"])
def test_gemm_full_size_batched_and_square(shape):
    """The benchmark's batched (L=8) and square shapes in their launch
    configuration (swizzled cluster map, default cluster): seeded rows of C of
    every batch against the oracle under the rigorous bound (32 rows per
    batch for L=8, 48 rows for the square)."""
    L, M, N, K = shape
    say(f"case GEMM full size L={L} M={M} N={N} K={K}")
    a, b = _ab(L, M, N, K, seed=1000)
    c = attn.cac_gemm(a, b, mapping=3)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(1234))
    n = 32 if L > 1 else 48
    for l in range(L):
        rows = np.unique(np.concatenate([[0, 255, 256, M - 1], rng.choice(M, n - 4, replace=False)]))
        ridx = torch.as_tensor(rows, device="cuda")
        check_gemm(f64(c[l].index_select(0, ridx)), f64(a[l].index_select(0, ridx)), f64(b[l]),
                   f"GEMM L={L} M={M} N={N} K={K} batch {l} sampled rows")
    del a, b, c
    torch.cuda.empty_cache()
