"""Every memory access of cac_gemm_kernel stays inside A, B and C (CPU).

A model of the kernel's address arithmetic (csrc/gemm_kernel.hpp, with its
constants read from that header) enumerated over every workgroup of the
library's own tile map (cac_gemm_map) at the benchmark's shapes, including
the batched one (L=8, M=16384, N=1024, K=4096).  Per batch the kernel
addresses A[l], B[l] and C[l] through buffer descriptors whose base is the
64-bit offset of batch l and whose size is that batch's bytes; the hardware
drops any 32-bit offset at or past the size.  So the kernel stays inside
the tensors if (1) every base + size lies inside the tensor, (2) the 32-bit
offsets never wrap (a wrapped offset would look in range), and (3) every
access is 16-byte aligned against a 16-byte-multiple size (whole accesses
in or out).  The tests check these for every tile, load and K step, and
that the stores touch only C's elements.
"""
import os
import re

import numpy as np
import pytest

import chiplet_numa_aware_amd as attn

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "chiplet_numa_aware_amd", "csrc", "gemm_kernel.hpp")


def _consts():
    text = open(HDR).read()
    c = {}
    for name in ("kGemmTile", "kGemmBK", "kGemmThreads"):
        c[name] = int(re.search(rf"constexpr int {name} = (\d+);", text).group(1))
    c["kGemmCPR"] = c["kGemmBK"] // 8
    c["kGemmLoads"] = c["kGemmTile"] * c["kGemmBK"] * 2 // 16 // c["kGemmThreads"]
    return c


OUT_OF_RANGE = 0x80000000  # kOutOfRange of attn_fwd_kernel.hpp


def _check_shape(L, M, N, K, mapping=3):
    c = _consts()
    T, BK, CPR, thr, loads = (c["kGemmTile"], c["kGemmBK"], c["kGemmCPR"],
                              c["kGemmThreads"], c["kGemmLoads"])
    tiles = attn.cac_gemm_map(mapping, L, M, N).astype(np.int64)   # (l, tm, tn) per workgroup
    assert tiles.shape[0] == L * (-(-M // T)) * (-(-N // T))
    l, tm, tn = tiles[:, 0], tiles[:, 1], tiles[:, 2]
    assert l.min() >= 0 and l.max() < L
    a_bytes, b_bytes, c_bytes = M * K * 2, N * K * 2, M * N * 2
    for size in (a_bytes, b_bytes, c_bytes):
        assert size % 16 == 0 and size < 2 ** 32
    # (1) per-batch windows inside the tensors
    assert int((l * M * K * 2 + a_bytes).max()) <= L * M * K * 2
    assert int((l * N * K * 2 + b_bytes).max()) <= L * N * K * 2
    assert int((l * M * N * 2 + c_bytes).max()) <= L * M * N * 2
    # (2) load offsets: soffset (tile row offset, capped) + voffset (row in
    # the tile, K position) for every thread slot, load and K step
    P = np.arange(thr)[:, None] + thr * np.arange(loads)[None, :]
    row = (P // CPR).ravel()
    slot = (P % CPR).ravel()
    n_steps = -(-K // BK)
    for base_rows, size in ((tm * T, a_bytes), (tn * T, b_bytes)):
        soff = np.minimum(base_rows * K * 2, size)
        # the swizzle permutes chunks within a row, so the K positions a row
        # covers per step are those of its slots
        kk = (np.arange(n_steps) * BK)[:, None] + (slot * 8)[None, :]
        voff = np.where(kk < K, row[None, :] * K * 2 + kk * 2, OUT_OF_RANGE)
        vmax, vmin = int(voff.max()), int(voff.min())
        assert int(soff.max()) + vmax < 2 ** 32, "a 32-bit buffer offset would wrap"
        assert vmin >= 0 and vmin % 16 == 0
        assert np.all(voff % 16 == 0) and np.all(soff % 16 == 0)
        # accesses whose offset is below the size lie wholly inside the batch's window
        in_range_max = int(soff.max()) + int(voff[voff < OUT_OF_RANGE].max())
        assert min(in_range_max, size - 16) + 16 <= size or in_range_max >= size
    # (3) stores: row < M and col < N are written, 8 bytes at col % 4 == 0
    rows = tm[:, None] * T + np.arange(T)[None, :]
    cols = tn[:, None] * T + np.arange(0, T, 4)[None, :]
    ok_r = rows < M
    ok_c = cols < N
    off_max = (np.where(ok_r, rows, 0).max(axis=1) * N + np.where(ok_c, cols, 0).max(axis=1)) * 2 + 8
    assert int(off_max.max()) <= c_bytes


@pytest.mark.parametrize("shape", [(8, 16384, 1024, 4096), (1, 16384, 16384, 16384),
                                   (1, 65536, 2048, 8192), (3, 1000, 520, 264),
                                   (2, 300, 1032, 8)],
                         ids=["batched_L8", "square_16k", "tall", "ragged", "tiny_k"])
def test_gemm_accesses_stay_inside_the_operands(shape):
    for mapping in range(4):
        _check_shape(*shape, mapping=mapping)


def test_the_model_catches_a_wrapping_offset():
    """Planted on the CPU: an A larger than 2^31 bytes (which the library's
    size check refuses) would let the capped tile offset plus the
    out-of-range marker pass 2^32; the model's wrap check fires."""
    with pytest.raises(AssertionError, match="wrap"):
        _check_shape(1, 1100000, 256, 1000)
