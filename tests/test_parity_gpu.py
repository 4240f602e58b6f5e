"""HIP attention forward (through the C ABI) against the fp64 oracle, on sizes
the oracle finishes in seconds: every output element is compared."""
import math

import numpy as np
import pytest
import torch

import chiplet_numa_aware_amd as attn
import oracle
from chiplet_numa_aware_amd import inputs
from tests.gpu_util import assert_close, f64, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _run(q, k, v, causal, mapping=3):
    o, lse = attn.attn_fwd(q, k, v, causal=causal, mapping=mapping)
    torch.cuda.synchronize()
    return o, lse


def _oracle(q, k, v, causal):
    return oracle.attention(f64(q), f64(k), f64(v), causal)


def test_c1_full_oracle_every_mapping():
    """MHA B=1, H=8, N=1024, d=128, non-causal: all outputs, all 8 mappings,
    bit-identical across mappings."""
    say("case C1 B=1 H=8 N=1024 d=128 non-causal seed=100")
    q, k, v = inputs.make_qkv(1, 8, 8, 1024, 128, seed=100, device="cpu")
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    o_ref, lse_ref = _oracle(q, k, v, False)
    outs = []
    for mapping in range(16):
        o, lse = _run(q, k, v, False, mapping)
        assert_close(f64(o), f64(lse), o_ref, lse_ref, f"C1 mapping {mapping}")
        outs.append((o.clone(), lse.clone()))
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])


SMALL = [
    # B, H_Q, H_KV, N, d, causal
    (1, 2, 2, 1, 128, False),
    (1, 2, 2, 1, 128, True),
    (1, 2, 1, 5, 64, True),
    (2, 4, 2, 100, 128, True),
    (1, 3, 3, 129, 56, False),
    (1, 3, 3, 129, 56, True),
    (1, 2, 2, 1000, 8, True),
    (1, 4, 4, 300, 72, False),
    (2, 8, 2, 640, 128, True),
    (1, 1, 1, 257, 120, True),
    (1, 16, 16, 512, 64, False),
    (1, 8, 8, 2048, 128, True),
    (3, 6, 3, 384, 96, False),
    (1, 12, 12, 1100, 128, True),
    (1, 6, 2, 333, 128, True),      # GQA, 3 query heads per KV head
    (2, 9, 3, 70, 64, False),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}_HQ{}_HKV{}_N{}_d{}_{}".format(
    *s[:5], "causal" if s[5] else "full"))
def test_small_shapes_full_oracle(shape):
    B, H_Q, H_KV, N, d, causal = shape
    say(f"case small {shape}")
    q, k, v = inputs.make_qkv(B, H_Q, H_KV, N, d, seed=7 + N + d, device="cpu")
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    o_ref, lse_ref = _oracle(q, k, v, causal)
    # 15 = swizzled head-first + longest first + balanced split: several of
    # these shapes have ACCs that a slice boundary splits (e.g. H=12, N=1100:
    # 5 row blocks per ACC, 7-8 workgroups per XCD).
    outs = []
    for mapping in (0, 3, 15):
        o, lse = _run(q, k, v, causal, mapping)
        assert_close(f64(o), f64(lse), o_ref, lse_ref, f"{shape} mapping {mapping}")
        outs.append((o, lse))
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])


@pytest.mark.parametrize("causal", [False, True])
def test_q_zero_gives_mean_of_v(causal):
    """All-equal scores: O_i = mean of the visible V rows, lse_i = ln |J|.
    On the GPU every P is exactly 1, so only the fp32 sum and the final bf16
    rounding separate O from the closed form."""
    B, H, N, d = 1, 4, 700, 128
    say(f"case q=0 causal={causal}")
    _, k, v = inputs.make_qkv(B, H, H, N, d, seed=31, device="cpu")
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16)
    o, lse = _run(q.to(DEV), k.to(DEV), v.to(DEV), causal)
    vf = f64(v)[0]
    cnt = np.arange(1, N + 1)[:, None] if causal else N
    mean = (np.cumsum(vf, axis=1) / cnt) if causal else np.broadcast_to(
        vf.mean(axis=1, keepdims=True), vf.shape)
    og = f64(o)[0]
    tol = 2.0 ** -8 * np.abs(mean) + 1e-5
    assert np.all(np.abs(og - mean) <= tol)
    lse_exp = np.log(np.arange(1, N + 1)) if causal else np.full(N, math.log(N))
    assert np.max(np.abs(f64(lse)[0] - lse_exp[None, :])) <= 1e-5


def test_causal_row0_is_v0_bit_exact():
    B, H_Q, H_KV, N, d = 2, 4, 2, 300, 128
    say("case causal row 0")
    q, k, v = inputs.make_qkv(B, H_Q, H_KV, N, d, seed=41, device=DEV)
    o, lse = _run(q, k, v, True)
    G = H_Q // H_KV
    for h in range(H_Q):
        assert torch.equal(o[:, h, 0], v[:, h // G, 0])
    s00 = (q[:, :, 0].float() * k.repeat_interleave(G, dim=1)[:, :, 0].float()).sum(-1) / math.sqrt(d)
    assert torch.max(torch.abs(lse[:, :, 0] - s00)).item() <= 1e-4


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_is_bitwise_repeated_mha(causal):
    B, H_Q, H_KV, N, d = 1, 8, 2, 900, 128
    say(f"case gqa==mha causal={causal}")
    q, k, v = inputs.make_qkv(B, H_Q, H_KV, N, d, seed=51, device=DEV)
    G = H_Q // H_KV
    o1, l1 = _run(q, k, v, causal)
    o2, l2 = _run(q, k.repeat_interleave(G, 1).contiguous(),
                  v.repeat_interleave(G, 1).contiguous(), causal)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_batch_slice_is_bitwise():
    B, H_Q, H_KV, N, d = 3, 4, 4, 520, 64
    say("case batch slice")
    q, k, v = inputs.make_qkv(B, H_Q, H_KV, N, d, seed=61, device=DEV)
    o, lse = _run(q, k, v, True)
    for b in range(B):
        ob, lb = _run(q[b:b + 1].contiguous(), k[b:b + 1].contiguous(),
                      v[b:b + 1].contiguous(), True)
        assert torch.equal(ob[0], o[b]) and torch.equal(lb[0], lse[b])


def test_one_hot_row():
    """K[j*] = c * Q[i] with a large score margin: O_i is V[j*]."""
    N, d = 256, 128
    say("case one-hot")
    q, k, v = inputs.make_qkv(1, 1, 1, N, d, seed=71, device="cpu")
    q = (q.float() * 0.05).to(torch.bfloat16)
    k = (k.float() * 0.05).to(torch.bfloat16)
    i, js = 200, 77
    qi = q[0, 0, i].double()
    c = 60.0 * math.sqrt(d) / float(qi @ qi)
    k[0, 0, js] = (c * q[0, 0, i].float()).to(torch.bfloat16)
    for causal in (False, True):
        o, lse = _run(q.to(DEV), k.to(DEV), v.to(DEV), causal)
        assert torch.max(torch.abs(o[0, 0, i].float().cpu() - v[0, 0, js].float())).item() <= 1e-2


@pytest.mark.parametrize("margin", [30.0, 300.0])
def test_score_jump_in_a_later_tile_every_element(margin):
    """One key row far down the sequence scores `margin` (natural units)
    above the rest for query row i: with 30 the running max is stale by
    ~43 log2 units when that tile arrives, with 300 by ~430, beyond the fp32
    range of exp2.  Every element of O and lse against the oracle, causal and
    not, and the same result under every mapping."""
    B, H, N, d = 1, 2, 2048, 128
    say(f"case score jump margin={margin}")
    q, k, v = inputs.make_qkv(B, H, H, N, d, seed=91, device="cpu")
    i, js = 1800, 1500
    for h in range(H):
        qi = q[0, h, i].double()
        c = margin * math.sqrt(d) / float(qi @ qi)
        k[0, h, js] = (c * q[0, h, i].float()).to(torch.bfloat16)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    for causal in (False, True):
        o_ref, lse_ref = _oracle(q, k, v, causal)
        o0, l0 = _run(q, k, v, causal, 0)
        assert_close(f64(o0), f64(l0), o_ref, lse_ref, f"jump {margin} causal={causal}")
        for mapping in (3, 7, 15):
            o, lse = _run(q, k, v, causal, mapping)
            assert torch.equal(o, o0) and torch.equal(lse, l0), mapping


def test_lse_may_be_null_and_o_is_unchanged():
    B, H, N, d = 1, 2, 333, 128
    say("case lse=NULL")
    q, k, v = inputs.make_qkv(B, H, H, N, d, seed=81, device=DEV)
    o1, _ = _run(q, k, v, True)
    o2, lse2 = attn.attn_fwd(q, k, v, causal=True, need_lse=False)
    torch.cuda.synchronize()
    assert lse2 is None and torch.equal(o1, o2)


def test_runs_on_a_side_stream():
    B, H, N, d = 1, 2, 256, 128
    say("case side stream")
    q, k, v = inputs.make_qkv(B, H, H, N, d, seed=91, device=DEV)
    o1, l1 = _run(q, k, v, False)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o2, l2 = attn.attn_fwd(q, k, v, causal=False, stream=s)
    s.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("shape", [(1, 3, 3, 129, 56, False), (1, 2, 2, 130, 128, True),
                                   (2, 4, 2, 200, 64, False)], ids=str)
def test_repeated_launches_identical(shape):
    """Shapes with idle waves and key tiles past the end, launched 30 times:
    every result is bit-identical and within the bar.  (Loads of tile 4 into
    the K buffer the prologue reads for tile 0 must wait for every wave's
    reads; a wave that got ahead made this shape wrong now and then.)"""
    B, H_Q, H_KV, N, d, causal = shape
    q, k, v = inputs.make_qkv(B, H_Q, H_KV, N, d, seed=11 + N, device="cpu")
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    o_ref, lse_ref = _oracle(q, k, v, causal)
    first = None
    for i in range(30):
        o, lse = _run(q, k, v, causal, 3 if i % 2 else 0)
        if first is None:
            assert_close(f64(o), f64(lse), o_ref, lse_ref, f"{shape} launch 0")
            first = (o.clone(), lse.clone())
        else:
            assert torch.equal(o, first[0]) and torch.equal(lse, first[1]), f"launch {i} differs"


@pytest.mark.parametrize("d", [128, 64])
def test_running_max_raised_inside_steady_tiles(d):
    """Key rows scaled by 1 + j/64, so the scores of later key tiles grow and
    the running max is raised every few tiles in the middle of the pipelined
    loop (a raise leaves the loop and resumes at the same tile); every
    element against the oracle, the same result under all 8 mappings, and
    repeated launches bit-identical."""
    B, H, N = 1, 2, 2048
    say(f"case growing scores d={d}")
    q, k, v = inputs.make_qkv(B, H, H, N, d, seed=123 + d, device="cpu")
    grow = (1.0 + torch.arange(N, dtype=torch.float32) / 64.0).view(1, 1, N, 1)
    k = (k.float() * grow).to(torch.bfloat16)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    for causal in (False, True):
        o_ref, lse_ref = _oracle(q, k, v, causal)
        o0, l0 = _run(q, k, v, causal, 0)
        assert_close(f64(o0), f64(l0), o_ref, lse_ref, f"growing d={d} causal={causal}")
        for mapping in range(1, 8):
            o, lse = _run(q, k, v, causal, mapping)
            assert torch.equal(o, o0) and torch.equal(lse, l0), f"mapping {mapping} differs"
        for _ in range(3):
            o, lse = _run(q, k, v, causal, 3)
            assert torch.equal(o, o0) and torch.equal(lse, l0), "repeated launch differs"
