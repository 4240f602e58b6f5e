"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, rejects bad arguments before touching a device, and its host
remap table equals the independent oracle's."""
import ctypes
import os
import random
import re

import numpy as np
import pytest

import chiplet_numa_aware_amd as attn
import oracle

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "attn_numa.h")


@pytest.fixture(scope="module")
def lib():
    return attn.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def _declared_codes():
    return {m.group(1): int(m.group(2)) for m in re.finditer(
        r"#define\s+(ATTN_E_\w+|ATTN_OK)\s+\(?(-?\d+)\)?", open(HEADER).read())}


def test_library_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) == {"attn_fwd", "attn_fwd_split", "attn_fwd_split_noalloc",
                          "attn_split_chunk", "attn_merge",
                          "attn_bwd", "attn_wg_map", "attn_num_xcd", "attn_block_m",
                          "attn_probe_placement", "attn_strerror"}
    for n in names:
        assert hasattr(lib, n), n


def test_block_m_sizes_the_tables(lib):
    """attn_block_m needs no GPU and sizes attn_wg_map's table."""
    bm = lib.attn_block_m()
    assert bm == attn.BLOCK_M and bm % 64 == 0
    for N in (1, bm - 1, bm, bm + 1, 5 * bm + 7):
        assert attn.attn_wg_map(3, 2, 4, 2, N, 8).shape == (2 * 4 * (-(-N // bm)), 3)


def test_head_size_limit(lib):
    """One head may hold at most 2^31 - 2^16 bytes (the range-checked buffer
    offsets stay below 2^32); the check runs before any device query."""
    c = _declared_codes()
    limit = (1 << 31) - (1 << 16)
    assert limit % 256 == 0
    kw = dict(B=1, H_Q=1, H_KV=1, d=128, causal=0)
    assert _fwd(lib, N=limit // 256 + 1, mapping=3, **kw) == c["ATTN_E_SHAPE"]
    # At the limit the shape passes and the (invalid) mapping is reported:
    # validation ends before anything could launch on the fake pointers.
    assert _fwd(lib, N=limit // 256, mapping=16, **kw) == c["ATTN_E_MAPPING"]


def test_strerror_covers_every_code(lib):
    codes = _declared_codes()
    assert codes["ATTN_OK"] == 0
    texts = set()
    for name, c in codes.items():
        t = attn.attn_strerror(c)
        assert t and t != "unknown error code", name
        texts.add(t)
    assert len(texts) == len(codes)
    assert attn.attn_strerror(12345) == "unknown error code"


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def _fwd(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, H_Q=8, H_KV=8,
         N=1024, d=128, causal=0, mapping=3):
    return lib.attn_fwd(q, k, v, o, lse, B, H_Q, H_KV, N, d, causal, mapping, None)


def test_fwd_argument_errors(lib):
    c = _declared_codes()
    for kw in ({"q": None}, {"k": None}, {"v": None}, {"o": None}):
        assert _fwd(lib, **kw) == c["ATTN_E_NULL"]
    for kw in ({"B": 0}, {"H_Q": 0}, {"H_KV": 0}, {"N": 0}, {"N": -5},
               {"H_Q": 12, "H_KV": 8}, {"B": 1 << 20, "H_Q": 1024, "N": 1 << 20}):
        assert _fwd(lib, **kw) == c["ATTN_E_SHAPE"], kw
    for d in (0, -8, 4, 12, 136, 256):
        assert _fwd(lib, d=d) == c["ATTN_E_HEAD_DIM"], d
    # one head larger than 2 GiB does not fit a buffer resource
    assert _fwd(lib, N=1 << 23, d=128, H_Q=1, H_KV=1) == c["ATTN_E_SHAPE"]
    for m in (-1, 16, 99):
        assert _fwd(lib, mapping=m) == c["ATTN_E_MAPPING"]
    for kw in ({"q": FAKE + 2}, {"k": FAKE + 8}, {"v": FAKE + 1},
               {"o": FAKE + 4}, {"lse": FAKE + 4}):
        assert _fwd(lib, **kw) == c["ATTN_E_ALIGN"], kw


def test_wg_map_and_probe_argument_errors(lib):
    c = _declared_codes()
    buf = np.zeros(64 * 3, dtype=np.int32)
    assert lib.attn_wg_map(3, 1, 8, 8, 1024, 8, None) == c["ATTN_E_NULL"]
    assert lib.attn_wg_map(3, 1, 8, 3, 1024, 8, buf.ctypes.data) == c["ATTN_E_SHAPE"]
    assert lib.attn_wg_map(3, 1, 8, 8, 1024, 0, buf.ctypes.data) == c["ATTN_E_SHAPE"]
    assert lib.attn_wg_map(16, 1, 8, 8, 1024, 8, buf.ctypes.data) == c["ATTN_E_MAPPING"]
    assert lib.attn_probe_placement(3, 1, 8, 8, 1024, None, None) == c["ATTN_E_NULL"]
    assert lib.attn_probe_placement(3, 0, 8, 8, 1024, FAKE, None) == c["ATTN_E_SHAPE"]
    assert lib.attn_probe_placement(16, 1, 8, 8, 1024, FAKE, None) == c["ATTN_E_MAPPING"]
    assert lib.attn_probe_placement(3, 1, 8, 8, 1024, FAKE + 4, None) == c["ATTN_E_ALIGN"]


def _shapes():
    shapes = [(1, 8, 8, 1024, 8), (1, 128, 128, 8192, 8), (1, 64, 8, 131072, 8),
              (2, 32, 4, 32768, 8), (2, 12, 12, 32768, 8), (1, 12, 12, 32768, 8),
              (1, 128, 128, 131072, 8), (1, 8, 8, 128 * 128, 4)]
    rng = random.Random(3)
    for _ in range(150):
        H_KV = rng.randint(1, 9)
        H_Q = H_KV * rng.randint(1, 4)
        shapes.append((rng.randint(1, 4), H_Q, H_KV, rng.randint(1, 2600),
                       rng.choice([1, 2, 3, 4, 6, 8, 16])))
    return shapes


@pytest.mark.parametrize("mode", list(range(16)))
def test_host_wg_map_equals_oracle(mode):
    for B, H_Q, H_KV, N, X in _shapes():
        got = attn.attn_wg_map(mode, B, H_Q, H_KV, N, X)
        W = oracle.num_workgroups(B, H_Q, N, attn.BLOCK_M)
        assert got.shape == (W, 3)
        if W > 20000:  # spot-check the large tables
            idx = np.random.default_rng(W).integers(0, W, 4000)
        else:
            idx = np.arange(W)
        exp = np.array([oracle.wg_map(mode, int(w), B, H_Q, N, X, attn.BLOCK_M, H_Q // H_KV)
                        for w in idx],
                       dtype=np.int32).reshape(-1, 3)
        assert np.array_equal(got[idx], exp), (mode, B, H_Q, H_KV, N, X)


def test_host_wg_map_is_bijection_on_headline_shape():
    for mode in range(16):
        t = attn.attn_wg_map(mode, 1, 128, 128, 131072, 8).astype(np.int64)
        key = (t[:, 0] * 128 + t[:, 1]) * 1024 + t[:, 2]
        assert np.unique(key).size == t.shape[0] == 128 * (131072 // attn.BLOCK_M)


def test_num_xcd_env_override(monkeypatch):
    """ATTN_NUM_XCD is read on every call; without a GPU the call reports
    that no device is visible."""
    lib = attn.load_library()
    import torch
    if torch.cuda.is_available():
        pytest.skip("covered by the GPU placement test")
    assert lib.attn_num_xcd() == _declared_codes()["ATTN_E_NO_DEVICE"]


def test_split_chunk_rule(lib):
    """ceil(N_kv / S) rounded up to whole 32-key tiles; the splits cover the
    keys exactly once."""
    c = _declared_codes()
    for N_kv, S in [(1, 1), (31, 1), (32, 2), (100, 4), (40, 4), (131072, 64), (1000, 7)]:
        chunk = attn.attn_split_chunk(N_kv, S)
        assert chunk % 32 == 0 and chunk >= -(-N_kv // S)
        assert chunk < -(-N_kv // S) + 32
        covered = sum(max(0, min((s + 1) * chunk, N_kv) - s * chunk) for s in range(S))
        assert covered == N_kv
    assert lib.attn_split_chunk(0, 1) == c["ATTN_E_SHAPE"]
    assert lib.attn_split_chunk(10, 0) == c["ATTN_E_SHAPE"]


def _split(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, H_Q=8, H_KV=8, N_q=16,
           N_kv=1024, d=128, causal=0, S=4, o_ws=FAKE, lse_ws=FAKE, mapping=3):
    return lib.attn_fwd_split(q, k, v, o, lse, B, H_Q, H_KV, N_q, N_kv, d, causal, S,
                              o_ws, lse_ws, mapping, None)


def test_split_and_merge_argument_errors(lib):
    """Rejected before anything could launch on the fake pointers."""
    c = _declared_codes()
    assert _split(lib, q=None) == c["ATTN_E_NULL"]
    assert _split(lib, o_ws=None) == c["ATTN_E_NULL"]
    assert _split(lib, lse_ws=None) == c["ATTN_E_NULL"]
    for kw in ({"N_q": 0}, {"N_kv": 0}, {"S": 0}, {"H_Q": 6, "H_KV": 4},
               {"B": 1 << 12, "H_Q": 1 << 10, "N_q": 256, "S": 1 << 10}):
        assert _split(lib, **kw) == c["ATTN_E_SHAPE"], kw
    assert _split(lib, d=12) == c["ATTN_E_HEAD_DIM"]
    assert _split(lib, mapping=16) == c["ATTN_E_MAPPING"]
    assert _split(lib, o_ws=FAKE + 4) == c["ATTN_E_ALIGN"]
    m = lambda **kw: lib.attn_merge(kw.get("op", FAKE), kw.get("lp", FAKE), kw.get("S", 2),
                                    kw.get("B", 1), kw.get("H", 2), kw.get("N", 3),
                                    kw.get("d", 64), kw.get("o", FAKE), kw.get("lse", None), None)
    assert m(op=None) == c["ATTN_E_NULL"]
    assert m(o=None) == c["ATTN_E_NULL"]
    assert m(S=0) == c["ATTN_E_SHAPE"]
    assert m(N=0) == c["ATTN_E_SHAPE"]
    assert m(d=7) == c["ATTN_E_HEAD_DIM"]
    assert m(lp=FAKE + 8) == c["ATTN_E_ALIGN"]


def test_bwd_argument_errors(lib):
    """attn_bwd rejects bad arguments before anything could launch on the
    fake pointers (every case below fails a host check)."""
    c = _declared_codes()

    def b(**kw):
        ptrs = [kw.get(n, FAKE) for n in ("q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "ws")]
        return lib.attn_bwd(*ptrs, kw.get("B", 1), kw.get("H_Q", 4), kw.get("H_KV", 2),
                            kw.get("N", 300), kw.get("d", 128), kw.get("causal", 1),
                            kw.get("mapping", 16 if "mapping_ok" not in kw else 3), None)

    for n in ("q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "ws"):
        assert b(**{n: None}) == c["ATTN_E_NULL"], n
    for kw in ({"N": 0}, {"B": 0}, {"H_Q": 6, "H_KV": 4}, {"H_KV": 0},
               {"B": 1 << 12, "H_Q": 1 << 12, "H_KV": 1 << 12, "N": 1 << 14},
               {"N": (1 << 31) // 256 + 1}):
        assert b(**kw) == c["ATTN_E_SHAPE"], kw
    for d in (0, 12, 136):
        assert b(d=d) == c["ATTN_E_HEAD_DIM"], d
    assert b() == c["ATTN_E_MAPPING"]          # mapping 16
    assert b(mapping=-1) == c["ATTN_E_MAPPING"]
    for n in ("q", "dout", "lse", "dk", "ws"):
        assert b(mapping_ok=1, **{n: FAKE + 4}) == c["ATTN_E_ALIGN"], n


GEMM_HEADER = os.path.join(os.path.dirname(HEADER), "cac_gemm.h")


def test_gemm_header_symbols_exported(lib):
    text = re.sub(r"/\*.*?\*/", "", open(GEMM_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(cac_\w+)\s*\(", text)))
    assert set(names) == {"cac_gemm", "cac_gemm_tile", "cac_gemm_map"}
    for n in names:
        assert hasattr(lib, n), n
    assert lib.cac_gemm_tile() == 256


def test_gemm_host_map_equals_oracle():
    import oracle
    t = attn.cac_gemm_tile()
    for mode in range(4):
        for L, M, N, g1, g2, X in [(1, 3 * t, 5 * t, 2, 2, 8), (2, 7 * t - 5, 3 * t, 4, 3, 8),
                                   (1, 64 * t, 8 * t, 0, 0, 8), (3, 5 * t, 5 * t - 8, 2, 3, 3),
                                   (1, 100, 40, 0, 0, 8), (2, 9 * t, 11 * t, 0, 0, 5)]:
            Mt, Nt = -(-M // t), -(-N // t)
            gm_ = min(g1 or 4, Mt)
            gn_ = min(g2 or 8, Nt)
            want = oracle.cac_tile_table(mode, L, Mt, Nt, gm_, gn_, X)
            got = attn.cac_gemm_map(mode, L, M, N, g1, g2, X)
            assert np.array_equal(got, want), (mode, L, M, N, g1, g2, X)


def test_gemm_argument_errors(lib):
    """Rejected before anything could launch on the fake pointers."""
    c = _declared_codes()

    def g(**kw):
        return lib.cac_gemm(kw.get("a", FAKE), kw.get("b", FAKE), kw.get("c", FAKE),
                            kw.get("L", 1), kw.get("M", 300), kw.get("N", 136), kw.get("K", 72),
                            kw.get("mapping", 4 if "mapping_ok" not in kw else 3),
                            kw.get("gm", 0), kw.get("gn", 0), None)

    for n in ("a", "b", "c"):
        assert g(**{n: None}) == c["ATTN_E_NULL"], n
    for kw in ({"L": 0}, {"M": 0}, {"N": 0}, {"K": 0}, {"N": 100}, {"K": 12},
               {"K": (1 << 20) + 8}, {"M": 1 << 20, "K": 2048}, {"N": 1 << 20, "K": 2048},
               {"M": 1 << 17, "N": 1 << 14}, {"L": 1 << 24, "M": 1 << 12, "N": 1 << 12},
               {"gm": -1, "mapping_ok": 1}, {"gn": -2, "mapping_ok": 1}):
        assert g(**kw) == c["ATTN_E_SHAPE"], kw
    assert g() == c["ATTN_E_MAPPING"]          # mapping 4
    assert g(mapping=-1) == c["ATTN_E_MAPPING"]
    for n in ("a", "b", "c"):
        assert g(mapping_ok=1, **{n: FAKE + 8}) == c["ATTN_E_ALIGN"], n
    out = np.empty((4, 3), dtype=np.int32)
    assert lib.cac_gemm_map(3, 1, 256, 256, 0, 0, 0, out.ctypes.data) == c["ATTN_E_SHAPE"]
    assert lib.cac_gemm_map(4, 1, 256, 256, 0, 0, 8, out.ctypes.data) == c["ATTN_E_MAPPING"]
    assert lib.cac_gemm_map(3, 1, 256, 256, 0, 0, 8, None) == c["ATTN_E_NULL"]


# ---- caller-given outputs and workspaces are checked before any launch -----
def test_check_out_rejects_every_bad_buffer():
    import torch
    dev = torch.device("cuda", 0)          # constructing it needs no GPU
    ok_shape = (1, 2, 3, 8)
    bad = [
        ("host tensor", torch.empty(ok_shape, dtype=torch.bfloat16), "must be on"),
        ("wrong shape", torch.empty((1, 2, 3, 16), dtype=torch.bfloat16), "of shape"),
        ("wrong dtype", torch.empty(ok_shape, dtype=torch.float16), "of shape"),
        ("not a tensor", np.zeros(ok_shape), "torch.Tensor"),
    ]
    for what, t, msg in bad:
        with pytest.raises(ValueError, match=msg):
            attn._check_out("o", t, ok_shape, torch.bfloat16, dev)


def test_check_out_rejects_non_contiguous_and_another_device():
    import torch
    t = torch.empty((6, 4), dtype=torch.float32).t()
    with pytest.raises(ValueError, match="contiguous"):
        attn._check_out("ws", t, (4, 6), torch.float32, torch.device("cuda", 0))
    with pytest.raises(ValueError, match="must be on cuda:1"):
        attn._check_out("ws", t.contiguous(), (4, 6), torch.float32, torch.device("cuda", 1))


def test_probe_placement_rejects_a_host_buffer(lib):
    import torch
    W = attn.num_workgroups(1, 8, 1024)
    with pytest.raises(ValueError, match="GPU tensor"):
        attn.attn_probe_placement(3, 1, 8, 8, 1024, out=torch.empty((W, 4), dtype=torch.int32))


def test_default_mapping_depends_on_the_mask():
    assert attn._mapping_id(None, causal=False) == attn.DEFAULT_MAPPING == 3
    assert attn._mapping_id(None, causal=True) == attn.DEFAULT_CAUSAL_MAPPING == 3 | 4 | 8
    assert attn._mapping_id("swizzled_head_first", causal=True) == 3
    assert attn._mapping_id(5, causal=True) == 5


def test_noalloc_rejects_oversize_before_touching_a_device(lib):
    """attn_fwd_split_noalloc checks the scratch size first: a call whose
    split partials exceed ATTN_SCRATCH_BYTES returns ATTN_E_SCRATCH with no
    device query (there is no GPU here), and bad shapes are still reported."""
    c = _declared_codes()
    text = open(HEADER).read()
    limit = int(re.search(r"#define ATTN_SCRATCH_BYTES \((\d+) \* 1024 \* 1024\)", text).group(1)) << 20
    assert limit == attn.SCRATCH_BYTES

    def n(B=4, H_Q=32, H_KV=8, N_q=64, N_kv=4096, d=128, S=64):
        return lib.attn_fwd_split_noalloc(FAKE, FAKE, FAKE, FAKE, None, B, H_Q, H_KV, N_q,
                                          N_kv, d, 1, S, 3, None)
    assert 64 * 4 * 32 * 64 * 129 * 4 > limit
    assert n() == c["ATTN_E_SCRATCH"]
    assert n(B=0) == c["ATTN_E_SHAPE"]
    assert n(d=12) == c["ATTN_E_HEAD_DIM"]
    # fits: validation passes the size check and stops at the missing GPU
    assert n(S=8, N_q=1) == c["ATTN_E_NO_DEVICE"]


def test_missing_library_raises_instead_of_falling_back(monkeypatch, tmp_path):
    """Without the built library every entry point fails loudly: there is no
    CPU path to fall back to."""
    monkeypatch.setattr(attn, "LIB_PATH", str(tmp_path / "libattn_numa.so"))
    monkeypatch.setattr(attn, "_lib", None)
    with pytest.raises(RuntimeError, match="is not built"):
        attn.load_library()
    # A host tensor is refused as well (no CPU path computes attention).
    import torch
    q = torch.zeros((1, 1, 4, 64), dtype=torch.bfloat16)
    with pytest.raises((RuntimeError, ValueError)):
        attn.attn_fwd(q, q, q)
