"""Python binding of libattn_numa (NUMA-aware attention for MI355X).

Argument marshalling only: every step of the attention forward and backward
passes runs in
the library's HIP kernels.  torch provides device memory and streams.  The
entry points have the names of the C ABI in include/attn_numa.h:

* ``attn_fwd(q, k, v, causal=False, mapping=None, o=None, lse=None)``
* ``attn_fwd_split(q, k, v, causal=False, num_splits=1, mapping=None, ...)``
* ``attn_fwd_split_noalloc(q, k, v, o, lse=None, causal=False, num_splits=1, ...)``
* ``attn_split_chunk(N_kv, num_splits)``
* ``attn_merge(o_parts, lse_parts, o=None, lse=None)``
* ``attn_bwd(q, k, v, o, dout, lse, causal=False, mapping=None, ...)``
* ``cac_gemm(a, b, mapping=3, group_m=0, group_n=0, c=None)`` (include/cac_gemm.h)
* ``cac_gemm_map(mapping, L, M, N, group_m, group_n, num_xcd)``
* ``cac_gemm_tile()``
* ``attn_wg_map(mapping, B, H_Q, H_KV, N, num_xcd)``
* ``attn_num_xcd()``
* ``attn_block_m()``
* ``attn_probe_placement(mapping, B, H_Q, H_KV, N, out=None)``
* ``attn_strerror(code)``

``mapping=None`` is swizzled head-first (3), and under a causal mask
3 | LONGEST_FIRST | BALANCED_SPLIT (15).  Caller-given outputs and
workspaces are checked (device, shape, dtype, contiguity) before any launch.

The library must be built (``python -m chiplet_numa_aware_amd.build``);
there is no fallback: a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch  # first, so the library binds to the HIP runtime torch loaded

__all__ = [
    "AttnError", "attn_fwd", "attn_fwd_split", "attn_fwd_split_noalloc", "SCRATCH_BYTES",
    "attn_split_chunk", "attn_merge", "attn_bwd",
    "cac_gemm", "cac_gemm_map", "cac_gemm_tile", "CAC_MAPPINGS",
    "attn_wg_map", "attn_num_xcd", "attn_block_m",
    "attn_probe_placement", "attn_strerror", "library_path", "load_library",
    "MAPPINGS", "row_blocks", "num_workgroups", "BLOCK_M",
    "LONGEST_FIRST", "BALANCED_SPLIT", "DEFAULT_MAPPING", "DEFAULT_CAUSAL_MAPPING",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "libattn_numa.so")

# Mapping modes (ATTN_MAP_* in include/attn_numa.h).
MAPPINGS = {
    "naive_block_first": 0,
    "naive_head_first": 1,
    "swizzled_block_first": 2,
    "swizzled_head_first": 3,
}

# Added to a mode (ATTN_MAP_LONGEST_FIRST, ATTN_MAP_BALANCED_SPLIT).
LONGEST_FIRST = 4
BALANCED_SPLIT = 8
# Default mappings: swizzled head-first, and under a causal mask also longest
# first and balanced splits.
DEFAULT_MAPPING = 3
DEFAULT_CAUSAL_MAPPING = 3 | LONGEST_FIRST | BALANCED_SPLIT

# Tile map modes of cac_gemm (CAC_MAP_* in include/cac_gemm.h).
CAC_MAPPINGS = {
    "naive_row_major": 0,
    "naive_cluster": 1,
    "swizzled_row_major": 2,
    "swizzled_cluster": 3,
}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {attn_strerror(code)} (code {code})")


def library_path() -> str:
    return LIB_PATH


def load_library():
    """Loads libattn_numa.so and declares its C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m chiplet_numa_aware_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp] + [i32] * 7 + [vp]
    lib.attn_fwd.restype = i32
    lib.attn_fwd_split.argtypes = [vp, vp, vp, vp, vp] + [i32] * 8 + [vp, vp, i32, vp]
    lib.attn_fwd_split.restype = i32
    lib.attn_fwd_split_noalloc.argtypes = [vp, vp, vp, vp, vp] + [i32] * 9 + [vp]
    lib.attn_fwd_split_noalloc.restype = i32
    lib.attn_split_chunk.argtypes = [i32, i32]
    lib.attn_split_chunk.restype = i32
    lib.attn_merge.argtypes = [vp, vp] + [i32] * 5 + [vp, vp, vp]
    lib.attn_merge.restype = i32
    lib.attn_bwd.argtypes = [vp] * 10 + [i32] * 7 + [vp]
    lib.attn_bwd.restype = i32
    lib.cac_gemm.argtypes = [vp, vp, vp] + [i32] * 7 + [vp]
    lib.cac_gemm.restype = i32
    lib.cac_gemm_tile.argtypes = []
    lib.cac_gemm_tile.restype = i32
    lib.cac_gemm_map.argtypes = [i32] * 7 + [vp]
    lib.cac_gemm_map.restype = i32
    lib.attn_wg_map.argtypes = [i32] * 6 + [vp]
    lib.attn_wg_map.restype = i32
    lib.attn_num_xcd.argtypes = []
    lib.attn_num_xcd.restype = i32
    lib.attn_block_m.argtypes = []
    lib.attn_block_m.restype = i32
    lib.attn_probe_placement.argtypes = [i32] * 5 + [vp, vp]
    lib.attn_probe_placement.restype = i32
    lib.attn_strerror.argtypes = [i32]
    lib.attn_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def attn_strerror(code: int) -> str:
    return load_library().attn_strerror(int(code)).decode()


def _check(code: int, where: str):
    if code != 0:
        raise AttnError(code, where)


def attn_block_m() -> int:
    """Query rows per workgroup (the row-block height)."""
    return int(load_library().attn_block_m())


def __getattr__(name):
    # BLOCK_M is the library's row-block height, read when first asked for.
    if name == "BLOCK_M":
        return attn_block_m()
    raise AttributeError(name)


def row_blocks(N: int) -> int:
    return -(-N // attn_block_m())


def num_workgroups(B: int, H_Q: int, N: int) -> int:
    return B * H_Q * row_blocks(N)


def _mapping_id(mapping, causal: bool = False) -> int:
    """Mode id of ``mapping`` (a name or an int).  None picks the default:
    swizzled head-first, plus longest first and balanced splits under a
    causal mask (the order that keeps each ACC's concurrent workgroups
    together in the K/V stream and balances the causal work of ACCs split
    between two XCDs; for a non-causal call both bits change nothing but the
    order of equal-length row blocks)."""
    if mapping is None:
        return DEFAULT_CAUSAL_MAPPING if causal else DEFAULT_MAPPING
    if isinstance(mapping, str):
        return MAPPINGS[mapping]
    return int(mapping)


def _check_out(name: str, t, shape, dtype, device: torch.device):
    """A caller-given output or workspace: a contiguous tensor of exactly
    ``shape`` and ``dtype`` on the inputs' GPU.  Raised before any launch,
    so that a wrong buffer is a ValueError and not a GPU memory fault."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device} (the inputs' device), not {t.device}")


def _stream_handle(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
             causal: bool = False, mapping=None, o: torch.Tensor | None = None,
             lse: torch.Tensor | None = None, need_lse: bool = True,
             stream: torch.cuda.Stream | None = None):
    """Attention forward on the GPU: returns (o, lse).

    q [B,H_Q,N,d], k and v [B,H_KV,N,d]: contiguous bf16 on one GPU.  o and
    lse are allocated when not given (lse is None when need_lse is False and
    no lse is given).  Enqueued on ``stream`` (default: torch's current
    stream); returns without synchronising.
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise ValueError(f"{name} must be a 4-D tensor")
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 GPU tensor")
    B, H_Q, N, d = q.shape
    H_KV = k.shape[1]
    if k.shape != (B, H_KV, N, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, H_KV, N, d] with q's B, N, d")
    _same_device(q, k, v)
    if o is None:
        o = torch.empty_like(q)
    _check_out("o", o, q.shape, torch.bfloat16, q.device)
    if lse is None and need_lse:
        lse = torch.empty((B, H_Q, N), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_out("lse", lse, (B, H_Q, N), torch.float32, q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        rc = lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                          lse.data_ptr() if lse is not None else None,
                          B, H_Q, H_KV, N, d, int(bool(causal)),
                          _mapping_id(mapping, causal), _stream_handle(stream, q.device))
    _check(rc, "attn_fwd")
    return o, lse


def _same_device(*ts):
    dev = ts[0].device
    for t in ts[1:]:
        if t.device != dev:
            raise ValueError(f"every input must be on {dev}; found one on {t.device}")


def _check_bf16(name, t):
    if not isinstance(t, torch.Tensor) or t.dim() != 4:
        raise ValueError(f"{name} must be a 4-D tensor")
    if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bf16 GPU tensor")


def _check_f32(name, t, shape):
    if (not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(shape)
            or t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda):
        raise ValueError(f"{name} must be a contiguous fp32 GPU tensor of shape {tuple(shape)}")


def attn_split_chunk(N_kv: int, num_splits: int) -> int:
    """Keys per split of attn_fwd_split (host, no GPU)."""
    rc = load_library().attn_split_chunk(int(N_kv), int(num_splits))
    if rc < 0:
        raise AttnError(rc, "attn_split_chunk")
    return rc


def attn_fwd_split(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                   causal: bool = False, num_splits: int = 1, mapping=None,
                   o: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                   o_ws: torch.Tensor | None = None, lse_ws: torch.Tensor | None = None,
                   need_lse: bool = True, stream: torch.cuda.Stream | None = None):
    """Attention of q [B,H_Q,N_q,d] over k, v [B,H_KV,N_kv,d], keys split in
    ``num_splits`` ranges and merged: returns (o, lse).  Causal is
    bottom-right aligned.  For num_splits > 1 the fp32 workspaces o_ws
    [S,B,H_Q,N_q,d] and lse_ws [S,B,H_Q,N_q] are allocated when not given;
    after the call they hold each split's partial result."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_bf16(name, t)
    B, H_Q, N_q, d = q.shape
    H_KV, N_kv = k.shape[1], k.shape[2]
    if k.shape != (B, H_KV, N_kv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, H_KV, N_kv, d] with q's B and d")
    _same_device(q, k, v)
    S = int(num_splits)
    if o is None:
        o = torch.empty_like(q)
    _check_out("o", o, q.shape, torch.bfloat16, q.device)
    if lse is None and need_lse:
        lse = torch.empty((B, H_Q, N_q), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_out("lse", lse, (B, H_Q, N_q), torch.float32, q.device)
    if S > 1:
        if o_ws is None:
            o_ws = torch.empty((S, B, H_Q, N_q, d), dtype=torch.float32, device=q.device)
        if lse_ws is None:
            lse_ws = torch.empty((S, B, H_Q, N_q), dtype=torch.float32, device=q.device)
        _check_out("o_ws", o_ws, (S, B, H_Q, N_q, d), torch.float32, q.device)
        _check_out("lse_ws", lse_ws, (S, B, H_Q, N_q), torch.float32, q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        rc = lib.attn_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr() if lse is not None else None,
                                B, H_Q, H_KV, N_q, N_kv, d, int(bool(causal)), S,
                                o_ws.data_ptr() if S > 1 else None,
                                lse_ws.data_ptr() if S > 1 else None,
                                _mapping_id(mapping, causal), _stream_handle(stream, q.device))
    _check(rc, "attn_fwd_split")
    return o, lse


# ATTN_SCRATCH_BYTES of include/attn_numa.h: the fixed device scratch of
# attn_fwd_split_noalloc.
SCRATCH_BYTES = 32 * 1024 * 1024


def attn_fwd_split_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                           o: torch.Tensor, lse: torch.Tensor | None = None,
                           causal: bool = False, num_splits: int = 1, mapping=None,
                           stream: torch.cuda.Stream | None = None):
    """attn_fwd_split with its split partials in the library's fixed device
    scratch (ATTN_SCRATCH_BYTES per GPU) instead of a workspace: for callers
    that cannot allocate.  The caller passes the outputs o (bf16, shaped
    like q) and optionally lse (fp32 [B, H_Q, N_q]); nothing is allocated.
    Calls that overlap on one GPU share the scratch and race."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_bf16(name, t)
    B, H_Q, N_q, d = q.shape
    H_KV, N_kv = k.shape[1], k.shape[2]
    if k.shape != (B, H_KV, N_kv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, H_KV, N_kv, d] with q's B and d")
    _same_device(q, k, v)
    _check_out("o", o, q.shape, torch.bfloat16, q.device)
    if lse is not None:
        _check_out("lse", lse, (B, H_Q, N_q), torch.float32, q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        rc = lib.attn_fwd_split_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                        lse.data_ptr() if lse is not None else None,
                                        B, H_Q, H_KV, N_q, N_kv, d, int(bool(causal)),
                                        int(num_splits), _mapping_id(mapping, causal),
                                        _stream_handle(stream, q.device))
    _check(rc, "attn_fwd_split_noalloc")
    return o, lse


def attn_merge(o_parts: torch.Tensor, lse_parts: torch.Tensor,
               o: torch.Tensor | None = None, lse: torch.Tensor | None = None,
               need_lse: bool = True, stream: torch.cuda.Stream | None = None):
    """Merge partial results o_parts fp32 [S,B,H_Q,N_q,d], lse_parts fp32
    [S,B,H_Q,N_q] into (o bf16 [B,H_Q,N_q,d], lse fp32 [B,H_Q,N_q])."""
    if o_parts.dim() != 5:
        raise ValueError("o_parts must be [S, B, H_Q, N_q, d]")
    S, B, H_Q, N_q, d = o_parts.shape
    _check_f32("o_parts", o_parts, (S, B, H_Q, N_q, d))
    _check_f32("lse_parts", lse_parts, (S, B, H_Q, N_q))
    _same_device(o_parts, lse_parts)
    if o is None:
        o = torch.empty((B, H_Q, N_q, d), dtype=torch.bfloat16, device=o_parts.device)
    _check_out("o", o, (B, H_Q, N_q, d), torch.bfloat16, o_parts.device)
    if lse is None and need_lse:
        lse = torch.empty((B, H_Q, N_q), dtype=torch.float32, device=o_parts.device)
    if lse is not None:
        _check_out("lse", lse, (B, H_Q, N_q), torch.float32, o_parts.device)
    lib = load_library()
    with torch.cuda.device(o_parts.device):
        rc = lib.attn_merge(o_parts.data_ptr(), lse_parts.data_ptr(), S, B, H_Q, N_q, d,
                            o.data_ptr(), lse.data_ptr() if lse is not None else None,
                            _stream_handle(stream, o_parts.device))
    _check(rc, "attn_merge")
    return o, lse


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
             dout: torch.Tensor, lse: torch.Tensor, causal: bool = False, mapping=None,
             dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
             dv: torch.Tensor | None = None, ws: torch.Tensor | None = None,
             stream: torch.cuda.Stream | None = None):
    """Gradients (dq, dk, dv) of sum(dout * o) for o, lse = attn_fwd(q, k, v,
    causal).  q, o, dout [B,H_Q,N,d] and k, v [B,H_KV,N,d] contiguous bf16;
    lse fp32 [B,H_Q,N].  Outputs and the fp32 workspace ws [B,H_Q,2,N] are
    allocated when not given.  Enqueued on ``stream``; returns without
    synchronising."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_bf16(name, t)
    B, H_Q, N, d = q.shape
    H_KV = k.shape[1]
    if k.shape != (B, H_KV, N, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, H_KV, N, d] with q's B, N, d")
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must be shaped like q")
    _check_f32("lse", lse, (B, H_Q, N))
    _same_device(q, k, v, o, dout, lse)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_out(name, t, ref.shape, torch.bfloat16, q.device)
    if ws is None:
        ws = torch.empty((B, H_Q, 2, N), dtype=torch.float32, device=q.device)
    _check_out("ws", ws, (B, H_Q, 2, N), torch.float32, q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        rc = lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                          dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                          dv.data_ptr(), ws.data_ptr(), B, H_Q, H_KV, N, d,
                          int(bool(causal)), _mapping_id(mapping, causal),
                          _stream_handle(stream, q.device))
    _check(rc, "attn_bwd")
    return dq, dk, dv


def cac_gemm_tile() -> int:
    """Rows and columns of one C tile of cac_gemm (host, no GPU)."""
    return int(load_library().cac_gemm_tile())


def _cac_mapping_id(mapping) -> int:
    if isinstance(mapping, str):
        return CAC_MAPPINGS[mapping]
    return int(mapping)


def cac_gemm(a: torch.Tensor, b: torch.Tensor, mapping=3, group_m: int = 0,
             group_n: int = 0, c: torch.Tensor | None = None,
             stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """C = A B^T (per batch) on the GPU.  a [L,M,K] or [M,K], b [L,N,K] or
    [N,K], contiguous bf16; returns c [L,M,N] (or [M,N]) bf16, allocated when
    not given.  ``mapping`` is the Compute Affinity Cluster tile map
    (CAC_MAPPINGS), group_m x group_n the cluster in 256 x 256 tiles (0: the
    library default).  Enqueued on ``stream``; returns without synchronising."""
    squeeze = a.dim() == 2
    a3 = a.unsqueeze(0) if squeeze else a
    b3 = b.unsqueeze(0) if b.dim() == 2 else b
    for name, t in (("a", a3), ("b", b3)):
        if t.dim() != 3 or t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 GPU tensor [L, rows, K]")
    L, M, K = a3.shape
    if b3.shape[0] != L or b3.shape[2] != K:
        raise ValueError("b must be [L, N, K] with a's L and K")
    _same_device(a3, b3)
    N = b3.shape[1]
    shape = (M, N) if squeeze else (L, M, N)
    if c is None:
        c = torch.empty(shape, dtype=torch.bfloat16, device=a.device)
    _check_out("c", c, shape, torch.bfloat16, a.device)
    lib = load_library()
    with torch.cuda.device(a.device):
        rc = lib.cac_gemm(a3.data_ptr(), b3.data_ptr(), c.data_ptr(), L, M, N, K,
                          _cac_mapping_id(mapping), int(group_m), int(group_n),
                          _stream_handle(stream, a.device))
    _check(rc, "cac_gemm")
    return c


def cac_gemm_map(mapping, L: int, M: int, N: int, group_m: int = 0, group_n: int = 0,
                 num_xcd: int = 8) -> np.ndarray:
    """(l, tile row, tile column) of every workgroup id of cac_gemm, int32
    [W, 3] (host, no GPU)."""
    t = cac_gemm_tile()
    W = L * (-(-M // t)) * (-(-N // t))
    out = np.empty((max(W, 1), 3), dtype=np.int32)
    rc = load_library().cac_gemm_map(_cac_mapping_id(mapping), L, M, N, int(group_m),
                                     int(group_n), num_xcd, out.ctypes.data)
    _check(rc, "cac_gemm_map")
    return out[:W]


def attn_wg_map(mapping, B: int, H_Q: int, H_KV: int, N: int,
                num_xcd: int) -> np.ndarray:
    """The (b, h, m) of every workgroup id, int32 [W, 3] (host, no GPU)."""
    W = num_workgroups(B, H_Q, N)
    out = np.empty((max(W, 1), 3), dtype=np.int32)
    rc = load_library().attn_wg_map(_mapping_id(mapping), B, H_Q, H_KV, N,
                                    num_xcd, out.ctypes.data)
    _check(rc, "attn_wg_map")
    return out[:W]


def attn_num_xcd() -> int:
    rc = load_library().attn_num_xcd()
    if rc < 0:
        raise AttnError(rc, "attn_num_xcd")
    return rc


def attn_probe_placement(mapping, B: int, H_Q: int, H_KV: int, N: int,
                         out: torch.Tensor | None = None, device="cuda",
                         stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """int32 [W, 4] on the GPU: (xcc_id, b, h, m) per workgroup id."""
    W = num_workgroups(B, H_Q, N)
    if out is None:
        out = torch.empty((W, 4), dtype=torch.int32, device=device)
    if not isinstance(out, torch.Tensor) or not out.is_cuda:
        raise ValueError("out must be a GPU tensor")
    _check_out("out", out, (W, 4), torch.int32, out.device)
    lib = load_library()
    with torch.cuda.device(out.device):
        rc = lib.attn_probe_placement(_mapping_id(mapping if mapping is not None else 3),
                                      B, H_Q, H_KV, N,
                                      out.data_ptr(),
                                      _stream_handle(stream, out.device))
    _check(rc, "attn_probe_placement")
    return out
