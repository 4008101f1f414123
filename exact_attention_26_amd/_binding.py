"""ctypes binding over libfa.so (declared in include/fa.h).

Argument marshalling only: torch tensors give device pointers and the current
HIP stream; every computation happens in the library's kernels.  If the
library has not been built the calls raise ``FaError`` -- there is no other
implementation behind these names.
"""
from __future__ import annotations

import ctypes
import math
import os

FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED, FA_ERR_HIP, FA_ERR_TOO_LARGE = 0, 1, 2, 3, 4
FA_NOALLOC_SCRATCH_BYTES = 32 << 20     # scratch fa_paged_decode_noalloc holds per GPU
FA_BF16, FA_F32 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class FaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_status_name(status)}")


def library_path() -> str:
    return os.environ.get("FA_LIBRARY", os.path.join(_HERE, "libfa.so"))


def load_library():
    """Load libfa.so once and declare the C signatures.  Raises if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise FaError(-1, f"libfa.so not built (expected at {path}); run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    c = ctypes
    lib.fa_fwd.restype = c.c_int
    lib.fa_fwd.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
                           c.c_int, c.c_int, c.c_int, c.c_int, c.c_int, c.c_float,
                           c.c_int, c.c_void_p]
    lib.fa_bwd_workspace_size.restype = c.c_size_t
    lib.fa_bwd_workspace_size.argtypes = [c.c_int] * 4
    lib.fa_bwd.restype = c.c_int
    lib.fa_bwd.argtypes = [c.c_void_p] * 9 + [c.c_int, c.c_int, c.c_int, c.c_int, c.c_int,
                                              c.c_float, c.c_int, c.c_void_p, c.c_size_t,
                                              c.c_void_p]
    lib.fa_paged_decode_workspace_size.restype = c.c_size_t
    lib.fa_paged_decode_workspace_size.argtypes = [c.c_int] * 5
    lib.fa_paged_decode.restype = c.c_int
    lib.fa_paged_decode.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p,
                                    c.c_void_p, c.c_void_p,
                                    c.c_int, c.c_int, c.c_int, c.c_int, c.c_int, c.c_int64,
                                    c.c_float, c.c_int, c.c_void_p, c.c_size_t, c.c_void_p]
    lib.fa_paged_decode_noalloc.restype = c.c_int
    lib.fa_paged_decode_noalloc.argtypes = [c.c_void_p] * 7 + [c.c_int] * 5 + [c.c_int64,
                                                                c.c_float, c.c_int, c.c_void_p]
    lib.fa_paged_prefill.restype = c.c_int
    lib.fa_paged_prefill.argtypes = [c.c_void_p] * 8 + [c.c_int, c.c_int, c.c_int, c.c_int, c.c_int,
                                                        c.c_int64, c.c_int, c.c_int, c.c_int,
                                                        c.c_float, c.c_int, c.c_void_p]
    lib.fa_tree_decode.restype = c.c_int
    lib.fa_tree_decode.argtypes = [c.c_void_p] * 9 + [c.c_int, c.c_int, c.c_int, c.c_int, c.c_int,
                                                      c.c_int64, c.c_int, c.c_int, c.c_float,
                                                      c.c_int, c.c_void_p]
    lib.fa_rope.restype = c.c_int
    lib.fa_rope.argtypes = [c.c_void_p] * 4 + [c.c_int] * 5 + [c.c_void_p]
    lib.fa_fwd_rope_workspace_size.restype = c.c_size_t
    lib.fa_fwd_rope_workspace_size.argtypes = [c.c_int] * 4
    lib.fa_fwd_rope.restype = c.c_int
    lib.fa_fwd_rope.argtypes = [c.c_void_p] * 7 + [c.c_int] * 5 + [c.c_float, c.c_int,
                                                                   c.c_void_p, c.c_size_t,
                                                                   c.c_void_p]
    lib.fa_status_string.restype = c.c_char_p
    lib.fa_status_string.argtypes = [c.c_int]
    lib.fa_last_hip_error.restype = c.c_int
    lib.fa_last_hip_error.argtypes = []
    _LIB = lib
    return lib


def _status_name(status: int) -> str:
    if status < 0:
        return "library not loaded"
    try:
        return load_library().fa_status_string(status).decode()
    except FaError:
        return f"status {status}"


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def fa_last_hip_error() -> int:
    return int(load_library().fa_last_hip_error())


def fa_bwd_workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(load_library().fa_bwd_workspace_size(B, H, N, d))


def fa_paged_decode_workspace_size(num_seqs: int, H: int, d: int, page_size: int,
                                   max_blocks_per_seq: int) -> int:
    return int(load_library().fa_paged_decode_workspace_size(num_seqs, H, d, page_size,
                                                             max_blocks_per_seq))


# --------------------------------------------------------------------------
# tensor-level calls (same names as the C entry points)
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    return 99  # the library answers FA_ERR_UNSUPPORTED


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_cache_dtypes(q, k_cache, v_cache):
    """The library is told q's dtype only: the caches must share it (checked
    before anything else, so a mismatch never reaches the kernels)."""
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError(f"k_cache and v_cache must have q's dtype ({q.dtype}); got "
                         f"{k_cache.dtype} and {v_cache.dtype}")


def _check_dense(name, t, device):
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def fa_fwd(q, k, v, o, lse, causal: bool, scale: float) -> None:
    """Call ``fa_fwd`` on ``[B][H][N][d]`` tensors; ``lse`` may be None."""
    if q.dim() != 4:
        raise ValueError("q must be [B][H][N][d]")
    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_dense(name, t, dev)
        if tuple(t.shape) != (B, H, N, d) or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q's shape and dtype")
    if lse is not None:
        _check_dense("lse", lse, dev)
        if tuple(lse.shape) != (B, H, N) or lse.dtype != _torch().float32:
            raise ValueError("lse must be float32 [B][H][N]")
    st = load_library().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                               B, H, N, d, int(bool(causal)), float(scale),
                               _dtype_code(q), _stream(dev))
    if st != FA_OK:
        raise FaError(st, "fa_fwd")


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, causal: bool, scale: float, workspace) -> None:
    """Call ``fa_bwd`` on ``[B][H][N][d]`` tensors; ``lse`` float32 [B][H][N];
    ``workspace`` a uint8 device tensor of at least ``fa_bwd_workspace_size`` bytes."""
    if q.dim() != 4:
        raise ValueError("q must be [B][H][N][d]")
    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq),
                    ("dk", dk), ("dv", dv)):
        _check_dense(name, t, dev)
        if tuple(t.shape) != (B, H, N, d) or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q's shape and dtype")
    _check_dense("lse", lse, dev)
    if tuple(lse.shape) != (B, H, N) or lse.dtype != _torch().float32:
        raise ValueError("lse must be float32 [B][H][N]")
    _check_dense("workspace", workspace, dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = load_library().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                               _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, int(bool(causal)),
                               float(scale), _dtype_code(q), _ptr(workspace), ws_bytes,
                               _stream(dev))
    if st != FA_OK:
        raise FaError(st, "fa_bwd")


def fa_paged_decode(q, k_cache, v_cache, block_table, seq_lens, o, lse, scale: float,
                    workspace) -> None:
    """Call ``fa_paged_decode``.  ``q``/``o``: [S][H][d]; caches
    [num_blocks][H][page_size][d]; ``block_table`` int32 [S][max_blocks];
    ``seq_lens`` int32 [S]; ``lse`` float32 [S][H] or None; ``workspace`` a
    uint8 device tensor of at least ``fa_paged_decode_workspace_size`` bytes."""
    torch = _torch()
    _check_cache_dtypes(q, k_cache, v_cache)
    S, H, d = q.shape
    nb, Hk, P, dk = k_cache.shape
    dev = q.device
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_table", block_table), ("seq_lens", seq_lens), ("o", o),
                    ("workspace", workspace)):
        _check_dense(name, t, dev)
    if (Hk, dk) != (H, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache/v_cache must be [num_blocks][H][page_size][d]")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != S or tuple(seq_lens.shape) != (S,):
        raise ValueError("block_table must be [S][max_blocks], seq_lens [S]")
    if tuple(o.shape) != (S, H, d) or o.dtype != q.dtype:
        raise ValueError("o must match q")
    if lse is not None:
        _check_dense("lse", lse, dev)
        if tuple(lse.shape) != (S, H) or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [S][H]")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = load_library().fa_paged_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
        _ptr(o), _ptr(lse), S, H, d, P, block_table.shape[1], nb, float(scale),
        _dtype_code(q), _ptr(workspace), ws_bytes, _stream(dev))
    if st != FA_OK:
        raise FaError(st, "fa_paged_decode")


def fa_paged_decode_noalloc(q, k_cache, v_cache, block_table, seq_lens, o, lse,
                            scale: float) -> None:
    """Call ``fa_paged_decode_noalloc``: ``fa_paged_decode`` without a
    workspace (the library's per-GPU scratch array holds the partials; calls
    that overlap on one GPU race).  Allocates nothing."""
    torch = _torch()
    _check_cache_dtypes(q, k_cache, v_cache)
    S, H, d = q.shape
    nb, Hk, P, dk = k_cache.shape
    dev = q.device
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_table", block_table), ("seq_lens", seq_lens), ("o", o)):
        _check_dense(name, t, dev)
    if (Hk, dk) != (H, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache/v_cache must be [num_blocks][H][page_size][d]")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != S or tuple(seq_lens.shape) != (S,):
        raise ValueError("block_table must be [S][max_blocks], seq_lens [S]")
    if tuple(o.shape) != (S, H, d) or o.dtype != q.dtype:
        raise ValueError("o must match q")
    if lse is not None:
        _check_dense("lse", lse, dev)
        if tuple(lse.shape) != (S, H) or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [S][H]")
    st = load_library().fa_paged_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
        _ptr(o), _ptr(lse), S, H, d, P, block_table.shape[1], nb, float(scale),
        _dtype_code(q), _stream(dev))
    if st != FA_OK:
        raise FaError(st, "fa_paged_decode_noalloc")


def fa_paged_prefill(q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q, o, lse,
                     max_q_len: int, causal: bool, scale: float) -> None:
    """Call ``fa_paged_prefill``.  ``q``/``o``: [total_q][H][d]; caches
    [num_blocks][H][page_size][d]; ``block_table`` int32 [S][max_blocks];
    ``seq_lens`` int32 [S]; ``cu_seqlens_q`` int32 [S+1]; ``lse`` float32
    [total_q][H] or None."""
    torch = _torch()
    _check_cache_dtypes(q, k_cache, v_cache)
    total_q, H, d = q.shape
    nb, Hk, P, dk = k_cache.shape
    dev = q.device
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_table", block_table), ("seq_lens", seq_lens),
                    ("cu_seqlens_q", cu_seqlens_q), ("o", o)):
        _check_dense(name, t, dev)
    if (Hk, dk) != (H, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache/v_cache must be [num_blocks][H][page_size][d]")
    S = block_table.shape[0]
    if any(t.dtype != torch.int32 for t in (block_table, seq_lens, cu_seqlens_q)):
        raise ValueError("block_table, seq_lens and cu_seqlens_q must be int32")
    if block_table.dim() != 2 or tuple(seq_lens.shape) != (S,) \
            or tuple(cu_seqlens_q.shape) != (S + 1,):
        raise ValueError("block_table must be [S][max_blocks], seq_lens [S], cu_seqlens_q [S+1]")
    if tuple(o.shape) != (total_q, H, d) or o.dtype != q.dtype:
        raise ValueError("o must match q")
    if lse is not None:
        _check_dense("lse", lse, dev)
        if tuple(lse.shape) != (total_q, H) or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [total_q][H]")
    st = load_library().fa_paged_prefill(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
        _ptr(cu_seqlens_q), _ptr(o), _ptr(lse), S, H, d, P, block_table.shape[1], nb, total_q,
        int(max_q_len), int(bool(causal)), float(scale), _dtype_code(q), _stream(dev))
    if st != FA_OK:
        raise FaError(st, "fa_paged_prefill")


def fa_tree_decode(q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q, tree_parents, o,
                   lse, max_q_len: int, scale: float) -> None:
    """Call ``fa_tree_decode``: as ``fa_paged_prefill`` plus ``tree_parents``
    (int32 [total_q], each node's parent among its sequence's nodes or -1)."""
    torch = _torch()
    _check_cache_dtypes(q, k_cache, v_cache)
    _check_dense("tree_parents", tree_parents, q.device)
    if tree_parents.dtype != torch.int32 or tuple(tree_parents.shape) != (q.shape[0],):
        raise ValueError("tree_parents must be int32 [total_q]")
    total_q, H, d = q.shape
    nb, Hk, P, dk = k_cache.shape
    dev = q.device
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_table", block_table), ("seq_lens", seq_lens),
                    ("cu_seqlens_q", cu_seqlens_q), ("o", o)):
        _check_dense(name, t, dev)
    if (Hk, dk) != (H, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache/v_cache must be [num_blocks][H][page_size][d]")
    S = block_table.shape[0]
    if any(t.dtype != torch.int32 for t in (block_table, seq_lens, cu_seqlens_q)):
        raise ValueError("block_table, seq_lens and cu_seqlens_q must be int32")
    if block_table.dim() != 2 or tuple(seq_lens.shape) != (S,) \
            or tuple(cu_seqlens_q.shape) != (S + 1,):
        raise ValueError("block_table must be [S][max_blocks], seq_lens [S], cu_seqlens_q [S+1]")
    if tuple(o.shape) != (total_q, H, d) or o.dtype != q.dtype:
        raise ValueError("o must match q")
    if lse is not None:
        _check_dense("lse", lse, dev)
        if tuple(lse.shape) != (total_q, H) or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [total_q][H]")
    st = load_library().fa_tree_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
        _ptr(cu_seqlens_q), _ptr(tree_parents), _ptr(o), _ptr(lse), S, H, d, P,
        block_table.shape[1], nb, total_q, int(max_q_len), float(scale), _dtype_code(q),
        _stream(dev))
    if st != FA_OK:
        raise FaError(st, "fa_tree_decode")


def _check_tables(rope_cos, rope_sin, N, d, device):
    torch = _torch()
    for name, t in (("rope_cos", rope_cos), ("rope_sin", rope_sin)):
        _check_dense(name, t, device)
        if t.dtype != torch.float32 or t.dim() != 2 or t.shape[0] < N or t.shape[1] != d // 2:
            raise ValueError(f"{name} must be float32 [>= N][d/2]")


def fa_rope(x, out, rope_cos, rope_sin) -> None:
    """Call ``fa_rope`` on ``[B][H][N][d]`` tensors (``out`` may be ``x``)."""
    if x.dim() != 4:
        raise ValueError("x must be [B][H][N][d]")
    B, H, N, d = x.shape
    _check_dense("x", x, x.device)
    _check_dense("out", out, x.device)
    if tuple(out.shape) != tuple(x.shape) or out.dtype != x.dtype:
        raise ValueError("out must match x")
    _check_tables(rope_cos, rope_sin, N, d, x.device)
    st = load_library().fa_rope(_ptr(x), _ptr(out), _ptr(rope_cos), _ptr(rope_sin), B, H, N, d,
                                _dtype_code(x), _stream(x.device))
    if st != FA_OK:
        raise FaError(st, "fa_rope")


def fa_fwd_rope_workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(load_library().fa_fwd_rope_workspace_size(B, H, N, d))


def fa_fwd_rope(q, k, v, o, lse, rope_cos, rope_sin, causal: bool, scale: float,
                workspace) -> None:
    """Call ``fa_fwd_rope``: ``fa_fwd`` on RoPE-rotated q and k."""
    if q.dim() != 4:
        raise ValueError("q must be [B][H][N][d]")
    B, H, N, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("workspace", workspace)):
        _check_dense(name, t, dev)
    for name, t in (("k", k), ("v", v), ("o", o)):
        if tuple(t.shape) != (B, H, N, d) or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q's shape and dtype")
    if lse is not None:
        _check_dense("lse", lse, dev)
        if tuple(lse.shape) != (B, H, N) or lse.dtype != _torch().float32:
            raise ValueError("lse must be float32 [B][H][N]")
    _check_tables(rope_cos, rope_sin, N, d, dev)
    st = load_library().fa_fwd_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                    _ptr(rope_cos), _ptr(rope_sin), B, H, N, d,
                                    int(bool(causal)), float(scale), _dtype_code(q),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(dev))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_rope")


# --------------------------------------------------------------------------
# convenience wrappers that allocate outputs with torch
# --------------------------------------------------------------------------
def attention(q, k, v, causal: bool = False, scale: float | None = None):
    """Exact attention forward.  Returns ``(o, lse)``; scale defaults to 1/sqrt(d)."""
    torch = _torch()
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, causal, scale)
    return o, lse


def attention_backward(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
                       workspace=None):
    """Exact attention backward from the forward's ``(o, lse)``.  Returns ``(dq, dk, dv)``;
    allocates the workspace if not given.  scale defaults to 1/sqrt(d)."""
    torch = _torch()
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = torch.empty(max(fa_bwd_workspace_size(B, H, N, d), 1), dtype=torch.uint8,
                                device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, causal, scale, workspace)
    return dq, dk, dv


def paged_prefill(q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q, max_q_len: int,
                  causal: bool = True, scale: float | None = None):
    """Prefill of new tokens against a paged KV cache.  Returns ``(o, lse)``."""
    torch = _torch()
    total_q, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((total_q, H), dtype=torch.float32, device=q.device)
    fa_paged_prefill(q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q, o, lse,
                     max_q_len, causal, scale)
    return o, lse


def tree_decode(q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q, tree_parents,
                max_q_len: int, scale: float | None = None):
    """Draft-tree verification against a paged KV cache.  Returns ``(o, lse)``."""
    torch = _torch()
    total_q, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((total_q, H), dtype=torch.float32, device=q.device)
    fa_tree_decode(q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q, tree_parents, o, lse,
                   max_q_len, scale)
    return o, lse


def rope(x, rope_cos, rope_sin):
    """RoPE of ``x [B][H][N][d]`` (row n at position n).  Returns a new tensor."""
    out = _torch().empty_like(x)
    fa_rope(x, out, rope_cos, rope_sin)
    return out


def attention_rope(q, k, v, rope_cos, rope_sin, causal: bool = False, scale: float | None = None,
                   workspace=None):
    """Attention of RoPE-rotated q and k, query rotation fused.  Returns ``(o, lse)``."""
    torch = _torch()
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = torch.empty(max(fa_fwd_rope_workspace_size(B, H, N, d), 1), dtype=torch.uint8,
                                device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    fa_fwd_rope(q, k, v, o, lse, rope_cos, rope_sin, causal, scale, workspace)
    return o, lse


def paged_decode(q, k_cache, v_cache, block_table, seq_lens, scale: float | None = None,
                 workspace=None):
    """Paged-KV decode.  Returns ``(o, lse)``; allocates the workspace if not given."""
    torch = _torch()
    S, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        n = fa_paged_decode_workspace_size(S, H, d, k_cache.shape[2], block_table.shape[1])
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((S, H), dtype=torch.float32, device=q.device)
    fa_paged_decode(q, k_cache, v_cache, block_table, seq_lens, o, lse, scale, workspace)
    return o, lse
