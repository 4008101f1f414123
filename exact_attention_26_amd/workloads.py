"""Seeded synthetic workloads shared by the tests, the bench and the oracle side.

This module only draws random numbers and arranges them into the layouts the
library takes (dense ``[B][H][N][d]`` tensors, a paged KV pool with a block
table).  It holds none of the attention arithmetic, imports nothing from the
library or from ``oracle/``, and needs only numpy.

Shapes follow the workloads the pages describe:

* the FlashAttention-2 attention benchmark ("FlashAttention-2 GPU work
  partitioning", iPLEX blog, section 4): sequence length 512 to 16k with the
  total token count fixed at 16k, head dimension 64 and 128, with and without
  the causal mask;
* a paged KV cache read through a block table, with prompt pages shared between
  sequences ("LLM study notes", DEVOCEAN tech blog, section "Paged attention").

Every value is drawn as float32 from ``numpy.random.default_rng`` and, for
bf16 workloads, rounded once to the nearest bf16 (ties to even).  The arrays
returned are float32 holding exactly those bf16 values, so the GPU side can
convert them to bf16 without any further rounding and the oracle can widen
them to float64 exactly.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "FwdConfig", "FWD_CONFIGS", "round_to_bf16", "fwd_inputs",
    "DecodeLayout", "decode_layout", "decode_q", "decode_pool", "decode_pool_pages",
    "page_valid_slots", "fwd_config_inputs", "bwd_dout",
    "DECODE_C4", "PrefillWorkload", "prefill_workload", "prefill_q", "PREFILL_P1",
    "tree_parents", "tree_workload", "TREE_T1", "rope_tables",
]


# --------------------------------------------------------------------------
# rounding (input preparation only)
# --------------------------------------------------------------------------
def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16, ties to even.

    Returns float32 values that are exactly representable in bf16.  NaN and
    infinities are not expected here (inputs are finite normals).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = ((u + bias) & np.uint32(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32)


# --------------------------------------------------------------------------
# dense forward workloads
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class FwdConfig:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "bf16" or "f32"
    causal: tuple         # modes the workload is run in
    seed: int
    sigma_qk: float = 1.0
    sigma_v: float = 1.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


def _sweep(n: int) -> FwdConfig:
    return FwdConfig(f"sweep_N{n}", B=16384 // n, H=32, N=n, d=64, dtype="bf16",
                     causal=(False, True), seed=2000 + n)


FWD_CONFIGS: dict[str, FwdConfig] = {
    # smoke: small enough for the oracle in well under a second
    "smoke": FwdConfig("smoke", B=1, H=2, N=256, d=64, dtype="f32", causal=(False,), seed=0),
    # forward bench: 16k tokens, d=128
    "fwd_b8_h16_n2048_d128": FwdConfig("fwd_b8_h16_n2048_d128", B=8, H=16, N=2048, d=128,
                                       dtype="bf16", causal=(False, True), seed=1),
    # sequence sweep at a fixed 16k tokens, d=64
    **{f"sweep_N{n}": _sweep(n) for n in (512, 1024, 2048, 4096, 8192, 16384)},
    # long context with large logits (std of q.k*scale is about 9)
    "long_b1_h16_n16384_d128": FwdConfig("long_b1_h16_n16384_d128", B=1, H=16, N=16384, d=128,
                                         dtype="bf16", causal=(True,), seed=3, sigma_qk=3.0),
}


def fwd_inputs(B: int, H: int, N: int, d: int, *, seed: int, dtype: str = "bf16",
               sigma_qk: float = 1.0, sigma_v: float = 1.0):
    """Draw q, k, v of shape ``[B][H][N][d]`` in the order q, k, v.

    Values are ``standard_normal * sigma`` in float32; for ``dtype="bf16"``
    each value is rounded once to bf16.  Returns float32 arrays.
    """
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    out = []
    for sigma in (sigma_qk, sigma_qk, sigma_v):
        x = rng.standard_normal(shape, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        if dtype == "bf16":
            x = round_to_bf16(x)
        elif dtype != "f32":
            raise ValueError(f"unknown dtype {dtype!r}")
        out.append(x)
    return tuple(out)


def fwd_config_inputs(cfg: FwdConfig):
    return fwd_inputs(cfg.B, cfg.H, cfg.N, cfg.d, seed=cfg.seed, dtype=cfg.dtype,
                      sigma_qk=cfg.sigma_qk, sigma_v=cfg.sigma_v)


def bwd_dout(B: int, H: int, N: int, d: int, *, seed: int, dtype: str = "bf16",
             sigma: float = 1.0) -> np.ndarray:
    """The incoming gradient dO of shape ``[B][H][N][d]`` for a backward pass.

    Drawn from its own stream (``default_rng([seed, 5])``), so the forward
    inputs of the same seed are unchanged; ``standard_normal * sigma``,
    rounded once to bf16 for ``dtype="bf16"``.
    """
    x = np.random.default_rng([seed, 5]).standard_normal((B, H, N, d), dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return x


def rope_tables(n_pos: int, d: int, base: float = 10000.0):
    """Cosine and sine tables ``[n_pos][d/2]`` float32 of the usual rotary
    frequencies: pair i of position p turns by p * base^(-2i/d) radians
    (angles formed in float64, then rounded once to float32).  The tables are
    inputs of the RoPE path; any other frequency schedule is just another table."""
    i = np.arange(d // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / d)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


# --------------------------------------------------------------------------
# paged KV decode workloads
# --------------------------------------------------------------------------
POOL_CHUNK_PAGES = 256   # pages per independently seeded chunk of the pool


@dataclass
class DecodeLayout:
    """A paged KV cache layout: which physical page holds which tokens.

    ``block_table[s, p]`` is the physical page holding tokens
    ``p*page_size .. p*page_size + page_size - 1`` of sequence ``s``.  Table
    entries past a sequence's last page point at ``poison_page``.
    ``k_cache``/``v_cache`` are laid out ``[num_blocks][H][page_size][d]``.
    """
    seed: int
    S: int
    H: int
    d: int
    page_size: int
    seq_lens: np.ndarray          # int32 [S]
    block_table: np.ndarray       # int32 [S][max_blocks]
    num_blocks: int
    poison_page: int
    shared_pages: np.ndarray      # int64 ids of pages referenced by two sequences
    spare_pages: np.ndarray       # int64 ids of pages no sequence references
    scale: float = field(default=0.0)

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    def used_pages(self, s: int) -> np.ndarray:
        n = -(-int(self.seq_lens[s]) // self.page_size) if self.seq_lens[s] > 0 else 0
        return self.block_table[s, :n].astype(np.int64)

    def distinct_pages(self) -> np.ndarray:
        ids = [self.used_pages(s) for s in range(self.S)]
        return np.unique(np.concatenate(ids)) if ids else np.zeros(0, np.int64)


def decode_layout(seed: int, *, S: int = 64, H: int = 32, d: int = 128, page_size: int = 16,
                  lens=None, len_range=(128, 8192), shared_prefix: int = 512,
                  spare: int = 64, max_blocks: int | None = None) -> DecodeLayout:
    """Build the block table of a shuffled paged KV pool.

    Lengths are drawn uniformly in ``len_range`` (inclusive) unless ``lens`` is
    given.  Sequences ``2i`` and ``2i+1`` share their first
    ``page_size * floor(min(shared_prefix, L_2i, L_2i+1) / page_size)`` tokens
    as the same physical pages (whole pages only).  Physical ids are a random
    permutation of the pool; ``spare`` pages are referenced by nobody, the first
    of them is the poison page that unused table entries point to.
    """
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = rng.integers(len_range[0], len_range[1] + 1, S)
    lens = np.asarray(lens, dtype=np.int64)
    if lens.shape != (S,):
        raise ValueError("lens must have S entries")
    npages = np.where(lens > 0, -(-lens // page_size), 0)
    if max_blocks is None:
        max_blocks = max(1, int(-(-len_range[1] // page_size)), int(npages.max(initial=0)))
    if npages.max(initial=0) > max_blocks:
        raise ValueError("a sequence needs more pages than max_blocks")
    shared = np.zeros(S, dtype=np.int64)        # shared pages at the head of each sequence
    for a in range(0, S - 1, 2):
        sp = (min(shared_prefix, int(lens[a]), int(lens[a + 1])) // page_size)
        shared[a] = shared[a + 1] = sp
    # logical pages that need their own physical page
    owners = []                                   # (s, p) in allocation order
    for s in range(S):
        start = shared[s] if (s % 2 == 1) else 0  # the second of a pair reuses the first's pages
        for p in range(int(start), int(npages[s])):
            owners.append((s, p))
    unique = len(owners)
    pool = unique + max(1, spare)
    perm = rng.permutation(pool).astype(np.int64)
    table = np.empty((S, max_blocks), dtype=np.int64)
    poison = int(perm[unique])
    table[:] = poison
    for idx, (s, p) in enumerate(owners):
        table[s, p] = perm[idx]
    shared_ids = []
    for s in range(1, S, 2):
        for p in range(int(shared[s])):
            table[s, p] = table[s - 1, p]
            shared_ids.append(table[s, p])
    return DecodeLayout(seed=seed, S=S, H=H, d=d, page_size=page_size,
                        seq_lens=lens.astype(np.int32), block_table=table.astype(np.int32),
                        num_blocks=pool, poison_page=poison,
                        shared_pages=np.unique(np.asarray(shared_ids, dtype=np.int64)),
                        spare_pages=np.sort(perm[unique:]), scale=1.0 / math.sqrt(d))


DECODE_C4 = dict(S=64, H=32, d=128, page_size=16, len_range=(128, 8192), shared_prefix=512,
                 spare=64, seed=4)


@dataclass
class PrefillWorkload:
    """New tokens of ``S`` sequences against a paged KV cache.

    ``layout.seq_lens[s]`` counts all cached tokens of sequence s, its new
    ones included (they are the last ``new_lens[s]``); the queries of the new
    tokens are packed ``[total_q][H][d]``, sequence s at rows
    ``cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1``.
    """
    layout: DecodeLayout
    new_lens: np.ndarray          # int32 [S]
    cu_seqlens_q: np.ndarray      # int32 [S+1]

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def max_q_len(self) -> int:
        return int(self.new_lens.max(initial=0))


def prefill_workload(seed: int, *, S: int = 16, H: int = 32, d: int = 128, page_size: int = 16,
                     ctx_range=(0, 4096), new_range=(256, 1792), ctx_lens=None, new_lens=None,
                     shared_prefix: int = 0, spare: int = 16) -> PrefillWorkload:
    """Draw context and new-token counts (uniform, inclusive ranges, from
    ``default_rng([seed, 7])``) unless given, then lay the pages out as the
    decode workload does (shuffled pool, optional shared prefixes, spare and
    poison pages)."""
    rng = np.random.default_rng([seed, 7])
    ctx = (rng.integers(ctx_range[0], ctx_range[1] + 1, S) if ctx_lens is None
           else np.asarray(ctx_lens, dtype=np.int64))
    new = (rng.integers(new_range[0], new_range[1] + 1, S) if new_lens is None
           else np.asarray(new_lens, dtype=np.int64))
    lens = ctx + new
    max_blocks = max(1, int(-(-int(lens.max(initial=1)) // page_size)))
    layout = decode_layout(seed, S=S, H=H, d=d, page_size=page_size, lens=lens,
                           len_range=(0, int(lens.max(initial=1))), shared_prefix=shared_prefix,
                           spare=spare, max_blocks=max_blocks)
    cu = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    return PrefillWorkload(layout=layout, new_lens=new.astype(np.int32), cu_seqlens_q=cu)


def prefill_q(w: PrefillWorkload, dtype: str = "bf16") -> np.ndarray:
    """Queries of the new tokens, ``[total_q][H][d]`` float32 (stream ``[seed, 3]``)."""
    rng = np.random.default_rng([w.layout.seed, 3])
    x = rng.standard_normal((w.total_q, w.layout.H, w.layout.d), dtype=np.float32)
    return round_to_bf16(x) if dtype == "bf16" else x


# prefill benchmark: 16 sequences with 0..4096 cached tokens each receive
# 256..1792 new ones (about 16k new tokens in all), H=32, d=128, pages of 16
PREFILL_P1 = dict(S=16, H=32, d=128, page_size=16, ctx_range=(0, 4096), new_range=(256, 1792),
                  seed=5)


def tree_parents(seed: int, new_lens, *, max_back: int = 8) -> np.ndarray:
    """Packed parent indices of one random draft tree per sequence, int32.

    Node 0 hangs off the committed tokens (-1); node i > 0 takes a parent
    uniformly among the ``max_back`` nodes before it, or -1 (another root)
    when the draw falls before node 0.  Parents precede children.  Stream
    ``default_rng([seed, 9])``.
    """
    rng = np.random.default_rng([seed, 9])
    out = []
    for n in np.asarray(new_lens, dtype=np.int64):
        par = np.empty(int(n), dtype=np.int32)
        for i in range(int(n)):
            par[i] = -1 if i == 0 else max(-1, int(rng.integers(i - max_back, i)))
        out.append(par)
    return np.concatenate(out) if out else np.zeros(0, np.int32)


def tree_workload(seed: int, *, S: int = 64, H: int = 32, d: int = 128, page_size: int = 16,
                  ctx_range=(128, 8192), nodes: int = 64, ctx_lens=None, new_lens=None,
                  shared_prefix: int = 512, spare: int = 64):
    """Draft trees of ``nodes`` nodes appended to contexts drawn as the decode
    workload draws its lengths; returns ``(PrefillWorkload, parents)``."""
    new = np.full(S, nodes, dtype=np.int64) if new_lens is None else new_lens
    wl = prefill_workload(seed, S=S, H=H, d=d, page_size=page_size, ctx_range=ctx_range,
                          new_range=(nodes, nodes), ctx_lens=ctx_lens, new_lens=new,
                          shared_prefix=shared_prefix, spare=spare)
    return wl, tree_parents(seed, wl.new_lens)


# tree verification benchmark: 64 sequences with 128..8192 committed tokens
# (pairs sharing a 512-token prefix) each verify a 64-node draft tree, H=32, d=128
TREE_T1 = dict(S=64, H=32, d=128, page_size=16, ctx_range=(128, 8192), nodes=64, seed=6)


def decode_q(layout: DecodeLayout, dtype: str = "bf16") -> np.ndarray:
    """The single query token of every sequence: ``[S][H][d]`` float32."""
    rng = np.random.default_rng([layout.seed, 0])
    x = rng.standard_normal((layout.S, layout.H, layout.d), dtype=np.float32)
    return round_to_bf16(x) if dtype == "bf16" else x


def _pool_chunk(layout: DecodeLayout, which: int, chunk: int, dtype: str) -> np.ndarray:
    lo = chunk * POOL_CHUNK_PAGES
    hi = min(layout.num_blocks, lo + POOL_CHUNK_PAGES)
    rng = np.random.default_rng([layout.seed, which, chunk])
    x = rng.standard_normal((hi - lo, layout.H, layout.page_size, layout.d), dtype=np.float32)
    return round_to_bf16(x) if dtype == "bf16" else x


def page_valid_slots(layout: DecodeLayout) -> np.ndarray:
    """Per physical page, how many leading slots some sequence reads (0 = none)."""
    valid = np.zeros(layout.num_blocks, dtype=np.int64)
    for s in range(layout.S):
        L = int(layout.seq_lens[s])
        used = layout.used_pages(s)
        if used.size == 0:
            continue
        counts = np.full(used.size, layout.page_size, dtype=np.int64)
        counts[-1] = L - (used.size - 1) * layout.page_size
        np.maximum.at(valid, used, counts)
    return valid


def _poison_mask(valid: np.ndarray, lo: int, hi: int, page_size: int) -> np.ndarray:
    """Boolean ``[hi-lo][page_size]``: slots no sequence may read."""
    return np.arange(page_size)[None, :] >= valid[lo:hi, None]


def decode_pool(layout: DecodeLayout, which: str, *, dtype: str = "bf16", poison: bool = False,
                chunk_callback=None, threads: int = 8):
    """The K (``which="k"``) or V (``"v"``) pool ``[num_blocks][H][page_size][d]``.

    Each chunk of ``POOL_CHUNK_PAGES`` pages comes from its own seeded stream,
    so any page can be regenerated on its own (``decode_pool_pages``).  With
    ``poison=True`` every slot that no sequence may read (tails past a
    sequence's length, spare pages, the poison page) holds NaN.

    If ``chunk_callback(lo, hi, array)`` is given, chunks are handed to it in
    order and nothing is returned (lets a caller stream the pool to a device).
    """
    wid = {"k": 1, "v": 2}[which]
    nchunks = -(-layout.num_blocks // POOL_CHUNK_PAGES)
    out = None if chunk_callback else np.empty(
        (layout.num_blocks, layout.H, layout.page_size, layout.d), dtype=np.float32)

    valid = page_valid_slots(layout) if poison else None

    def make(c):
        x = _pool_chunk(layout, wid, c, dtype)
        if poison:
            lo = c * POOL_CHUNK_PAGES
            m = _poison_mask(valid, lo, lo + x.shape[0], layout.page_size)
            x[np.broadcast_to(m[:, None, :, None], x.shape)] = np.nan
        return c, x

    with ThreadPoolExecutor(max(1, threads)) as ex:
        window = []
        for c in range(nchunks):
            window.append(ex.submit(make, c))
            if len(window) >= 2 * threads or c == nchunks - 1:
                for fut in window:
                    ci, x = fut.result()
                    lo = ci * POOL_CHUNK_PAGES
                    if chunk_callback:
                        chunk_callback(lo, lo + x.shape[0], x)
                    else:
                        out[lo:lo + x.shape[0]] = x
                window = []
    return out


def decode_pool_pages(layout: DecodeLayout, which: str, pages, *, dtype: str = "bf16",
                      poison: bool = False) -> dict:
    """Regenerate only the given physical pages: ``{page_id: [H][page_size][d]}``."""
    wid = {"k": 1, "v": 2}[which]
    pages = sorted(set(int(p) for p in pages))
    by_chunk: dict[int, list[int]] = {}
    for p in pages:
        by_chunk.setdefault(p // POOL_CHUNK_PAGES, []).append(p)
    out = {}
    valid = page_valid_slots(layout) if poison else None
    for c, ps in by_chunk.items():
        x = _pool_chunk(layout, wid, c, dtype)
        lo = c * POOL_CHUNK_PAGES
        if poison:
            m = _poison_mask(valid, lo, lo + x.shape[0], layout.page_size)
            x[np.broadcast_to(m[:, None, :, None], x.shape)] = np.nan
        for p in ps:
            out[p] = x[p - lo].copy()
    return out
