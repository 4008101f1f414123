"""CPU oracle for exact attention -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call this module.  It shares no code with the HIP
path (``exact_attention_26_amd/``) and imports nothing from it.

Everything is computed in float64 with numpy, straight from the definition,
materialising the score matrix (one block of query rows at a time, which only
bounds memory and does not change the arithmetic):

    S = scale * Q K^T                      (similarity = dot product, scaled)
    S_ij = -inf where key j is hidden      (causal: j > i)
    m_i = max_j S_ij,  P = exp(S - m),  l_i = sum_j P_ij
    O = (P V) / l,     LSE_i = m_i + ln l_i

Sources: "LLM study notes" (DEVOCEAN tech blog), section on the self-attention
computation (Q/K/V, dot-product similarity, division by the square root of the
key dimension, softmax, weighting of the values); "Flash Attention" (velog
@myungum), section 1 (scaled dot-product attention, several heads side by
side) and section 2 (the method computes exact attention, so its result is this
definition up to rounding); "How does Flash Attention reduce memory traffic in
local inference?" (ZimaSpace blog), section on standard attention (the naive
form that stores the full score matrix -- which is what this oracle is).  The
causal mask is the one of "FlashAttention-2 GPU work partitioning" (iPLEX blog,
section 4): a query sees the current and earlier tokens.  Paged decode follows
"LLM study notes", section "Paged attention": a block table maps each
sequence's logical pages to physical pages of the cache.

Readings where the pages are silent (all pinned by tests in tests/test_oracle.py):
  * the scale multiplies Q K^T before the max and the exponential;
  * LSE is the natural log of sum_j exp(S_ij), with S already scaled;
  * causal is square with no offset: query i sees keys 0..i;
  * decode: the single query of a sequence sees all of its seq_len cached
    tokens; seq_len <= 0 gives O = 0 and LSE = -inf (the empty sum);
  * prefill over the paged cache: a sequence's new tokens are the last ones of
    its seq_len cached tokens, so causal query i of n new ones sees positions
    0 .. seq_len - n + i; a query that sees nothing gets O = 0, LSE = -inf;
  * tree attention (speculative decoding): a draft tree's node sees the
    committed tokens and the nodes on its own path from the root (its
    ancestors and itself), nothing else of the tree;
  * RoPE: consecutive pairs (x[2i], x[2i+1]) of a row form one complex
    number, rotated by the angle whose cosine and sine the caller's tables
    hold for the row's position and pair i.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["attention_fp64", "attention_bruteforce", "paged_gather_fp64", "paged_decode_fp64",
           "paged_prefill_fp64", "tree_ancestors", "tree_decode_fp64", "rope_fp64",
           "attention_rope_fp64", "attention_backward_fp64"]


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def attention_fp64(q, k, v, *, causal: bool = False, scale: float | None = None,
                   rows=None, row_block: int = 256):
    """Exact attention in float64.

    q: ``[..., Nq, d]``, k and v: ``[..., Nk, d]`` (same leading dims).  With
    ``causal`` the mask is square (``Nq == Nk``) and query i sees keys
    ``0..i``.  ``rows`` optionally selects query rows (indices into Nq); the
    result then has ``len(rows)`` rows and each row is exactly the row the full
    call would give.  ``scale`` defaults to ``1/sqrt(d)``.

    Returns ``(o [..., R, d], lse [..., R])`` as float64.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    *lead, nq, d = q.shape
    nk = k.shape[-2]
    if k.shape[:-2] != tuple(lead) or v.shape[:-2] != tuple(lead) or k.shape[-1] != d \
            or v.shape[-2] != nk:
        raise ValueError("q, k, v shapes do not agree")
    if causal and nq != nk:
        raise ValueError("causal attention here is square (Nq == Nk)")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(nq) if rows is None else np.asarray(rows, dtype=np.int64).reshape(-1)
    g = int(np.prod(lead)) if lead else 1
    qf = q.reshape(g, nq, d)
    kf = k.reshape(g, nk, d)
    vf = v.reshape(g, nk, v.shape[-1])
    o = np.empty((g, rows.size, v.shape[-1]), dtype=np.float64)
    lse = np.empty((g, rows.size), dtype=np.float64)
    keys = np.arange(nk)
    for gi in range(g):
        for r0 in range(0, rows.size, row_block):
            rr = rows[r0:r0 + row_block]
            s = scale * (qf[gi, rr, :] @ kf[gi].T)              # [r, nk]
            if causal:
                s = np.where(keys[None, :] > rr[:, None], -np.inf, s)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            l = p.sum(axis=1, keepdims=True)
            o[gi, r0:r0 + rr.size] = (p @ vf[gi]) / l
            lse[gi, r0:r0 + rr.size] = (m + np.log(l))[:, 0]
    return o.reshape(*lead, rows.size, v.shape[-1]), lse.reshape(*lead, rows.size)


def attention_bruteforce(q, k, v, *, causal: bool = False, scale: float | None = None):
    """Scalar loops over Python floats, for tiny inputs (N <= 16).

    For one head: ``q [Nq][d]``, ``k [Nk][d]``, ``v [Nk][dv]`` as nested
    sequences.  Uses the softmax exactly as defined, exp(s_ij) / sum_j exp(s_ij)
    with no max subtraction (so keep |s| well below 700), and ``math.fsum`` for
    the sums.  Returns ``(o, lse)`` as nested lists.
    """
    q = [[float(x) for x in row] for row in q]
    k = [[float(x) for x in row] for row in k]
    v = [[float(x) for x in row] for row in v]
    d = len(q[0])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o, lse = [], []
    for i, qi in enumerate(q):
        seen = [j for j in range(len(k)) if not (causal and j > i)]
        w = [math.exp(scale * math.fsum(a * b for a, b in zip(qi, k[j]))) for j in seen]
        z = math.fsum(w)
        o.append([math.fsum(w[t] * v[j][c] for t, j in enumerate(seen)) / z
                  for c in range(len(v[0]))])
        lse.append(math.log(z))
    return o, lse


def paged_gather_fp64(k_cache, v_cache, block_table, seq_len: int, seq: int, head: int):
    """Logical K and V rows ``[L][d]`` of one (sequence, head), read through the table.

    Logical page p of the sequence holds tokens ``p*page_size ..
    p*page_size + page_size - 1`` and lives in physical page
    ``block_table[seq][p]`` of a ``[num_blocks][H][page_size][d]`` cache.
    Only the first ``seq_len`` tokens are returned (slots past the end of the
    last page are never touched).
    """
    page_size = k_cache.shape[2]
    n_pages = -(-seq_len // page_size)
    if n_pages > block_table.shape[1]:
        raise ValueError("seq_len exceeds the block table")
    ks, vs = [], []
    for p in range(n_pages):
        blk = int(block_table[seq][p])
        take = min(page_size, seq_len - p * page_size)
        ks.append(_as64(k_cache[blk, head, :take, :]))
        vs.append(_as64(v_cache[blk, head, :take, :]))
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def paged_decode_fp64(q, k_cache, v_cache, block_table, seq_lens, *, scale: float | None = None,
                      pairs=None):
    """One query per sequence against a paged KV cache, float64.

    q: ``[S][H][d]``; caches ``[num_blocks][H][page_size][d]``; block_table
    ``[S][max_blocks]``; seq_lens ``[S]``.  The query of sequence s sees all of
    its ``seq_lens[s]`` tokens.  ``pairs`` optionally lists ``(s, h)`` to
    compute; the result then holds those entries in order.

    Returns ``(o, lse)``: ``[S][H][d]`` and ``[S][H]`` (or ``[len(pairs)][d]``
    and ``[len(pairs)]``).  ``seq_lens[s] <= 0`` gives ``o = 0``,
    ``lse = -inf``.
    """
    S, H, d = np.shape(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    want = [(s, h) for s in range(S) for h in range(H)] if pairs is None else list(pairs)
    o = np.zeros((len(want), d), dtype=np.float64)
    lse = np.full(len(want), -np.inf, dtype=np.float64)
    for n, (s, h) in enumerate(want):
        L = int(seq_lens[s])
        if L <= 0:
            continue
        ks, vs = paged_gather_fp64(k_cache, v_cache, block_table, L, s, h)
        oo, ll = attention_fp64(_as64(q[s, h])[None, :], ks, vs, causal=False, scale=scale)
        o[n] = oo[0]
        lse[n] = ll[0]
    if pairs is None:
        return o.reshape(S, H, d), lse.reshape(S, H)
    return o, lse


def paged_prefill_fp64(q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q, *,
                       causal: bool = True, scale: float | None = None, rows=None):
    """A batch of sequences, each with new query tokens, against a paged KV cache, float64.

    Sequence s holds ``L = seq_lens[s]`` cached tokens, read through its row of
    the block table ("LLM study notes", section "Paged attention"); its new
    tokens are the last ``n_s = cu_seqlens_q[s+1] - cu_seqlens_q[s]`` of them,
    and their queries are rows ``cu_seqlens_q[s] ..`` of the packed ``q``.
    Query i of the sequence stands at position ``L - n_s + i``; with ``causal``
    it sees the keys at positions ``0 .. L - n_s + i`` (the current and earlier
    tokens, "FlashAttention-2 GPU work partitioning", section 4), otherwise all
    L keys.  A query that sees no key gets o = 0 and lse = -inf (the empty sum).

    q: ``[total_q][H][d]``; caches ``[num_blocks][H][page_size][d]``;
    block_table ``[S][max_blocks]``; seq_lens ``[S]``; cu_seqlens_q ``[S+1]``.
    ``rows`` optionally lists packed query rows to compute (result in that
    order).  Returns ``(o [R][H][d], lse [R][H])`` as float64.
    """
    q = _as64(q)
    total_q, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    S = cu.size - 1
    want = np.arange(total_q) if rows is None else np.asarray(rows, dtype=np.int64).reshape(-1)
    o = np.zeros((want.size, H, d), dtype=np.float64)
    lse = np.full((want.size, H), -np.inf, dtype=np.float64)
    for s in range(S):
        lo, hi = int(cu[s]), int(cu[s + 1])
        sel = np.nonzero((want >= lo) & (want < hi))[0]
        if sel.size == 0:
            continue
        L = int(seq_lens[s])
        if L <= 0:
            continue
        i = want[sel] - lo                                  # index among the new tokens
        pos = L - (hi - lo) + i                             # position of each query
        keys = np.arange(L)
        for h in range(H):
            ks, vs = paged_gather_fp64(k_cache, v_cache, block_table, L, s, h)
            sc = scale * (q[want[sel], h, :] @ ks.T)        # [rows, L]
            if causal:
                sc = np.where(keys[None, :] > pos[:, None], -np.inf, sc)
            m = sc.max(axis=1, keepdims=True)
            seen = np.isfinite(m[:, 0])
            p = np.exp(sc[seen] - m[seen])
            l = p.sum(axis=1, keepdims=True)
            o[sel[seen], h] = (p @ vs) / l
            lse[sel[seen], h] = (m[seen] + np.log(l))[:, 0]
    return o, lse


def tree_ancestors(parents) -> list:
    """For each node of a draft tree, the set of nodes on its path from the
    root: itself, its parent, its parent's parent, ...  ``parents[i]`` is the
    index of node i's parent among the tree's nodes, or -1 when node i hangs
    directly off the committed tokens.  Nodes come parents-first
    (``parents[i] < i``); a parent index outside ``[0, i)`` is taken as -1.
    """
    out = []
    for i, p in enumerate(int(x) for x in parents):
        path = {i}
        while 0 <= p < i and p not in path:
            path.add(p)
            p = int(parents[p]) if 0 <= int(parents[p]) < p else -1
        out.append(path)
    return out


def tree_decode_fp64(q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q, parents, *,
                     scale: float | None = None):
    """Verification of a draft token tree in one pass, float64.

    "LLM study notes" (DEVOCEAN tech blog), speculative decoding section: a
    draft model proposes candidate tokens organised as a tree, each node one
    token, and the target model computes all nodes in a single forward pass
    with tree attention.  Here sequence s holds ``L = seq_lens[s]`` cached
    tokens read through its block table ("Paged attention" section); its
    ``n = cu_seqlens_q[s+1] - cu_seqlens_q[s]`` tree nodes are the last n of
    them, in node order, and their queries are rows ``cu_seqlens_q[s] ..`` of
    ``q``.  Node i sees the L - n committed tokens and the nodes of its own
    path from the root (``tree_ancestors``); ``parents`` is packed like ``q``.

    Returns ``(o [total_q][H][d], lse [total_q][H])``; a node that sees
    nothing gets o = 0, lse = -inf.
    """
    q = _as64(q)
    total_q, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    o = np.zeros((total_q, H, d), dtype=np.float64)
    lse = np.full((total_q, H), -np.inf, dtype=np.float64)
    for s in range(cu.size - 1):
        lo, hi = int(cu[s]), int(cu[s + 1])
        n, L = hi - lo, int(seq_lens[s])
        if n <= 0 or L <= 0:
            continue
        ctx = L - n
        paths = tree_ancestors(np.asarray(parents)[lo:hi])
        # keys node i sees: the committed tokens, then its path's tree tokens
        seen_of = [np.concatenate([np.arange(max(ctx, 0)),
                                   np.array(sorted(ctx + j for j in paths[i] if 0 <= ctx + j < L),
                                            dtype=np.int64)]).astype(np.int64)
                   for i in range(n)]
        for h in range(H):
            ks, vs = paged_gather_fp64(k_cache, v_cache, block_table, L, s, h)
            scores = scale * (ks @ q[lo:hi, h].T)             # [L, n]: every key, every node
            for i in range(n):
                seen = seen_of[i]
                if seen.size == 0:
                    continue
                sc = scores[seen, i]
                m = sc.max()
                p = np.zeros(L)                                # unseen keys weigh nothing
                p[seen] = np.exp(sc - m)
                o[lo + i, h] = (p @ vs) / p.sum()
                lse[lo + i, h] = m + np.log(p.sum())
    return o, lse


def rope_fp64(x, cos, sin, positions=None):
    """Rotary position embedding, float64.

    "LLM study notes" (DEVOCEAN tech blog), RoPE section: each token's
    embedding is read as complex numbers and rotated in the complex plane by
    an angle given by the token's absolute position, so that the inner
    product of two rotated vectors depends on their relative position only.
    Here the complex numbers are consecutive pairs, z_i = x[2i] + j x[2i+1],
    and row n of ``x [..., N, d]`` is rotated by the angle of position
    ``positions[n]`` (default n): z_i -> z_i * (cos[p, i] + j sin[p, i]),
    with ``cos``, ``sin`` of shape ``[P, d/2]``.
    """
    x = _as64(x)
    n, d = x.shape[-2], x.shape[-1]
    pos = np.arange(n) if positions is None else np.asarray(positions, dtype=np.int64)
    c = _as64(cos)[pos]                                 # [N, d/2]
    s = _as64(sin)[pos]
    re, im = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = re * c - im * s
    out[..., 1::2] = re * s + im * c
    return out


def attention_rope_fp64(q, k, v, cos, sin, *, causal: bool = False, scale: float | None = None,
                        rows=None, row_block: int = 256):
    """Attention of RoPE-rotated queries and keys (row n at position n), float64:
    ``attention_fp64(rope(q), rope(k), v)``."""
    return attention_fp64(rope_fp64(q, cos, sin), rope_fp64(k, cos, sin), v, causal=causal,
                          scale=scale, rows=rows, row_block=row_block)


def attention_backward_fp64(q, k, v, do, *, causal: bool = False, scale: float | None = None,
                            row_block: int | None = None):
    """Gradients of O = softmax(scale * Q K^T) V with respect to Q, K, V, float64.

    Written from the chain rule of the definition above, with the softmax
    probabilities materialised per (batch, head):
        P = softmax(S) row-wise (hidden keys get P = 0),
        dV = P^T dO,
        dP = dO V^T,
        dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)       (softmax Jacobian),
        dQ = scale * dS K,   dK = scale * dS^T Q.
    The backward pass the pages describe reuses the forward's stored row
    statistics and recomputes the scores blockwise ("PagedAttention vs
    FlashAttention: key differences", training section; "LLM study notes",
    FlashAttention core principles: recomputation); the result it must reach is
    this plain gradient.  Note sum_k P_ik dP_ik = sum_d dO_id O_id.

    ``row_block`` (default: all rows at once) takes the query rows in blocks
    of that many, which only bounds memory: each row's P, dP, dS and dQ are
    computed exactly as above, and dK, dV add up the blocks' contributions.

    q, k, v, do: ``[..., N, d]``.  Returns ``(dq, dk, dv)`` as float64.
    """
    q, k, v, do = (_as64(x) for x in (q, k, v, do))
    *lead, n, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rb = n if row_block is None else max(1, int(row_block))
    g = int(np.prod(lead)) if lead else 1
    qf, kf, vf, dof = (x.reshape(g, n, d) for x in (q, k, v, do))
    dq = np.empty_like(qf)
    dk = np.zeros_like(kf)
    dv = np.zeros_like(vf)
    keys = np.arange(n)
    for gi in range(g):
        for r0 in range(0, n, rb):
            rows = np.arange(r0, min(n, r0 + rb))
            s_ = scale * (qf[gi, rows] @ kf[gi].T)
            if causal:
                s_ = np.where(keys[None, :] > rows[:, None], -np.inf, s_)
            m = s_.max(axis=1, keepdims=True)
            p_ = np.exp(s_ - m)
            p_ /= p_.sum(axis=1, keepdims=True)
            dv[gi] += p_.T @ dof[gi, rows]
            dp = dof[gi, rows] @ vf[gi].T
            ds = p_ * (dp - (p_ * dp).sum(axis=1, keepdims=True))
            dq[gi, rows] = scale * (ds @ kf[gi])
            dk[gi] += scale * (ds.T @ qf[gi, rows])
    shape = tuple(lead) + (n, d)
    return dq.reshape(shape), dk.reshape(shape), dv.reshape(shape)
