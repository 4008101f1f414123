"""Pins for the tree-attention oracle (verification of a draft token tree):

  * a hand-derived fixture (tests/golden/tree_two_sequences_page2.json):
    siblings do not see each other, a node sees its parent chain and the
    committed tokens, two roots hang off the same context;
  * the path sets themselves on hand-written trees, including parents out of
    range (taken as roots);
  * a chain tree (each node the child of the previous one) is causal prefill
    of the same tokens (the prefill oracle, pinned in test_oracle_prefill.py);
  * a star tree (every node a child of the context) is, node by node, plain
    attention over the context plus that node (the dense oracle);
  * a node's result does not move when the K/V of a node off its path change,
    and does move when those of a node on its path change;
  * planted mistakes (self hidden, siblings visible, context hidden,
    descendants instead of ancestors, parents ignored) each fail a pin.
"""
import math

import numpy as np
import pytest

import golden_values as gv
from oracle import (attention_fp64, paged_gather_fp64, paged_prefill_fp64, tree_ancestors,
                    tree_decode_fp64)


def _golden():
    fx = gv.load("tree_two_sequences_page2.json")
    return fx, (gv.array(fx["q"]), gv.array(fx["k_cache"]), gv.array(fx["v_cache"]),
                np.array(fx["block_table"], dtype=np.int32),
                np.array(fx["seq_lens"], dtype=np.int32),
                np.array(fx["cu_seqlens_q"], dtype=np.int32),
                np.array(fx["parents"], dtype=np.int32))


def _batch(rng, ctx, parents_per_seq, H=2, d=8, P=4):
    """Random caches for sequences of ``ctx[s]`` committed tokens followed by
    the nodes of ``parents_per_seq[s]``; shuffled pages, NaN in unused slots."""
    S = len(ctx)
    news = [len(p) for p in parents_per_seq]
    lens = np.array([c + n for c, n in zip(ctx, news)], dtype=np.int32)
    pages = -(-int(lens.max()) // P)
    table = rng.permutation(S * pages).astype(np.int32).reshape(S, pages)
    kc = np.full((S * pages + 1, H, P, d), np.nan)
    vc = np.full((S * pages + 1, H, P, d), np.nan)
    for s in range(S):
        for t in range(int(lens[s])):
            kc[table[s, t // P], :, t % P] = rng.standard_normal((H, d))
            vc[table[s, t // P], :, t % P] = rng.standard_normal((H, d))
    cu = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q = rng.standard_normal((int(cu[-1]), H, d))
    parents = np.concatenate([np.asarray(p, dtype=np.int32) for p in parents_per_seq])
    return q, kc, vc, table, lens, cu, parents


def pin_golden(tree):
    fx, (q, kc, vc, bt, sl, cu, par) = _golden()
    o, lse = tree(q, kc, vc, bt, sl, cu, par, scale=gv.value(fx["scale"]))
    np.testing.assert_allclose(o, gv.array(fx["expected"]["o"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, gv.array(fx["expected"]["lse"]), rtol=0, atol=1e-12)


def pin_chain_is_causal_prefill(tree):
    rng = np.random.default_rng(51)
    ctx = [7, 0, 12]
    chains = [[-1] + list(range(n - 1)) for n in (5, 9, 1)]
    q, kc, vc, bt, sl, cu, par = _batch(rng, ctx, chains)
    o, lse = tree(q, kc, vc, bt, sl, cu, par, scale=0.4)
    ro, rl = paged_prefill_fp64(q, kc, vc, bt, sl, cu, causal=True, scale=0.4)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def pin_star_is_context_plus_self(tree):
    rng = np.random.default_rng(52)
    ctx = [6, 10]
    stars = [[-1] * 4, [-1] * 3]
    q, kc, vc, bt, sl, cu, par = _batch(rng, ctx, stars)
    o, lse = tree(q, kc, vc, bt, sl, cu, par, scale=0.3)
    for s in range(2):
        L = int(sl[s])
        for h in range(q.shape[1]):
            ks, vs = paged_gather_fp64(kc, vc, bt, L, s, h)
            for i in range(len(stars[s])):
                keep = list(range(ctx[s])) + [ctx[s] + i]
                row = cu[s] + i
                ro, rl = attention_fp64(q[row, h][None], ks[keep], vs[keep], scale=0.3)
                np.testing.assert_allclose(o[row, h], ro[0], rtol=0, atol=1e-12)
                np.testing.assert_allclose(lse[row, h], rl[0], rtol=0, atol=1e-12)


def pin_only_the_path_matters(tree):
    rng = np.random.default_rng(53)
    parents = [-1, 0, 0, 1, 2, 2, -1]
    q, kc, vc, bt, sl, cu, par = _batch(rng, [5], [parents])
    o, lse = tree(q, kc, vc, bt, sl, cu, par, scale=0.5)
    paths = [{0}, {0, 1}, {0, 2}, {0, 1, 3}, {0, 2, 4}, {0, 2, 5}, {6}]
    P = kc.shape[2]
    for j in range(len(parents)):                 # disturb node j's K and V
        kc2, vc2 = kc.copy(), vc.copy()
        t = 5 + j
        kc2[bt[0, t // P], :, t % P] += 1.0
        vc2[bt[0, t // P], :, t % P] -= 2.0
        o2, _ = tree(q, kc2, vc2, bt, sl, cu, par, scale=0.5)
        for i, path in enumerate(paths):
            moved = not np.allclose(o2[i], o[i], rtol=0, atol=1e-13)
            assert moved == (j in path), (i, j)


PINS = [pin_golden, pin_chain_is_causal_prefill, pin_star_is_context_plus_self,
        pin_only_the_path_matters]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_tree_oracle_passes_pin(pin):
    pin(tree_decode_fp64)


def test_tree_ancestors_by_hand():
    assert tree_ancestors([-1, 0, 0, 1, 1, 2, -1, 6]) == [
        {0}, {0, 1}, {0, 2}, {0, 1, 3}, {0, 1, 4}, {0, 2, 5}, {6}, {6, 7}]
    # parents must precede their children; anything else hangs off the context
    assert tree_ancestors([5, -7, 1, 3]) == [{0}, {1}, {1, 2}, {3}]


def _mutant(kind):
    def tree(q, kc, vc, table, lens, cu, parents, *, scale=None):
        total, H, d = q.shape
        P = kc.shape[2]
        o = np.zeros((total, H, d))
        lse = np.full((total, H), -np.inf)
        for s in range(len(cu) - 1):
            lo, hi = int(cu[s]), int(cu[s + 1])
            n, L = hi - lo, int(lens[s])
            ctx = L - n
            par = [int(p) for p in parents[lo:hi]]
            for i in range(n):
                if kind == "siblings_visible":
                    path = set(range(i + 1))
                elif kind == "descendants":
                    path = {j for j in range(n) if i in tree_ancestors(par)[j]}
                elif kind == "parents_ignored":
                    path = {i}
                else:
                    path = tree_ancestors(par)[i]
                if kind == "self_hidden":
                    path = path - {i}
                seen = [t for t in range(L)
                        if (t < ctx and kind != "context_hidden") or (t >= ctx and t - ctx in path)]
                for h in range(H):
                    if not seen:
                        continue
                    ks = np.array([kc[table[s, t // P], h, t % P] for t in seen])
                    vs = np.array([vc[table[s, t // P], h, t % P] for t in seen])
                    sc = scale * (ks @ q[lo + i, h])
                    m = sc.max()
                    w = np.exp(sc - m)
                    o[lo + i, h] = (w @ vs) / w.sum()
                    lse[lo + i, h] = m + math.log(w.sum())
        return o, lse
    return tree


@pytest.mark.parametrize("kind", ["self_hidden", "siblings_visible", "context_hidden",
                                  "descendants", "parents_ignored"])
def test_tree_mutant_is_caught(kind):
    caught = []
    for pin in PINS:
        try:
            pin(_mutant(kind))
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"tree mutant {kind} passed every pin"


def test_tree_unmutated_copy_passes():
    for pin in PINS:
        pin(_mutant("none"))
