"""Pins for the paged prefill oracle (new tokens of several sequences against a
paged KV cache), checked against things other than itself:

  * a hand-derived fixture (tests/golden/prefill_offset_page2.json) that fixes
    the position of the new tokens (the last n of the L cached ones), a
    sequence with more new queries than cached tokens (its first query sees
    nothing), an empty sequence and NaN in the slots nobody may read;
  * the dense oracle (itself pinned in tests/test_oracle.py): when every
    cached token is new (n = L) and the table is the identity, prefill is
    ordinary causal (or full) attention of the sequence;
  * the decode oracle (pinned there too): a single new token is a decode step,
    and in general new query i is a decode step of the sequence cut to its
    first L - n + i + 1 tokens;
  * a shuffled table gives the same result as the identity table;
  * planted mistakes (offset ignored, causal off by one, keys cut to the new
    tokens, packed rows indexed by sequence, mask inverted) each fail a pin.
"""
import math

import numpy as np
import pytest

import golden_values as gv
from oracle import attention_fp64, paged_decode_fp64, paged_prefill_fp64


def _golden():
    fx = gv.load("prefill_offset_page2.json")
    return fx, (gv.array(fx["q"]), gv.array(fx["k_cache"]), gv.array(fx["v_cache"]),
                np.array(fx["block_table"], dtype=np.int32),
                np.array(fx["seq_lens"], dtype=np.int32),
                np.array(fx["cu_seqlens_q"], dtype=np.int32))


def _scatter(k, v, page_size, table, lens):
    """Dense per-sequence K/V ``[S][H][Lmax][d]`` into pages; slots past each
    length and pages no sequence uses are NaN."""
    S, H, Lmax, d = k.shape
    nb = int(table.max()) + 2
    kc = np.full((nb, H, page_size, d), np.nan)
    vc = np.full((nb, H, page_size, d), np.nan)
    for s in range(S):
        for t in range(int(lens[s])):
            kc[table[s, t // page_size], :, t % page_size] = k[s, :, t]
            vc[table[s, t // page_size], :, t % page_size] = v[s, :, t]
    return kc, vc


def _batch(rng, lens, news, H=2, d=8, P=4, shuffle=True):
    S = len(lens)
    Lmax = max(max(lens), 1)
    pages = -(-Lmax // P)
    cu = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    k = rng.standard_normal((S, H, Lmax, d))
    v = rng.standard_normal((S, H, Lmax, d))
    q = rng.standard_normal((int(cu[-1]), H, d))
    ids = rng.permutation(S * pages) if shuffle else np.arange(S * pages)
    table = ids.astype(np.int32).reshape(S, pages)
    lens = np.array(lens, dtype=np.int32)
    kc, vc = _scatter(k, v, P, table, lens)
    return q, k, v, kc, vc, table, lens, cu


def pin_golden(prefill):
    fx, (q, kc, vc, bt, sl, cu) = _golden()
    for mode, causal in (("causal", True), ("noncausal", False)):
        o, lse = prefill(q, kc, vc, bt, sl, cu, causal=causal, scale=gv.value(fx["scale"]))
        np.testing.assert_allclose(o, gv.array(fx["expected"][mode]["o"]), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, gv.array(fx["expected"][mode]["lse"]), rtol=0, atol=1e-12)


def pin_all_new_is_dense(prefill):
    rng = np.random.default_rng(41)
    lens = [9, 16, 1, 13]
    q, k, v, kc, vc, table, sl, cu = _batch(rng, lens, lens)
    for causal in (True, False):
        o, lse = prefill(q, kc, vc, table, sl, cu, causal=causal, scale=0.4)
        for s, L in enumerate(lens):
            qs = q[cu[s]:cu[s + 1]].transpose(1, 0, 2)           # [H][L][d]
            ro, rl = attention_fp64(qs, k[s, :, :L], v[s, :, :L], causal=causal, scale=0.4)
            np.testing.assert_allclose(o[cu[s]:cu[s + 1]], ro.transpose(1, 0, 2), rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[cu[s]:cu[s + 1]], rl.T, rtol=0, atol=1e-12)


def pin_rows_are_decode_steps(prefill):
    rng = np.random.default_rng(42)
    lens, news = [11, 7, 5, 9], [3, 1, 5, 4]
    q, k, v, kc, vc, table, sl, cu = _batch(rng, lens, news)
    o, lse = prefill(q, kc, vc, table, sl, cu, causal=True, scale=0.3)
    for s in range(len(lens)):
        n = news[s]
        for i in range(n):
            cut = np.array([lens[s] - n + i + 1], dtype=np.int32)
            row = cu[s] + i
            do, dl = paged_decode_fp64(q[row][None], kc, vc, table[s:s + 1], cut, scale=0.3)
            np.testing.assert_allclose(o[row], do[0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[row], dl[0], rtol=0, atol=1e-12)
    # non-causal: every new query is a decode step over all L tokens
    o, lse = prefill(q, kc, vc, table, sl, cu, causal=False, scale=0.3)
    for s in range(len(lens)):
        for row in range(cu[s], cu[s + 1]):
            do, dl = paged_decode_fp64(q[row][None], kc, vc, table[s:s + 1], sl[s:s + 1], scale=0.3)
            np.testing.assert_allclose(o[row], do[0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[row], dl[0], rtol=0, atol=1e-12)


def pin_shuffled_equals_identity(prefill):
    lens, news = [10, 6, 12], [4, 6, 2]
    a = _batch(np.random.default_rng(43), lens, news, shuffle=False)
    b = _batch(np.random.default_rng(43), lens, news, shuffle=True)
    for causal in (True, False):
        oa, la = prefill(a[0], a[3], a[4], a[5], a[6], a[7], causal=causal, scale=0.5)
        ob, lb = prefill(b[0], b[3], b[4], b[5], b[6], b[7], causal=causal, scale=0.5)
        np.testing.assert_allclose(oa, ob, rtol=0, atol=1e-14)
        np.testing.assert_allclose(la, lb, rtol=0, atol=1e-14)


PINS = [pin_golden, pin_all_new_is_dense, pin_rows_are_decode_steps, pin_shuffled_equals_identity]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_prefill_oracle_passes_pin(pin):
    pin(paged_prefill_fp64)


def test_prefill_rows_argument():
    fx, (q, kc, vc, bt, sl, cu) = _golden()
    o, lse = paged_prefill_fp64(q, kc, vc, bt, sl, cu, causal=True, scale=1.0, rows=[4, 0])
    eo = gv.array(fx["expected"]["causal"]["o"])
    el = gv.array(fx["expected"]["causal"]["lse"])
    np.testing.assert_allclose(o, eo[[4, 0]], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, el[[4, 0]], rtol=0, atol=1e-12)


def _mutant(kind):
    def prefill(q, kc, vc, table, lens, cu, *, causal=True, scale=None):
        total, H, d = q.shape
        P = kc.shape[2]
        o = np.zeros((total, H, d))
        lse = np.full((total, H), -np.inf)
        for s in range(len(cu) - 1):
            n = int(cu[s + 1] - cu[s])
            L = int(lens[s])
            if kind == "keys_are_new_tokens":
                L = min(L, n)
            for i in range(n):
                row = s + i if kind == "rows_by_sequence" else int(cu[s]) + i
                if row >= total:
                    continue
                pos = i if kind == "offset_ignored" else L - n + i
                for h in range(H):
                    sc, vs = [], []
                    for t in range(L):
                        if causal:
                            hidden = t >= pos if kind == "off_by_one" else t > pos
                            if kind == "inverted":
                                hidden = t < pos
                            if hidden:
                                continue
                        kk = kc[table[s, t // P], h, t % P]
                        sc.append(scale * float(q[row, h] @ kk))
                        vs.append(vc[table[s, t // P], h, t % P])
                    if not sc:
                        continue
                    m = max(sc)
                    w = np.exp(np.array(sc) - m)
                    o[row, h] = (w[:, None] * np.array(vs)).sum(0) / w.sum()
                    lse[row, h] = m + math.log(w.sum())
        return o, lse
    return prefill


@pytest.mark.parametrize("kind", ["offset_ignored", "off_by_one", "keys_are_new_tokens",
                                  "rows_by_sequence", "inverted"])
def test_prefill_mutant_is_caught(kind):
    caught = []
    for pin in PINS:
        try:
            pin(_mutant(kind))
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"prefill mutant {kind} passed every pin"


def test_prefill_unmutated_copy_passes():
    for pin in PINS:
        pin(_mutant("none"))
