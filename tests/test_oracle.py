"""Pins for the CPU oracle: it is checked against things other than itself.

Each pin is a function of an attention callable ``attn(q, k, v, causal=, scale=)
-> (o, lse)`` (or of a paged-decode callable), so the same pins run on

  * the oracle itself -- every pin must pass, and
  * deliberately broken copies of it ("mutants": dropped scale, transposed
    scores, causal off by one, no max subtraction, log base 2, no
    normalisation, wrong value rows; for paging: no table indirection, wrong
    slot order, reading past the sequence end, wrong head) -- every mutant must
    fail at least one pin.

What pins the oracle:
  * hand-derived closed-form fixtures in tests/golden/ (exact rationals and
    logarithms),
  * a scalar brute-force loop (pure Python floats, softmax exactly as defined,
    no max subtraction) on N <= 16,
  * closed forms: constant V, all-zero Q (mean of V, LSE = ln of the number of
    visible keys), causal row 0, N = 1,
  * invariants: rows of the softmax sum to one, a common shift of every key
    (huge logits) leaves O unchanged and shifts LSE exactly, key/value
    permutation invariance and query permutation equivariance,
  * PyTorch's own scaled_dot_product_attention on the CPU in float64,
  * the blockwise online-softmax recurrence of the pages' pseudocode
    ("Flash Attention", velog @myungum, section 2), written independently
    here, reaching the same result for several block shapes (including ragged
    ones),
  * paging: identity table == dense, shuffled table == identity table, shared
    prefix pages == copied pages, decode == last row of causal attention.
"""
import math

import numpy as np
import pytest

import golden_values as gv
from oracle import attention_bruteforce, attention_fp64, paged_decode_fp64

RNG = np.random.default_rng(12345)


# ---------------------------------------------------------------------------
# dense pins
# ---------------------------------------------------------------------------
def pin_golden(attn):
    for name in gv.names("sdpa_"):
        fx = gv.load(name)
        q, k, v = gv.array(fx["q"]), gv.array(fx["k"]), gv.array(fx["v"])
        scale = gv.value(fx["scale"])
        for mode, causal in (("noncausal", False), ("causal", True)):
            o, lse = attn(q, k, v, causal=causal, scale=scale)
            exp = fx["expected"][mode]
            np.testing.assert_allclose(o, gv.array(exp["o"]), rtol=0, atol=1e-12,
                                       err_msg=f"{name} {mode} o")
            np.testing.assert_allclose(lse, gv.array(exp["lse"]), rtol=0, atol=1e-12,
                                       err_msg=f"{name} {mode} lse")


def pin_bruteforce(attn):
    rng = np.random.default_rng(7)
    for n, d in ((1, 1), (2, 3), (5, 4), (9, 8), (16, 5), (13, 16)):
        q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
        for causal in (False, True):
            scale = 1.0 / math.sqrt(d)
            o, lse = attn(q, k, v, causal=causal, scale=scale)
            ob, lb = attention_bruteforce(q.tolist(), k.tolist(), v.tolist(),
                                          causal=causal, scale=scale)
            np.testing.assert_allclose(o, np.array(ob), rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, np.array(lb), rtol=0, atol=1e-12)


def pin_constant_v(attn):
    rng = np.random.default_rng(8)
    q, k = rng.standard_normal((2, 3, 37, 16)), rng.standard_normal((2, 3, 37, 16))
    v = np.full((2, 3, 37, 16), 0.5)
    for causal in (False, True):
        o, _ = attn(q, k, v, causal=causal, scale=0.25)
        np.testing.assert_allclose(o, 0.5, rtol=0, atol=1e-14)


def pin_zero_q(attn):
    rng = np.random.default_rng(9)
    n, d = 29, 8
    q = np.zeros((n, d))
    k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    o, lse = attn(q, k, v, causal=False, scale=0.3)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (n, 1)), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, math.log(n), rtol=0, atol=1e-13)
    o, lse = attn(q, k, v, causal=True, scale=0.3)
    prefix_mean = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(o, prefix_mean, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, np.log(np.arange(1, n + 1)), rtol=0, atol=1e-13)


def pin_causal_row0_and_n1(attn):
    rng = np.random.default_rng(10)
    q, k, v = (rng.standard_normal((11, 6)) for _ in range(3))
    o, lse = attn(q, k, v, causal=True, scale=0.7)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-14)
    assert abs(lse[0] - 0.7 * math.fsum(q[0] * k[0])) < 1e-13
    o, lse = attn(q[:1], k[:1], v[:1], causal=False, scale=0.7)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-14)


def pin_rows_sum_to_one(attn):
    rng = np.random.default_rng(11)
    n, d, scale = 23, 7, 0.4
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    for causal in (False, True):
        _, lse = attn(q, k, v, causal=causal, scale=scale)
        for i in range(n):
            seen = range(i + 1) if causal else range(n)
            total = math.fsum(math.exp(scale * math.fsum(q[i] * k[j]) - lse[i]) for j in seen)
            assert abs(total - 1.0) < 1e-12


def pin_shift_invariance(attn):
    # adding the same vector w to every key adds scale*q_i.w to row i of S:
    # softmax is unchanged, LSE moves by exactly that.  |shift| ~ 1e3 would
    # overflow exp() unless the row maximum is subtracted first.
    rng = np.random.default_rng(12)
    n, d, scale = 17, 8, 0.5
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    q[:, 0] = np.sign(q[:, 0]) * (1.0 + np.abs(q[:, 0]))
    w = np.zeros(d)
    w[0] = 1500.0
    for causal in (False, True):
        o0, l0 = attn(q, k, v, causal=causal, scale=scale)
        o1, l1 = attn(q, k + w, v, causal=causal, scale=scale)
        np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-9)
        np.testing.assert_allclose(l1 - l0, scale * (q @ w), rtol=1e-12, atol=1e-9)


def pin_permutations(attn):
    rng = np.random.default_rng(13)
    n, d = 19, 6
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    perm = rng.permutation(n)
    o, lse = attn(q, k, v, causal=False, scale=0.3)
    o2, l2 = attn(q, k[perm], v[perm], causal=False, scale=0.3)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, lse, rtol=0, atol=1e-13)
    o3, l3 = attn(q[perm], k, v, causal=False, scale=0.3)
    np.testing.assert_allclose(o3, o[perm], rtol=0, atol=1e-13)
    np.testing.assert_allclose(l3, lse[perm], rtol=0, atol=1e-13)


def pin_torch_sdpa(attn):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(14)
    q, k, v = (rng.standard_normal((2, 3, 33, 16)) for _ in range(3))
    for causal in (False, True):
        o, _ = attn(q, k, v, causal=causal, scale=0.2)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            is_causal=causal, scale=0.2).numpy()
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def _blockwise(q, k, v, br, bc, causal, scale):
    """Online softmax over key blocks, as the pages' pseudocode describes it:
    per (query block, key block) a block row max and row sum, merged into the
    running (m, l, O) by rescaling both sides to the new maximum."""
    n, d = q.shape
    o = np.zeros((n, v.shape[1]))
    l = np.zeros(n)
    m = np.full(n, -np.inf)
    for j0 in range(0, n, bc):
        kj, vj = k[j0:j0 + bc], v[j0:j0 + bc]
        for i0 in range(0, n, br):
            s = scale * (q[i0:i0 + br] @ kj.T)
            if causal:
                qi = np.arange(i0, min(n, i0 + br))[:, None]
                kk = np.arange(j0, min(n, j0 + bc))[None, :]
                s = np.where(kk > qi, -np.inf, s)
            mt = s.max(axis=1)
            live = np.isfinite(mt)                        # rows with a visible key here
            pt = np.where(live[:, None], np.exp(s - np.where(live, mt, 0.0)[:, None]), 0.0)
            lt = pt.sum(axis=1)
            mi = m[i0:i0 + br]
            mn = np.maximum(mi, mt)
            a_old = np.where(np.isfinite(mi), np.exp(mi - mn), 0.0)
            a_new = np.where(live, np.exp(mt - np.where(live, mn, 0.0)), 0.0)
            ln = a_old * l[i0:i0 + br] + a_new * lt
            o[i0:i0 + br] = (l[i0:i0 + br, None] * a_old[:, None] * o[i0:i0 + br]
                             + a_new[:, None] * (pt @ vj)) / ln[:, None]
            l[i0:i0 + br], m[i0:i0 + br] = ln, mn
    return o, m + np.log(l)


def pin_blockwise_recurrence(attn):
    rng = np.random.default_rng(15)
    n, d = 45, 8
    q, k, v = (rng.standard_normal((n, d)) * 2 for _ in range(3))
    for br, bc in ((1, 1), (4, 7), (16, 16), (45, 8), (64, 64)):
        for causal in (False, True):
            ob, lb = _blockwise(q, k, v, br, bc, causal, 0.35)
            o, lse = attn(q, k, v, causal=causal, scale=0.35)
            np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-12)


DENSE_PINS = [pin_golden, pin_bruteforce, pin_constant_v, pin_zero_q, pin_causal_row0_and_n1,
              pin_rows_sum_to_one, pin_shift_invariance, pin_permutations, pin_torch_sdpa,
              pin_blockwise_recurrence]


@pytest.mark.parametrize("pin", DENSE_PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(pin):
    pin(attention_fp64)


def test_rows_argument_selects_rows():
    q, k, v = (RNG.standard_normal((2, 70, 8)) for _ in range(3))
    rows = np.array([69, 0, 33, 34, 5])
    for causal in (False, True):
        o, lse = attention_fp64(q, k, v, causal=causal, scale=0.3)
        os_, ls = attention_fp64(q, k, v, causal=causal, scale=0.3, rows=rows, row_block=2)
        # same arithmetic; BLAS may block a 2-row product differently (rounding order only)
        np.testing.assert_allclose(os_, o[:, rows], rtol=0, atol=1e-14)
        np.testing.assert_allclose(ls, lse[:, rows], rtol=0, atol=1e-14)


def test_default_scale_is_inverse_sqrt_d():
    q, k, v = (RNG.standard_normal((9, 16)) for _ in range(3))
    o1, l1 = attention_fp64(q, k, v)
    o2, l2 = attention_fp64(q, k, v, scale=0.25)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# ---------------------------------------------------------------------------
# mutants: plausible mistakes planted in a copy of the definition
# ---------------------------------------------------------------------------
def _mutant(kind):
    def attn(q, k, v, *, causal=False, scale=None):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        d = q.shape[-1]
        if scale is None:
            scale = 1.0 / math.sqrt(d)
        if kind == "no_scale":
            scale = 1.0
        s = scale * (q @ np.swapaxes(k, -1, -2))
        if kind == "transposed_scores":
            s = np.swapaxes(s, -1, -2)
        n = s.shape[-1]
        i = np.arange(s.shape[-2])[:, None]
        j = np.arange(n)[None, :]
        if causal:
            hidden = (j >= i) if kind == "causal_strict" else (j > i)
            if kind == "causal_inverted":
                hidden = j < i
            s = np.where(hidden, -np.inf, s)
        m = s.max(axis=-1, keepdims=True)
        if kind == "no_max_shift":
            m = np.zeros_like(m)
        with np.errstate(all="ignore"):
            p = np.exp(s - m)
            l = p.sum(axis=-1, keepdims=True)
            vv = v[..., ::-1, :] if kind == "reversed_values" else v
            o = p @ vv
            if kind != "no_normalise":
                o = o / l
            lse = m + (np.log2(l) if kind == "lse_log2" else np.log(l))
            if kind == "lse_without_max":
                lse = np.log(l)
        return o, lse[..., 0]
    attn.__name__ = kind
    return attn


DENSE_MUTANTS = ["no_scale", "transposed_scores", "causal_strict", "causal_inverted",
                 "no_max_shift", "no_normalise", "reversed_values", "lse_log2", "lse_without_max"]


def _fails_some_pin(fn, pins):
    failed = []
    for pin in pins:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except (AssertionError, ValueError, FloatingPointError, OverflowError):
            failed.append(pin.__name__)
    return failed


def test_unmutated_copy_passes_every_pin():
    # the mutant factory with no mutation must pass, or the mutant test proves nothing
    assert _fails_some_pin(_mutant("none"), DENSE_PINS) == []


@pytest.mark.parametrize("kind", DENSE_MUTANTS)
def test_dense_mutant_is_caught(kind):
    assert _fails_some_pin(_mutant(kind), DENSE_PINS), f"mutant {kind} passed every pin"


# ---------------------------------------------------------------------------
# paged pins
# ---------------------------------------------------------------------------
def _golden_paged():
    fx = gv.load("paged_page4.json")
    return (gv.array(fx["q"]), gv.array(fx["k_cache"]), gv.array(fx["v_cache"]),
            np.array(fx["block_table"], dtype=np.int32), np.array(fx["seq_lens"], dtype=np.int32),
            gv.value(fx["scale"]), gv.array(fx["expected"]["o"]), gv.array(fx["expected"]["lse"]))


def ppin_golden(decode):
    q, kc, vc, bt, sl, scale, eo, el = _golden_paged()
    o, lse = decode(q, kc, vc, bt, sl, scale=scale)
    np.testing.assert_allclose(o, eo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, el, rtol=0, atol=1e-12)


def _paged_from_dense(k, v, page_size, table):
    """Scatter dense K/V ``[S][H][Lmax][d]`` into pages following ``table``;
    unused slots are NaN."""
    S, H, Lmax, d = k.shape
    nb = int(table.max()) + 1
    kc = np.full((nb, H, page_size, d), np.nan)
    vc = np.full((nb, H, page_size, d), np.nan)
    for s in range(S):
        for p in range(-(-Lmax // page_size)):
            t0 = p * page_size
            take = min(page_size, Lmax - t0)
            kc[table[s, p], :, :take] = k[s, :, t0:t0 + take]
            vc[table[s, p], :, :take] = v[s, :, t0:t0 + take]
    return kc, vc


def ppin_identity_and_shuffled_tables(decode):
    rng = np.random.default_rng(21)
    S, H, d, P = 3, 2, 8, 4
    lens = np.array([9, 4, 12], dtype=np.int32)
    Lmax = 12
    q = rng.standard_normal((S, H, d))
    k = rng.standard_normal((S, H, Lmax, d))
    v = rng.standard_normal((S, H, Lmax, d))
    pages = Lmax // P
    ident = np.arange(S * pages, dtype=np.int32).reshape(S, pages)
    shuf = rng.permutation(S * pages).astype(np.int32).reshape(S, pages)
    ref_o = np.zeros((S, H, d))
    ref_l = np.zeros((S, H))
    for s in range(S):
        L = lens[s]
        o1, l1 = attention_fp64(q[s][:, None, :], k[s, :, :L], v[s, :, :L], scale=0.3)
        ref_o[s], ref_l[s] = o1[:, 0], l1[:, 0]
    for table in (ident, shuf):
        kc, vc = _paged_from_dense(k, v, P, table)
        # poison what no sequence may read: tails past each length
        for s in range(S):
            L = lens[s]
            for t in range(L, Lmax):
                kc[table[s, t // P], :, t % P] = np.nan
                vc[table[s, t // P], :, t % P] = np.nan
        o, lse = decode(q, kc, vc, table, lens, scale=0.3)
        np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-12)


def ppin_shared_prefix_equals_copies(decode):
    rng = np.random.default_rng(22)
    H, d, P = 2, 4, 4
    q = rng.standard_normal((2, H, d))
    kc = rng.standard_normal((7, H, P, d))
    vc = rng.standard_normal((7, H, P, d))
    shared = np.array([[0, 1, 2], [0, 1, 3]], dtype=np.int32)       # pages 0,1 shared
    kc2 = np.concatenate([kc, kc[0:2]], axis=0)                       # copies at 7, 8
    vc2 = np.concatenate([vc, vc[0:2]], axis=0)
    copied = np.array([[0, 1, 2], [7, 8, 3]], dtype=np.int32)
    lens = np.array([11, 10], dtype=np.int32)
    o1, l1 = decode(q, kc, vc, shared, lens, scale=0.5)
    o2, l2 = decode(q, kc2, vc2, copied, lens, scale=0.5)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-14)


def ppin_decode_is_last_causal_row(decode):
    rng = np.random.default_rng(23)
    H, d, P, L = 3, 8, 4, 14
    q = rng.standard_normal((1, H, L, d))
    k = rng.standard_normal((1, H, L, d))
    v = rng.standard_normal((1, H, L, d))
    o_dense, l_dense = attention_fp64(q[0], k[0], v[0], causal=True, scale=0.3)
    table = rng.permutation(4).astype(np.int32)[None, :]
    kc, vc = _paged_from_dense(k, v, P, table)
    o, lse = decode(q[:, :, L - 1, :], kc, vc, table, np.array([L], np.int32), scale=0.3)
    np.testing.assert_allclose(o[0], o_dense[:, L - 1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0], l_dense[:, L - 1], rtol=0, atol=1e-12)


PAGED_PINS = [ppin_golden, ppin_identity_and_shuffled_tables, ppin_shared_prefix_equals_copies,
              ppin_decode_is_last_causal_row]


@pytest.mark.parametrize("pin", PAGED_PINS, ids=lambda p: p.__name__)
def test_paged_oracle_passes_pin(pin):
    pin(paged_decode_fp64)


def test_paged_pairs_argument():
    q, kc, vc, bt, sl, scale, eo, el = _golden_paged()
    o, lse = paged_decode_fp64(q, kc, vc, bt, sl, scale=scale, pairs=[(3, 0), (0, 0)])
    np.testing.assert_allclose(o, eo[[3, 0], 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, el[[3, 0], 0], rtol=0, atol=1e-12)


def _paged_mutant(kind):
    def decode(q, kc, vc, table, lens, *, scale=None):
        S, H, d = q.shape
        P = kc.shape[2]
        o = np.zeros((S, H, d))
        lse = np.full((S, H), -np.inf)
        for s in range(S):
            L = int(lens[s])
            if L <= 0:
                continue
            npg = -(-L // P)
            for h in range(H):
                ks, vs = [], []
                for p in range(npg):
                    blk = p if kind == "no_indirection" else int(table[s][p])
                    hh = 0 if kind == "head_zero" else h
                    take = P if kind == "read_whole_last_page" else min(P, L - p * P)
                    kk, vv = kc[blk, hh, :take], vc[blk, hh, :take]
                    if kind == "reversed_slots":           # token t read from slot P-1-t
                        kk, vv = kc[blk, hh, ::-1][:take], vc[blk, hh, ::-1][:take]
                    if kind == "k_slots_reversed":         # keys and values out of step
                        kk = kc[blk, hh, ::-1][P - take:]
                    ks.append(kk)
                    vs.append(vv)
                oo, ll = attention_fp64(q[s, h][None], np.concatenate(ks), np.concatenate(vs),
                                        scale=scale)
                o[s, h], lse[s, h] = oo[0], ll[0]
        return o, lse
    return decode


@pytest.mark.parametrize("kind", ["no_indirection", "head_zero", "read_whole_last_page",
                                  "reversed_slots", "k_slots_reversed"])
def test_paged_mutant_is_caught(kind):
    assert _fails_some_pin(_paged_mutant(kind), PAGED_PINS), f"paged mutant {kind} passed"


def test_paged_unmutated_copy_passes():
    assert _fails_some_pin(_paged_mutant("none"), PAGED_PINS) == []


def test_paged_rejects_table_overflow():
    q, kc, vc, bt, sl, scale, _, _ = _golden_paged()
    with pytest.raises(ValueError):
        paged_decode_fp64(q, kc, vc, bt, np.array([13, 4, 0, 5], np.int32), scale=scale)
