"""Pins for the backward oracle (gradients of exact attention).

What pins it, other than itself:
  * PyTorch autograd through scaled_dot_product_attention, CPU, float64;
  * central finite differences of the (separately pinned) forward oracle on
    tiny inputs, every coordinate;
  * closed forms: dO = 0 gives zero gradients; with all-equal scores (Q = 0) dV
    is the average of dO over the queries that see each key; N = 1 gives
    dQ = dK = 0 and dV = dO; the row-shift invariance of the forward makes the
    gradient of every key sum to zero along any direction the shift test uses:
    sum_j dK_j = 0 for non-causal attention (adding w to all keys changes nothing);
  * planted mistakes (dropped scale, missing the softmax-Jacobian row term,
    transposed P in dV, causal mask ignored) each fail at least one pin.
"""
import math

import numpy as np
import pytest

from oracle import attention_backward_fp64, attention_fp64


def pin_torch_autograd(bwd):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(31)
    q, k, v, do = (rng.standard_normal((2, 3, 19, 8)) for _ in range(4))
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, do, causal=causal, scale=0.3)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                               scale=0.3)
        out.backward(torch.from_numpy(do))
        np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)


def pin_finite_differences(bwd):
    rng = np.random.default_rng(32)
    n, d, scale = 5, 3, 0.7
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    eps = 1e-6
    for causal in (False, True):
        grads = bwd(q, k, v, do, causal=causal, scale=scale)

        def loss(qq, kk, vv):
            o, _ = attention_fp64(qq, kk, vv, causal=causal, scale=scale)
            return float(np.sum(o * do))
        for which, g in enumerate(grads):
            num = np.zeros((n, d))
            for i in range(n):
                for j in range(d):
                    args = [q.copy(), k.copy(), v.copy()]
                    args[which][i, j] += eps
                    up = loss(*args)
                    args[which][i, j] -= 2 * eps
                    num[i, j] = (up - loss(*args)) / (2 * eps)
            np.testing.assert_allclose(g, num, rtol=0, atol=1e-7)


def pin_closed_forms(bwd):
    rng = np.random.default_rng(33)
    n, d = 9, 4
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    zero = np.zeros((n, d))
    for causal in (False, True):
        for g in bwd(q, k, v, zero, causal=causal, scale=0.5):
            np.testing.assert_allclose(g, 0.0, rtol=0, atol=1e-15)
    do = rng.standard_normal((n, d))
    # Q = 0: every visible score is equal, P_ij = 1/#visible(i)
    _, _, dv = bwd(np.zeros((n, d)), k, v, do, causal=False, scale=0.5)
    np.testing.assert_allclose(dv, np.tile(do.mean(axis=0), (n, 1)), rtol=0, atol=1e-13)
    _, _, dv = bwd(np.zeros((n, d)), k, v, do, causal=True, scale=0.5)
    w = do / np.arange(1, n + 1)[:, None]                 # query i spreads 1/(i+1) over keys 0..i
    expect = np.cumsum(w[::-1], axis=0)[::-1]             # key j gets sum over i >= j
    np.testing.assert_allclose(dv, expect, rtol=0, atol=1e-13)
    # N = 1: O = V, so dQ = dK = 0 and dV = dO
    dq, dk, dv = bwd(q[:1], k[:1], v[:1], do[:1], causal=False, scale=0.5)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)
    np.testing.assert_allclose(dv, do[:1], atol=1e-15)
    # adding one vector to every key leaves O unchanged (non-causal): sum_j dK_j = 0
    _, dk, _ = bwd(q, k, v, do, causal=False, scale=0.5)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)


BWD_PINS = [pin_torch_autograd, pin_finite_differences, pin_closed_forms]


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda p: p.__name__)
def test_backward_oracle_passes_pin(pin):
    pin(attention_backward_fp64)


def _mutant(kind):
    def bwd(q, k, v, do, *, causal=False, scale=None):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        n, d = q.shape[-2], q.shape[-1]
        if scale is None:
            scale = 1.0 / math.sqrt(d)
        s = scale * (q @ np.swapaxes(k, -1, -2))
        if causal and kind != "no_causal":
            s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, s)
        p = np.exp(s - s.max(axis=-1, keepdims=True))
        p /= p.sum(axis=-1, keepdims=True)
        pt = np.swapaxes(p, -1, -2)
        dv = (p if kind == "dv_untransposed" else pt) @ do
        dp = do @ np.swapaxes(v, -1, -2)
        row = 0.0 if kind == "no_row_term" else (p * dp).sum(axis=-1, keepdims=True)
        ds = p * (dp - row)
        sc = 1.0 if kind == "no_scale" else scale
        return sc * (ds @ k), sc * (np.swapaxes(ds, -1, -2) @ q), dv
    return bwd


@pytest.mark.parametrize("kind", ["no_scale", "no_row_term", "dv_untransposed", "no_causal"])
def test_backward_mutant_is_caught(kind):
    caught = []
    for pin in BWD_PINS:
        try:
            pin(_mutant(kind))
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"backward mutant {kind} passed every pin"


def test_backward_unmutated_copy_passes():
    for pin in BWD_PINS:
        pin(_mutant("none"))


def test_backward_row_blocks_bound_memory_only():
    # the row-blocked form (used at N = 16384) is the same gradient: every
    # pin above, and agreement with the unblocked form on ragged blocks
    for pin in BWD_PINS:
        pin(lambda *a, **kw: attention_backward_fp64(*a, row_block=4, **kw))
    rng = np.random.default_rng(34)
    q, k, v, do = (rng.standard_normal((2, 37, 8)) for _ in range(4))
    for causal in (False, True):
        full = attention_backward_fp64(q, k, v, do, causal=causal, scale=0.4)
        for rb in (1, 5, 16, 36):
            part = attention_backward_fp64(q, k, v, do, causal=causal, scale=0.4, row_block=rb)
            for a, b in zip(full, part):
                np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)
