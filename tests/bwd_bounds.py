"""Element-wise error bounds for the bf16 attention backward (test tolerance model).

The kernel rounds the probabilities P and the score gradients dS to bf16
before they enter the matrix products (relative error at most 2^-9 each), it
takes delta_i = dO_i . O_i from the bf16 output O (whose own rounding is again
up to 2^-9 of |O|), accumulates in fp32 and rounds the result to bf16.  Each
of these errors is a small multiple of 2^-9 of the same sums taken over
absolute values:

    |dV_j err| <~ 2^-9 * sum_i P_ij |dO_i|
    |dQ_i err| <~ 2^-9 * |scale| * sum_j A_ij |K_j|
    |dK_j err| <~ 2^-9 * |scale| * sum_i A_ij |Q_i|
    with A_ij = P_ij (|dP_ij| + |delta_i| + sum_d |dO_id| |O_id|)

(three such terms for dQ and dK: the dS rounding, the delta error and the
output rounding).  The tests accept |kernel - oracle| <= 2^-6 times these sums
(a factor of about 2.7 over the three terms) plus 1e-6.  A sum over absolute
values, not the result itself, is the right scale: dK and dQ are sums of terms
of both signs and may cancel to nearly zero while the rounding errors of the
terms do not.
"""
import math

import numpy as np

REL = 2.0 ** -6
ABS = 1e-6


def backward_bounds(q, k, v, do, o, *, causal: bool, scale: float, row_block: int = 1024):
    """Bounds ``(bq, bk, bv)`` for one head: q, k, v, do, o are ``[N][d]``."""
    q, k, v, do, o = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do, o))
    n = q.shape[0]
    bq = np.empty_like(q)
    bk = np.zeros_like(k)
    bv = np.zeros_like(v)
    keys = np.arange(n)
    adelta = np.sum(np.abs(do) * np.abs(o), axis=1)
    for r0 in range(0, n, row_block):
        rows = np.arange(r0, min(n, r0 + row_block))
        s = scale * (q[rows] @ k.T)
        if causal:
            s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        dp = do[rows] @ v.T
        delta = np.sum(p * dp, axis=1, keepdims=True)
        a = p * (np.abs(dp) + np.abs(delta) + adelta[rows, None])
        bv += p.T @ np.abs(do[rows])
        bq[rows] = abs(scale) * (a @ np.abs(k))
        bk += abs(scale) * (a.T @ np.abs(q[rows]))
    return REL * bq + ABS, REL * bk + ABS, REL * bv + ABS


def check_within(name, got, want, bound):
    """Assert |got - want| <= bound element-wise; returns the worst ratio."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    assert not np.isnan(got).any(), f"{name}: NaN in GPU result"
    ratio = np.abs(got - want) / bound
    worst = float(ratio.max()) if ratio.size else 0.0
    if worst > 1.0:
        idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(f"{name}: error {abs(got[idx] - want[idx]):.3e} at {idx} exceeds "
                             f"bound {bound[idx]:.3e} (ratio {worst:.2f}); max-abs error "
                             f"{np.abs(got - want).max():.3e}")
    return worst
