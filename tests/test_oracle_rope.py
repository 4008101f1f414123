"""Pins for the RoPE oracle (rotary position embedding of queries and keys):

  * a hand-computed rotation (quarter and half turns of a single pair);
  * the complex-number form written with numpy's complex type, which is how
    the pages describe it ("LLM study notes", RoPE section);
  * each pair keeps its length; position 0 (cos 1, sin 0) is the identity;
  * relative position: <rope(q) at p, rope(k) at r> = <rope(q) at p - r, k>
    for tables built from angles linear in the position;
  * at the attention level: moving every position by the same amount leaves
    O and LSE unchanged, and all-zero angles give plain attention;
  * planted mistakes (angle sign flipped, halves instead of consecutive pairs,
    cosine and sine swapped, keys left unrotated) each fail a pin.
"""
import numpy as np
import pytest

from oracle import attention_fp64, attention_rope_fp64, rope_fp64


def _angles(n_pos, d, base=10000.0, shift=0):
    i = np.arange(d // 2)
    return (np.arange(n_pos)[:, None] + shift) * base ** (-2.0 * i[None, :] / d)


def _tables(ang):
    return np.cos(ang), np.sin(ang)


def pin_by_hand(rope):
    ang = np.array([[0.0], [np.pi / 2], [np.pi]])
    c, s = _tables(ang)
    x = np.array([[1.0, 2.0], [1.0, 0.0], [1.0, 2.0]])
    out = rope(x, c, s)
    np.testing.assert_allclose(out, [[1.0, 2.0], [0.0, 1.0], [-1.0, -2.0]], rtol=0, atol=1e-15)


def pin_complex_form(rope):
    rng = np.random.default_rng(81)
    x = rng.standard_normal((3, 11, 16))
    ang = _angles(11, 16)
    out = rope(x, *_tables(ang))
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * ang)
    np.testing.assert_allclose(out[..., 0::2], z.real, rtol=0, atol=1e-13)
    np.testing.assert_allclose(out[..., 1::2], z.imag, rtol=0, atol=1e-13)


def pin_norms_and_identity(rope):
    rng = np.random.default_rng(82)
    x = rng.standard_normal((7, 8))
    out = rope(x, *_tables(_angles(7, 8)))
    np.testing.assert_allclose(np.hypot(out[:, 0::2], out[:, 1::2]),
                               np.hypot(x[:, 0::2], x[:, 1::2]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(out[0], x[0], rtol=0, atol=0)


def pin_relative_position(rope):
    rng = np.random.default_rng(83)
    d, n = 16, 40
    c, s = _tables(_angles(n, d))
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for p, r in ((7, 3), (39, 0), (20, 19), (12, 12)):
        rq = rope(np.tile(q, (n, 1)), c, s)[p]
        rk = rope(np.tile(k, (n, 1)), c, s)[r]
        rel = rope(np.tile(q, (n, 1)), c, s)[p - r]
        np.testing.assert_allclose(rq @ rk, rel @ k, rtol=0, atol=1e-12)


def pin_attention_shift(rope):
    rng = np.random.default_rng(84)
    q, k, v = (rng.standard_normal((2, 30, 16)) for _ in range(3))
    for causal in (False, True):
        def attn(tables):
            c, s = tables
            return attention_fp64(rope(q, c, s), rope(k, c, s), v, causal=causal, scale=0.3)
        o1, l1 = attn(_tables(_angles(30, 16)))
        o2, l2 = attn(_tables(_angles(30, 16, shift=1000)))
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-11)
        np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-11)
        o0, l0 = attn(_tables(np.zeros((30, 8))))
        r0, rl0 = attention_fp64(q, k, v, causal=causal, scale=0.3)
        np.testing.assert_allclose(o0, r0, rtol=0, atol=1e-14)


PINS = [pin_by_hand, pin_complex_form, pin_norms_and_identity, pin_relative_position,
        pin_attention_shift]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_rope_oracle_passes_pin(pin):
    pin(rope_fp64)


def test_attention_rope_is_attention_of_rotated_inputs():
    rng = np.random.default_rng(85)
    q, k, v = (rng.standard_normal((2, 20, 8)) for _ in range(3))
    c, s = _tables(_angles(20, 8))
    o, lse = attention_rope_fp64(q, k, v, c, s, causal=True, scale=0.5)
    ro, rl = attention_fp64(rope_fp64(q, c, s), rope_fp64(k, c, s), v, causal=True, scale=0.5)
    np.testing.assert_array_equal(o, ro)
    np.testing.assert_array_equal(lse, rl)


def _mutant(kind):
    def rope(x, cos, sin):
        x = np.asarray(x, dtype=np.float64)
        n = x.shape[-2]
        c, s = np.asarray(cos)[:n], np.asarray(sin)[:n]
        if kind == "sign":
            s = -s
        if kind == "swapped":
            c, s = s, c
        if kind == "halves":
            h = x.shape[-1] // 2
            re, im = x[..., :h], x[..., h:]
            return np.concatenate([re * c - im * s, re * s + im * c], axis=-1)
        re, im = x[..., 0::2], x[..., 1::2]
        out = np.empty_like(x)
        out[..., 0::2] = re * c - im * s
        out[..., 1::2] = re * s + im * c
        return out
    return rope


@pytest.mark.parametrize("kind", ["sign", "swapped", "halves"])
def test_rope_mutant_is_caught(kind):
    caught = []
    for pin in PINS:
        try:
            pin(_mutant(kind))
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"rope mutant {kind} passed every pin"


def test_keys_left_unrotated_is_caught():
    # rotating only the queries breaks the relative-position property
    rng = np.random.default_rng(86)
    q, k, v = (rng.standard_normal((1, 25, 16)) for _ in range(3))
    outs = []
    for shift in (0, 1000):
        c, s = _tables(_angles(25, 16, shift=shift))
        outs.append(attention_fp64(rope_fp64(q, c, s), k, v, scale=0.3)[0])
    assert not np.allclose(outs[0], outs[1], rtol=0, atol=1e-6)


def test_rope_unmutated_copy_passes():
    for pin in PINS:
        pin(_mutant("none"))
