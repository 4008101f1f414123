"""RoPE parity: fa_rope and fa_fwd_rope through the C ABI against the fp64 oracle.

Tolerances.  fa_rope computes each rotated pair in fp32 from exact bf16 inputs
and fp32 tables and rounds it to bf16: per element at most half a bf16 ulp of
the result (2^-9 relative) plus fp32 rounding of the two products
(2^-20 of their magnitudes, generously).  The fused forward feeds bf16 rotated
queries and keys to the matrix unit, so it is compared (a) with the oracle on
those bf16-rounded rotated rows at the forward's usual tolerances, and (b) with
the oracle on exact rotations at the forward's tolerances widened by the
largest score change the operand rounding can cause in the row,
delta_i = 2^-8 * |scale| * max_j sum_d |q_id| |k_jd| (LSE moves by at most
delta_i, each probability by a factor within 1 +- 2 delta_i).
"""
import math

import numpy as np
import pytest

import exact_attention_26_amd as fa
from exact_attention_26_amd import workloads as w
from gpu_util import LSE_ATOL, O_ATOL, assert_close, say, to_dev, to_host
from oracle import attention_fp64, attention_rope_fp64, rope_fp64

pytestmark = pytest.mark.gpu


def _tables(N, d, device, base=10000.0):
    import torch
    c, s = w.rope_tables(N, d, base)
    return c, s, torch.from_numpy(c).to(device), torch.from_numpy(s).to(device)


def test_rope_elementwise(gpu_device):
    import torch
    for (B, H, N, d) in ((1, 2, 1, 64), (2, 3, 300, 128), (1, 1, 4096, 64)):
        x = w.fwd_inputs(B, H, N, d, seed=900 + N)[0]
        c, s, cd, sd = _tables(N, d, gpu_device)
        say(f"rope elementwise B={B} H={H} N={N} d={d}")
        xd = to_dev(x, "bf16", gpu_device)
        got = to_host(fa.rope(xd, cd, sd))
        ref = rope_fp64(x, c, s)
        re, im = x[..., 0::2].astype(np.float64), x[..., 1::2].astype(np.float64)
        mag = np.abs(re) * np.abs(c) + np.abs(im) * np.abs(s) + np.abs(re) * np.abs(s) \
            + np.abs(im) * np.abs(c)
        bound = np.empty_like(ref)
        bound[..., 0::2] = mag
        bound[..., 1::2] = mag
        bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -20 * bound + 1e-30
        err = np.abs(got - ref)
        assert (err <= bound).all(), float((err / bound).max())
        # in place gives the same bits
        fa.fa_rope(xd, xd, cd, sd)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(xd), got)


def _row_delta(qr, kr, scale, causal):
    """2^-8 |scale| max_j sum_d |q_id||k_jd| per row (visible keys only)."""
    a = np.abs(qr) @ np.swapaxes(np.abs(kr), -1, -2)
    if causal:
        n = a.shape[-1]
        a = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], 0.0, a)
    return 2.0 ** -8 * abs(scale) * a.max(axis=-1)


def _check_fused(tag, q, k, v, c, s, causal, scale, o, lse, rows=None):
    qr, kr = rope_fp64(q, c, s), rope_fp64(k, c, s)
    qb = w.round_to_bf16(qr.astype(np.float32)).astype(np.float64)
    kb = w.round_to_bf16(kr.astype(np.float32)).astype(np.float64)
    # (a) the bf16 operands the matrix unit sees
    ro, rl = attention_fp64(qb, kb, v, causal=causal, scale=scale, rows=rows)
    assert_close(f"{tag} o (bf16 operands)", o, ro, O_ATOL["bf16"])
    assert_close(f"{tag} lse (bf16 operands)", lse, rl, LSE_ATOL["bf16"])
    # (b) exact rotations, tolerance widened by the operand rounding
    eo, el = attention_rope_fp64(q, k, v, c, s, causal=causal, scale=scale, rows=rows)
    delta = _row_delta(qr if rows is None else qr[..., rows, :], kr, scale, causal
                       if rows is None else False)
    vmax = np.abs(v).max(axis=-2, keepdims=True)[..., 0, :].max(axis=-1)
    tol_o = O_ATOL["bf16"] + 2.0 * delta[..., None] * vmax[..., None, None]
    tol_l = LSE_ATOL["bf16"] + delta
    assert (np.abs(o - eo) <= tol_o).all(), f"{tag}: o off the exact rotation"
    assert (np.abs(lse - el) <= tol_l).all(), f"{tag}: lse off the exact rotation"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_rope_edges(gpu_device, d, causal):
    for n in (1, 17, 64, 129, 300):
        q, k, v = w.fwd_inputs(2, 2, n, d, seed=910 + n)
        c, s, cd, sd = _tables(n, d, gpu_device)
        say(f"fwd_rope N={n} d={d} causal={causal}")
        o, lse = fa.attention_rope(*(to_dev(x, "bf16", gpu_device) for x in (q, k, v)), cd, sd,
                                   causal=causal, scale=1 / math.sqrt(d))
        _check_fused(f"N={n}", q, k, v, c, s, causal, 1 / math.sqrt(d), to_host(o), to_host(lse))


def test_fwd_rope_negative_scale(gpu_device):
    n, d = 300, 128
    q, k, v = w.fwd_inputs(1, 2, n, d, seed=931)
    c, s, cd, sd = _tables(n, d, gpu_device)
    for causal in (False, True):
        say(f"fwd_rope N={n} d={d} scale=-0.2 causal={causal}")
        o, lse = fa.attention_rope(*(to_dev(x, "bf16", gpu_device) for x in (q, k, v)), cd, sd,
                                   causal=causal, scale=-0.2)
        _check_fused(f"scale=-0.2 causal={causal}", q, k, v, c, s, causal, -0.2, to_host(o),
                     to_host(lse))


def test_fwd_rope_stream_edges(gpu_device):
    """d = 128, N a multiple of 64 from 704 up (the persistent stream): N not
    a multiple of the 256-row block (rows past N in the last block of every
    head), a negative scale, several blocks per work group; against the
    oracle and bitwise against fa_rope(q), fa_rope(k), fa_fwd."""
    import torch
    d = 128
    for (B, H, n, scale) in ((1, 3, 960, -0.2), (2, 2, 1088, 1 / math.sqrt(d))):
        q, k, v = w.fwd_inputs(B, H, n, d, seed=977 + n)
        c, s, cd, sd = _tables(n, d, gpu_device)
        qd, kd, vd = (to_dev(x, "bf16", gpu_device) for x in (q, k, v))
        rows = np.array([0, 1, 255, 256, 511, 700, n - 65, n - 64, n - 2, n - 1])
        for causal in (False, True):
            say(f"fwd_rope stream B={B} H={H} N={n} scale={scale:.3f} causal={causal}")
            o, lse = fa.attention_rope(qd, kd, vd, cd, sd, causal=causal, scale=scale)
            uo, ul = fa.attention(fa.rope(qd, cd, sd), fa.rope(kd, cd, sd), vd, causal=causal,
                                  scale=scale)
            torch.cuda.synchronize()
            assert torch.equal(o, uo) and torch.equal(lse, ul)
            for b, h in ((0, 0), (B - 1, H - 1)):
                _check_fused(f"N={n} b={b} h={h} causal={causal}", q[b, h], k[b, h], v[b, h],
                             c, s, causal, scale, to_host(o[b, h, rows]),
                             to_host(lse[b, h, rows]), rows=rows)


def test_fwd_rope_full_size_and_matches_unfused(gpu_device):
    """The forward bench workload (B=8 H=16 N=2048 d=128) with RoPE: sampled
    rows against the oracle; and the fused call gives the same bits as
    fa_rope(q), fa_rope(k) and fa_fwd one after the other."""
    import torch
    cfg = w.FWD_CONFIGS["fwd_b8_h16_n2048_d128"]
    q, k, v = w.fwd_config_inputs(cfg)
    c, s, cd, sd = _tables(cfg.N, cfg.d, gpu_device)
    qd, kd, vd = (to_dev(x, "bf16", gpu_device) for x in (q, k, v))
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 1000, 2046, 2047],
                                     rng.choice(cfg.N, 30, replace=False)]))
    for causal in (False, True):
        say(f"fwd_rope full causal={causal}")
        o, lse = fa.attention_rope(qd, kd, vd, cd, sd, causal=causal, scale=cfg.scale)
        uo, ul = fa.attention(fa.rope(qd, cd, sd), fa.rope(kd, cd, sd), vd, causal=causal,
                              scale=cfg.scale)
        torch.cuda.synchronize()
        assert torch.equal(o, uo) and torch.equal(lse, ul)
        for b, h in ((0, 0), (cfg.B - 1, cfg.H - 1)):
            _check_fused(f"b={b} h={h} causal={causal}", q[b, h], k[b, h], v[b, h], c, s, causal,
                         cfg.scale, to_host(o[b, h, rows]), to_host(lse[b, h, rows]), rows=rows)


def test_fwd_rope_rejections(gpu_device):
    import torch
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16, device=gpu_device)
    c = torch.zeros((64, 32), dtype=torch.float32, device=gpu_device)
    small = torch.empty(8, dtype=torch.uint8, device=gpu_device)
    o = torch.empty_like(q)
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_rope(q, q, q, o, None, c, c, False, 0.125, small)
    assert e.value.status == 1
    qf = q.float()
    with pytest.raises(fa.FaError) as e:
        fa.attention_rope(qf, qf, qf, c, c)
    assert e.value.status == 2
