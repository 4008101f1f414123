"""Backward parity: the HIP backward through the C ABI against the fp64 oracle.

Inputs q, k, v come from the forward workloads and dO from ``bwd_dout``; O and
LSE handed to the backward are the oracle's (O rounded to bf16, LSE to fp32),
except in the end-to-end tests, which feed the HIP forward's own outputs as a
training step does.  Tolerances: tests/bwd_bounds.py.
"""
import math

import numpy as np
import pytest

import exact_attention_26_amd as fa
from exact_attention_26_amd import workloads as w
from bwd_bounds import backward_bounds, check_within
from gpu_util import say, to_dev, to_host
from oracle import attention_backward_fp64, attention_fp64

pytestmark = pytest.mark.gpu


def _bwd(q, k, v, o, lse, do, causal, scale, device):
    """HIP backward; o and lse are host arrays (o already bf16-exact)."""
    import torch
    qd, kd, vd, od, dod = (to_dev(x, "bf16", device) for x in (q, k, v, o, do))
    ld = torch.from_numpy(np.ascontiguousarray(lse, dtype=np.float32)).to(device)
    dq, dk, dv = fa.attention_backward(qd, kd, vd, od, ld, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return to_host(dq), to_host(dk), to_host(dv)


def _check_all(tag, got, q, k, v, do, o_used, causal, scale):
    """Compare every head of got = (dq, dk, dv) with the oracle."""
    ref = attention_backward_fp64(q, k, v, do, causal=causal, scale=scale)
    B, H = q.shape[:2]
    worst = 0.0
    for b in range(B):
        for h in range(H):
            bounds = backward_bounds(q[b, h], k[b, h], v[b, h], do[b, h], o_used[b, h],
                                     causal=causal, scale=scale)
            for name, g, r, bd in zip(("dq", "dk", "dv"), got, ref, bounds):
                worst = max(worst, check_within(f"{tag} {name} b={b} h={h}", g[b, h], r[b, h], bd))
    return worst


def _case(B, H, n, d, seed, causal, scale, device, sigma_qk=1.0):
    q, k, v = w.fwd_inputs(B, H, n, d, seed=seed, sigma_qk=sigma_qk)
    do = w.bwd_dout(B, H, n, d, seed=seed)
    o, lse = attention_fp64(q, k, v, causal=causal, scale=scale)
    ob = w.round_to_bf16(o.astype(np.float32))
    got = _bwd(q, k, v, ob, lse.astype(np.float32), do, causal, scale, device)
    return _check_all(f"N={n} d={d} causal={causal}", got, q, k, v, do, ob, causal, scale)


EDGE_N = [1, 2, 17, 63, 64, 65, 127, 128, 129, 200, 255, 256, 257, 300]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_edge_lengths(gpu_device, d, causal):
    for n in EDGE_N:
        say(f"bwd bf16 B=1 H=2 N={n} d={d} causal={causal}")
        _case(1, 2, n, d, 300 + n, causal, 1.0 / math.sqrt(d), gpu_device)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_several_tiles(gpu_device, causal):
    # several 128-key blocks and 64-row tiles with a ragged tail, large logits
    say(f"bwd bf16 B=2 H=2 N=1000 d=128 causal={causal} sigma_qk=2")
    _case(2, 2, 1000, 128, 41, causal, 1.0 / math.sqrt(128), gpu_device, sigma_qk=2.0)


def test_bwd_scale_values(gpu_device):
    # zero scale (uniform attention, dQ = dK = 0), negative and large scales
    for scale in (0.0, -0.1, 0.3):
        for causal in (False, True):
            say(f"bwd bf16 N=200 d=64 scale={scale} causal={causal}")
            _case(1, 2, 200, 64, 51, causal, scale, gpu_device)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_after_hip_forward(gpu_device, causal):
    """A training step: the HIP forward's O and LSE feed the HIP backward."""
    import torch
    n, d = 777, 128
    scale = 1.0 / math.sqrt(d)
    q, k, v = w.fwd_inputs(2, 2, n, d, seed=61)
    do = w.bwd_dout(2, 2, n, d, seed=61)
    qd, kd, vd, dod = (to_dev(x, "bf16", gpu_device) for x in (q, k, v, do))
    say(f"bwd after fwd N={n} d={d} causal={causal}")
    o, lse = fa.attention(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa.attention_backward(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    _check_all("fwd+bwd", (to_host(dq), to_host(dk), to_host(dv)), q, k, v, do, to_host(o),
               causal, scale)


def test_bwd_deterministic(gpu_device):
    import torch
    n, d = 500, 128
    q, k, v = w.fwd_inputs(2, 3, n, d, seed=71)
    do = w.bwd_dout(2, 3, n, d, seed=71)
    qd, kd, vd, dod = (to_dev(x, "bf16", gpu_device) for x in (q, k, v, do))
    say("bwd determinism N=500 d=128 causal")
    o, lse = fa.attention(qd, kd, vd, causal=True)
    a = fa.attention_backward(qd, kd, vd, o, lse, dod, causal=True)
    b = fa.attention_backward(qd, kd, vd, o, lse, dod, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_workspace_contents_do_not_matter(gpu_device, d):
    """The row statistics are written by the backward itself (rows past N of
    the last 32-row block as zeros): a workspace full of NaN bytes gives the
    same bits as a zeroed one; N = 300 leaves 20 padded rows in the last block."""
    import torch
    B, H, n = 1, 3, 300
    q, k, v = w.fwd_inputs(B, H, n, d, seed=81)
    do = w.bwd_dout(B, H, n, d, seed=81)
    qd, kd, vd, dod = (to_dev(x, "bf16", gpu_device) for x in (q, k, v, do))
    nbytes = fa.fa_bwd_workspace_size(B, H, n, d)
    for causal in (False, True):
        say(f"bwd workspace poison N={n} d={d} causal={causal}")
        o, lse = fa.attention(qd, kd, vd, causal=causal)
        ws0 = torch.zeros(nbytes, dtype=torch.uint8, device=gpu_device)
        wsn = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=gpu_device)
        a = fa.attention_backward(qd, kd, vd, o, lse, dod, causal=causal, workspace=ws0)
        b = fa.attention_backward(qd, kd, vd, o, lse, dod, causal=causal, workspace=wsn)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y)
            assert torch.isfinite(x.float()).all()


def test_bwd_rejections(gpu_device):
    import torch
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16, device=gpu_device)
    lse = torch.zeros((1, 1, 64), dtype=torch.float32, device=gpu_device)
    with pytest.raises(fa.FaError) as e:                  # workspace too small
        fa.attention_backward(q, q, q, q, lse, q,
                              workspace=torch.empty(16, dtype=torch.uint8, device=gpu_device))
    assert e.value.status == 1
    qf = q.float()
    with pytest.raises(fa.FaError) as e:                  # fp32 backward: no kernel
        fa.attention_backward(qf, qf, qf, qf, lse, qf)
    assert e.value.status == 2
    q96 = torch.zeros((1, 1, 64, 96), dtype=torch.bfloat16, device=gpu_device)
    with pytest.raises(fa.FaError) as e:                  # d = 96: no kernel
        fa.attention_backward(q96, q96, q96, q96, lse, q96)
    assert e.value.status == 2


FULL = ["fwd_b8_h16_n2048_d128", "sweep_N512", "sweep_N4096", "sweep_N16384",
        "long_b1_h16_n16384_d128"]


@pytest.mark.parametrize("name", FULL)
def test_bwd_full_size_sampled_heads(gpu_device, name):
    """Full-size workloads, all heads on the GPU (forward then backward, the
    launch configuration the bench times); the oracle checks whole heads."""
    import torch
    cfg = w.FWD_CONFIGS[name]
    q, k, v = w.fwd_config_inputs(cfg)
    do = w.bwd_dout(cfg.B, cfg.H, cfg.N, cfg.d, seed=cfg.seed)
    qd, kd, vd, dod = (to_dev(x, cfg.dtype, gpu_device) for x in (q, k, v, do))
    rng = np.random.default_rng(cfg.seed + 1)
    heads = [(cfg.B - 1, cfg.H - 1), (int(rng.integers(cfg.B)), int(rng.integers(cfg.H)))]
    if cfg.N >= 16384:
        heads = heads[:1]
    for causal in cfg.causal:
        say(f"bwd full {name} causal={causal}")
        o, lse = fa.attention(qd, kd, vd, causal=causal, scale=cfg.scale)
        dq, dk, dv = fa.attention_backward(qd, kd, vd, o, lse, dod, causal=causal,
                                           scale=cfg.scale)
        torch.cuda.synchronize()
        for b, h in heads:
            args = (q[b, h], k[b, h], v[b, h], do[b, h])
            ref = attention_backward_fp64(*args, causal=causal, scale=cfg.scale, row_block=2048)
            bounds = backward_bounds(*args, to_host(o[b, h]), causal=causal, scale=cfg.scale)
            for nm, g, r, bd in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, bounds):
                check_within(f"{name} {nm} b={b} h={h}", to_host(g[b, h]), r, bd)
