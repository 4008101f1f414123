"""Forward parity: the HIP kernel through the C ABI against the fp64 oracle."""
import math

import numpy as np
import pytest

import exact_attention_26_amd as fa
from exact_attention_26_amd import workloads as w
from gpu_util import LSE_ATOL, O_ATOL, assert_close, sample_rows, say, to_dev, to_host
from oracle import attention_fp64

pytestmark = pytest.mark.gpu


def _run(q, k, v, dtype, causal, scale, device):
    import torch
    qd, kd, vd = (to_dev(x, dtype, device) for x in (q, k, v))
    o, lse = fa.attention(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return to_host(o), to_host(lse)


def test_smoke_config_fp32(gpu_device):
    cfg = w.FWD_CONFIGS["smoke"]
    q, k, v = w.fwd_config_inputs(cfg)
    say("fwd smoke fp32 B=1 H=2 N=256 d=64")
    o, lse = _run(q, k, v, "f32", False, cfg.scale, gpu_device)
    ro, rl = attention_fp64(q, k, v, causal=False, scale=cfg.scale)
    assert_close("o", o, ro, O_ATOL["f32"])
    assert_close("lse", lse, rl, LSE_ATOL["f32"])


EDGE_N = [1, 2, 15, 16, 17, 31, 33, 63, 64, 65, 100, 127, 128, 129, 255, 256, 257, 300, 513]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_lengths_bf16(gpu_device, d, causal):
    for n in EDGE_N:
        q, k, v = w.fwd_inputs(2, 3, n, d, seed=100 + n)
        say(f"fwd bf16 B=2 H=3 N={n} d={d} causal={causal}")
        o, lse = _run(q, k, v, "bf16", causal, 1.0 / math.sqrt(d), gpu_device)
        ro, rl = attention_fp64(q, k, v, causal=causal, scale=1.0 / math.sqrt(d))
        assert_close(f"o N={n}", o, ro, O_ATOL["bf16"])
        assert_close(f"lse N={n}", lse, rl, LSE_ATOL["bf16"])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_lengths_fp32(gpu_device, d, causal):
    for n in (1, 17, 64, 129, 300):
        q, k, v = w.fwd_inputs(1, 2, n, d, seed=200 + n, dtype="f32")
        say(f"fwd f32 B=1 H=2 N={n} d={d} causal={causal}")
        o, lse = _run(q, k, v, "f32", causal, 1.0 / math.sqrt(d), gpu_device)
        ro, rl = attention_fp64(q, k, v, causal=causal, scale=1.0 / math.sqrt(d))
        assert_close(f"o N={n}", o, ro, O_ATOL["f32"])
        assert_close(f"lse N={n}", lse, rl, LSE_ATOL["f32"])


@pytest.mark.parametrize("causal", [False, True])
def test_several_tiles_full_compare(gpu_device, causal):
    # spans several 128-row blocks and 64-key tiles with a ragged tail
    q, k, v = w.fwd_inputs(2, 4, 1000, 128, seed=31, sigma_qk=2.0)
    say(f"fwd bf16 B=2 H=4 N=1000 d=128 causal={causal} sigma_qk=2")
    o, lse = _run(q, k, v, "bf16", causal, 1 / math.sqrt(128), gpu_device)
    ro, rl = attention_fp64(q, k, v, causal=causal, scale=1 / math.sqrt(128))
    assert_close("o", o, ro, O_ATOL["bf16"])
    assert_close("lse", lse, rl, LSE_ATOL["bf16"])


def test_scale_is_applied(gpu_device):
    q, k, v = w.fwd_inputs(1, 2, 200, 64, seed=41)
    for scale in (0.0, 0.05, 0.3):
        say(f"fwd bf16 scale={scale}")
        o, lse = _run(q, k, v, "bf16", False, scale, gpu_device)
        ro, rl = attention_fp64(q, k, v, causal=False, scale=scale)
        assert_close("o", o, ro, O_ATOL["bf16"])
        assert_close("lse", lse, rl, LSE_ATOL["bf16"])


@pytest.mark.parametrize("d", [64, 128])
def test_negative_scale(gpu_device, d):
    # softmax(scale * s) with scale < 0 favours the smallest scores; the sign
    # has to reach the scores, not only the exponent's factor
    q, k, v = w.fwd_inputs(1, 2, 333, d, seed=43 + d)
    for dtype in ("bf16", "f32"):
        for causal in (False, True):
            say(f"fwd {dtype} d={d} N=333 scale=-0.2 causal={causal}")
            o, lse = _run(q, k, v, dtype, causal, -0.2, gpu_device)
            ro, rl = attention_fp64(q, k, v, causal=causal, scale=-0.2)
            assert_close(f"o {dtype} causal={causal}", o, ro, O_ATOL[dtype])
            assert_close(f"lse {dtype} causal={causal}", lse, rl, LSE_ATOL[dtype])


def test_huge_logit_shift(gpu_device):
    # a common offset of about +-100 on every score of a row: exp() overflows
    # (or underflows to an all-zero row) unless the running maximum is subtracted
    q, k, v = w.fwd_inputs(1, 1, 300, 64, seed=51)
    k = k.copy()
    k[..., 0] += 24.0
    k = w.round_to_bf16(k)                   # both sides see the same bf16 keys
    q = q.copy()
    q[..., 0] = np.where(q[..., 0] >= 0, 4.0, -4.0)
    for causal in (False, True):
        say(f"fwd bf16 shifted keys causal={causal}")
        o, lse = _run(q, k, v, "bf16", causal, 1.0, gpu_device)
        ro, rl = attention_fp64(q, k, v, causal=causal, scale=1.0)
        assert np.abs(rl).max() > 88.0       # beyond the range of exp in fp32
        assert_close("o", o, ro, O_ATOL["bf16"])
        assert_close("lse", lse, rl, LSE_ATOL["bf16"])


FULL = ["fwd_b8_h16_n2048_d128"] + [f"sweep_N{n}" for n in (512, 1024, 2048, 4096, 8192, 16384)] \
    + ["long_b1_h16_n16384_d128"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_rows(gpu_device, name):
    """Full-size configs in the bench's launch configuration; oracle on sampled rows."""
    import torch
    cfg = w.FWD_CONFIGS[name]
    q, k, v = w.fwd_config_inputs(cfg)
    qd, kd, vd = (to_dev(x, cfg.dtype, gpu_device) for x in (q, k, v))
    rng = np.random.default_rng(cfg.seed)
    heads = [(0, 0), (cfg.B - 1, cfg.H - 1), (int(rng.integers(cfg.B)), int(rng.integers(cfg.H)))]
    for causal in cfg.causal:
        say(f"fwd full {name} causal={causal}")
        o, lse = fa.attention(qd, kd, vd, causal=causal, scale=cfg.scale)
        torch.cuda.synchronize()
        for b, h in heads:
            rows = sample_rows(cfg.N, rng)
            ro, rl = attention_fp64(q[b, h], k[b, h], v[b, h], causal=causal, scale=cfg.scale,
                                    rows=rows)
            assert_close(f"o b={b} h={h}", to_host(o[b, h, rows]), ro, O_ATOL[cfg.dtype])
            assert_close(f"lse b={b} h={h}", to_host(lse[b, h, rows]), rl, LSE_ATOL[cfg.dtype])
        del o, lse


def test_grid_beyond_65535_work_groups(gpu_device):
    """B=1 H=2048 N=8192 d=128: 65 536 work groups in both launch
    configurations (2048 heads x 32 blocks of 256 rows; 2048 heads x 32 causal
    pairs of 128-row blocks), so the 1-D grid and its XCD remap run past the
    16-bit range.  Inputs are drawn on the device (seeded, N(0,1)); the oracle
    gets the sampled heads' rows."""
    import torch
    B, H, N, d = 1, 2048, 8192, 128
    gen = torch.Generator(device=gpu_device)
    gen.manual_seed(2048)
    qd, kd, vd = (torch.randn((B, H, N, d), device=gpu_device, generator=gen,
                              dtype=torch.float32).to(torch.bfloat16) for _ in range(3))
    rng = np.random.default_rng(2048)
    heads = [0, 1, 1023, 2046, 2047, int(rng.integers(H))]
    host = {h: tuple(t[0, h].float().cpu().numpy().astype(np.float64) for t in (qd, kd, vd))
            for h in heads}
    for causal in (False, True):
        say(f"fwd grid B={B} H={H} N={N} d={d} causal={causal}")
        o, lse = fa.attention(qd, kd, vd, causal=causal)
        torch.cuda.synchronize()
        for h in heads:
            rows = sample_rows(N, rng)
            q, k, v = host[h]
            ro, rl = attention_fp64(q, k, v, causal=causal, scale=1 / math.sqrt(d), rows=rows)
            assert_close(f"o h={h}", to_host(o[0, h, rows]), ro, O_ATOL["bf16"])
            assert_close(f"lse h={h}", to_host(lse[0, h, rows]), rl, LSE_ATOL["bf16"])
        del o, lse
    del qd, kd, vd
    torch.cuda.empty_cache()


@pytest.mark.parametrize("causal", [False, True])
def test_long_sequence_sampled_rows(gpu_device, causal):
    """N = 32768 keys (512 key tiles; 128 blocks of 256 rows without the mask,
    256 blocks of 128 paired into 128 work groups with it), a ragged N too;
    oracle on sampled rows."""
    import torch
    for n in (32768, 32768 - 77):
        q, k, v = w.fwd_inputs(1, 2, n, 128, seed=81 + n)
        qd, kd, vd = (to_dev(x, "bf16", gpu_device) for x in (q, k, v))
        say(f"fwd long B=1 H=2 N={n} d=128 causal={causal}")
        o, lse = fa.attention(qd, kd, vd, causal=causal)
        torch.cuda.synchronize()
        rng = np.random.default_rng(n)
        for h in range(2):
            rows = sample_rows(n, rng, extra=24)
            ro, rl = attention_fp64(q[0, h], k[0, h], v[0, h], causal=causal,
                                    scale=1 / math.sqrt(128), rows=rows)
            assert_close(f"o N={n} h={h}", to_host(o[0, h, rows]), ro, O_ATOL["bf16"])
            assert_close(f"lse N={n} h={h}", to_host(lse[0, h, rows]), rl, LSE_ATOL["bf16"])
        del o, lse, qd, kd, vd


@pytest.mark.parametrize("shape", [(12, 16, 704), (3, 100, 1024), (2, 8, 1088), (3, 100, 1000),
                                   (64, 16, 200)])
@pytest.mark.parametrize("scale_sign", [1.0, -1.0])
@pytest.mark.parametrize("causal", [False, True])
def test_many_blocks_per_work_group(gpu_device, shape, scale_sign, causal):
    """The persistent d=128 grid (N a multiple of 64, at least eleven key
    tiles).  Non-causal: 576 blocks of 256 rows for N = 704 (2.25 blocks per
    work group, every third block with rows past N), 1200 full blocks for
    N = 1024, and 80 blocks for N = 1088 (fewer blocks than compute units,
    the last block of a head holding 64 rows).  Causal: units of a long and a
    short block of one head, and a lone middle block when a head has an odd
    number of blocks (N = 704: blocks 2+0 and 1, of 11+4 and 8 key tiles;
    N = 1088: 4+0, 3+1 and 2, the long block of the first unit holding 64
    rows).  A ragged N = 1000 and a short N = 200 run on the per-block grid.
    Sampled heads against the oracle, both signs of the scale (a negative
    one flips the query operand at each block start)."""
    B, H, N = shape
    d = 128
    q, k, v = w.fwd_inputs(B, H, N, d, seed=900 + N)
    scale = scale_sign / math.sqrt(d)
    say(f"fwd many blocks B={B} H={H} N={N} d={d} causal={causal} scale={scale:+.4f}")
    o, lse = _run(q, k, v, "bf16", causal, scale, gpu_device)
    rng = np.random.default_rng(N)
    heads = [(0, 0), (0, H - 1), (B // 2, H // 2), (B - 1, H - 1),
             (int(rng.integers(B)), int(rng.integers(H)))]
    for b, h in heads:
        rows = sample_rows(N, rng, extra=24)
        ro, rl = attention_fp64(q[b, h], k[b, h], v[b, h], causal=causal, scale=scale, rows=rows)
        assert_close(f"o b={b} h={h}", o[b, h, rows], ro, O_ATOL["bf16"])
        assert_close(f"lse b={b} h={h}", lse[b, h, rows], rl, LSE_ATOL["bf16"])


def test_deterministic(gpu_device):
    import torch
    q, k, v = w.fwd_inputs(2, 4, 777, 128, seed=61)
    qd, kd, vd = (to_dev(x, "bf16", gpu_device) for x in (q, k, v))
    for causal in (False, True):
        say(f"fwd determinism causal={causal}")
        o1, l1 = fa.attention(qd, kd, vd, causal=causal)
        o2, l2 = fa.attention(qd, kd, vd, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_lse_none_and_errors(gpu_device):
    import torch
    q, k, v = w.fwd_inputs(1, 2, 70, 64, seed=71)
    qd, kd, vd = (to_dev(x, "bf16", gpu_device) for x in (q, k, v))
    o = torch.empty_like(qd)
    say("fwd lse=None")
    fa.fa_fwd(qd, kd, vd, o, None, False, 0.125)
    torch.cuda.synchronize()
    ro, _ = attention_fp64(q, k, v, scale=0.125)
    assert_close("o", to_host(o), ro, O_ATOL["bf16"])
    q96 = torch.zeros((1, 1, 8, 96), dtype=torch.bfloat16, device=gpu_device)
    with pytest.raises(fa.FaError) as ei:
        fa.attention(q96, q96, q96)
    assert ei.value.status == 2
