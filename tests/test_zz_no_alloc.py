"""The allocation-free paged decode (fa_paged_decode_noalloc) against the
decode with a caller-provided workspace (fa_paged_decode), through the C ABI.

Both run the same kernels, so their outputs must agree bit for bit; the
oracle checks both to the decode's tolerances as well.  Two calls in a row,
the second smaller than the first, show that the scratch array's leftover
contents from one call do not leak into the next.
"""
import numpy as np
import pytest

import exact_attention_26_amd as fa
from exact_attention_26_amd import workloads as w
from gpu_util import LSE_ATOL, O_ATOL, assert_close, say, to_dev, to_host
from oracle import paged_decode_fp64

pytestmark = pytest.mark.gpu


def _case(seed, lens, d, H):
    L = w.decode_layout(seed, S=len(lens), H=H, d=d, lens=lens, shared_prefix=64, spare=3,
                        len_range=(1, max(lens)))
    q = w.decode_q(L)
    kc = w.decode_pool(L, "k", poison=True)
    vc = w.decode_pool(L, "v", poison=True)
    return L, q, kc, vc


def _both(L, q, kc, vc, device):
    import torch
    qd, kd, vd = (to_dev(x, "bf16", device) for x in (q, kc, vc))
    bt = torch.from_numpy(L.block_table).to(device)
    sl = torch.from_numpy(L.seq_lens).to(device)
    ws = torch.empty(fa.fa_paged_decode_workspace_size(L.S, L.H, L.d, L.page_size, L.max_blocks),
                     dtype=torch.uint8, device=device)
    o_ws, o_na = torch.empty_like(qd), torch.full_like(qd, float("nan"))
    l_ws = torch.empty((L.S, L.H), dtype=torch.float32, device=device)
    l_na = torch.full_like(l_ws, float("nan"))
    fa.fa_paged_decode(qd, kd, vd, bt, sl, o_ws, l_ws, L.scale, ws)
    fa.fa_paged_decode_noalloc(qd, kd, vd, bt, sl, o_na, l_na, L.scale)
    torch.cuda.synchronize()
    return (to_host(o_ws), to_host(l_ws)), (to_host(o_na), to_host(l_na))


def _check(tag, L, q, kc, vc, with_ws, no_alloc):
    assert np.array_equal(with_ws[0], no_alloc[0]), f"{tag}: o differs from fa_paged_decode"
    assert np.array_equal(with_ws[1], no_alloc[1]), f"{tag}: lse differs from fa_paged_decode"
    ro, rl = paged_decode_fp64(q, kc, vc, L.block_table, L.seq_lens, scale=L.scale)
    assert_close(f"{tag} o", no_alloc[0], ro, O_ATOL["bf16"])
    assert_close(f"{tag} lse", no_alloc[1], rl, LSE_ATOL["bf16"])


def test_noalloc_matches_workspace_decode_twice(gpu_device):
    # first call: 40 sequences of up to 6000 tokens (up to 12 splits each), H=8, d=128
    rng = np.random.default_rng(91)
    lens = [int(x) for x in rng.integers(1, 6001, 40)] + [0, 1, 16, 513]
    L1, q1, k1, v1 = _case(91, lens, d=128, H=8)
    say(f"noalloc call 1: S={L1.S} H={L1.H} d=128 max_len={max(lens)}")
    a1, b1 = _both(L1, q1, k1, v1, gpu_device)
    _check("call 1", L1, q1, k1, v1, a1, b1)
    # second call, smaller: 3 sequences of up to 700 tokens, H=2, d=64; the
    # scratch array still holds the first call's partials
    L2, q2, k2, v2 = _case(92, [700, 33, 250], d=64, H=2)
    say(f"noalloc call 2: S={L2.S} H={L2.H} d=64")
    a2, b2 = _both(L2, q2, k2, v2, gpu_device)
    _check("call 2", L2, q2, k2, v2, a2, b2)


def test_noalloc_refuses_what_does_not_fit(gpu_device):
    import torch
    # 64 sequences x 32 heads with 16384-token tables (32 splits each) need
    # 34 MB of partials, more than the 32 MiB scratch array: nothing runs
    q = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device=gpu_device)
    pool = torch.zeros((4, 32, 16, 128), dtype=torch.bfloat16, device=gpu_device)
    bt = torch.zeros((64, 1024), dtype=torch.int32, device=gpu_device)
    sl = torch.ones(64, dtype=torch.int32, device=gpu_device)
    o = torch.zeros_like(q)
    say("noalloc refuses 34 MB of partials")
    with pytest.raises(fa.FaError) as e:
        fa.fa_paged_decode_noalloc(q, pool, pool, bt, sl, o, None, 0.1)
    assert e.value.status == fa.FA_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert not o.any()
