"""Paged prefill parity: fa_paged_prefill through the C ABI against the fp64 oracle."""
import math

import numpy as np
import pytest

import exact_attention_26_amd as fa
from exact_attention_26_amd import workloads as w
from gpu_util import LSE_ATOL, O_ATOL, assert_close, say, to_dev, to_host
from oracle import paged_prefill_fp64

pytestmark = pytest.mark.gpu


def _pools(wl, poison=True):
    kc = w.decode_pool(wl.layout, "k", poison=poison)
    vc = w.decode_pool(wl.layout, "v", poison=poison)
    return kc, vc


def _run(wl, q, kc, vc, causal, device, table=None, seq_lens=None, max_q_len=None, scale=None):
    import torch
    L = wl.layout
    scale = L.scale if scale is None else scale
    table = L.block_table if table is None else table
    seq_lens = L.seq_lens if seq_lens is None else seq_lens
    o, lse = fa.paged_prefill(to_dev(q, "bf16", device), to_dev(kc, "bf16", device),
                              to_dev(vc, "bf16", device),
                              torch.from_numpy(np.ascontiguousarray(table)).to(device),
                              torch.from_numpy(np.ascontiguousarray(seq_lens)).to(device),
                              torch.from_numpy(wl.cu_seqlens_q).to(device),
                              max_q_len or wl.max_q_len, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return to_host(o), to_host(lse)


def _check(tag, got, want):
    o, lse = got
    ro, rl = want
    assert_close(f"{tag} o", o, ro, O_ATOL["bf16"])
    assert_close(f"{tag} lse", lse, rl, LSE_ATOL["bf16"])


EDGE = [  # (cached tokens before the new ones, new tokens)
    (0, 1), (0, 16), (0, 17), (5, 1), (100, 28), (40, 64), (63, 65), (0, 129),
    (200, 200), (1000, 7), (3, 300), (16, 128),
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_edge_batches(gpu_device, d, causal):
    ctx = [c for c, _ in EDGE]
    new = [n for _, n in EDGE]
    wl = w.prefill_workload(601 + d, S=len(EDGE), H=3, d=d, ctx_lens=ctx, new_lens=new,
                            shared_prefix=32, spare=4)
    q = w.prefill_q(wl)
    kc, vc = _pools(wl)
    L = wl.layout
    say(f"prefill edges d={d} causal={causal} S={len(EDGE)}")
    got = _run(wl, q, kc, vc, causal, gpu_device)
    want = paged_prefill_fp64(q, kc, vc, L.block_table, L.seq_lens, wl.cu_seqlens_q,
                              causal=causal, scale=L.scale)
    _check(f"d={d} causal={causal}", got, want)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_short_and_empty_sequences(gpu_device, causal):
    # sequence 1 holds fewer cached tokens than new queries (its first queries
    # see nothing under the causal mask), sequence 2 holds none at all
    new = [40, 70, 5, 33]
    wl = w.prefill_workload(611, S=4, H=2, d=128, ctx_lens=[10, 0, 0, 0], new_lens=new, spare=4)
    wl.layout.seq_lens[:] = np.array([50, 30, 0, 33], dtype=np.int32)
    q = w.prefill_q(wl)
    kc, vc = _pools(wl)
    L = wl.layout
    say(f"prefill short/empty causal={causal}")
    got = _run(wl, q, kc, vc, causal, gpu_device)
    want = paged_prefill_fp64(q, kc, vc, L.block_table, L.seq_lens, wl.cu_seqlens_q,
                              causal=causal, scale=L.scale)
    assert np.isinf(want[1]).any()
    _check(f"short causal={causal}", got, want)


def test_prefill_negative_scale(gpu_device):
    wl = w.prefill_workload(615, S=3, H=2, d=128, ctx_lens=[0, 70, 300], new_lens=[45, 130, 9],
                            spare=4)
    q = w.prefill_q(wl)
    kc, vc = _pools(wl)
    L = wl.layout
    for causal in (True, False):
        say(f"prefill scale=-0.2 causal={causal}")
        got = _run(wl, q, kc, vc, causal, gpu_device, scale=-0.2)
        want = paged_prefill_fp64(q, kc, vc, L.block_table, L.seq_lens, wl.cu_seqlens_q,
                                  causal=causal, scale=-0.2)
        _check(f"negative scale causal={causal}", got, want)


def test_prefill_unresolvable_page_is_not_seen(gpu_device):
    # an out-of-range table entry hides its page; the same result as a
    # sequence without that page (the page lies before every new token)
    wl = w.prefill_workload(621, S=2, H=2, d=128, ctx_lens=[64, 40], new_lens=[20, 9], spare=4)
    q = w.prefill_q(wl)
    kc, vc = _pools(wl)
    L = wl.layout
    bad = L.block_table.copy()
    bad[0, 1] = L.num_blocks + 7                      # tokens 16..31 of sequence 0
    bad[1, 0] = -3                                    # tokens 0..15 of sequence 1
    ref_table = L.block_table.copy()
    ref_table[0, 1:-1] = L.block_table[0, 2:]
    ref_table[1, 0:-1] = L.block_table[1, 1:]
    ref_lens = L.seq_lens - 16
    for causal in (True, False):
        say(f"prefill unresolvable pages causal={causal}")
        got = _run(wl, q, kc, vc, causal, gpu_device, table=bad)
        want = paged_prefill_fp64(q, kc, vc, ref_table, ref_lens, wl.cu_seqlens_q,
                                  causal=causal, scale=L.scale)
        _check(f"bad pages causal={causal}", got, want)


def test_prefill_length_clamped_to_table(gpu_device):
    # seq_lens beyond max_blocks * 16 read only the table's pages
    wl = w.prefill_workload(631, S=2, H=2, d=64, ctx_lens=[30, 0], new_lens=[34, 48], spare=4)
    q = w.prefill_q(wl)
    kc, vc = _pools(wl)
    L = wl.layout
    big = L.seq_lens.copy()
    big[0] += 1000
    say("prefill clamped length")
    got = _run(wl, q, kc, vc, False, gpu_device, seq_lens=big)
    cap = np.minimum(big, L.max_blocks * L.page_size).astype(np.int32)
    want = paged_prefill_fp64(q, kc, vc, L.block_table, cap, wl.cu_seqlens_q, causal=False,
                              scale=L.scale)
    _check("clamped", got, want)


def test_prefill_full_size_sampled_rows(gpu_device):
    """The bench workload (16 sequences, about 16k new tokens, H=32, d=128),
    NaN-poisoned pools, in the bench's launch configuration; sampled rows."""
    wl = w.prefill_workload(**w.PREFILL_P1)
    q = w.prefill_q(wl)
    kc, vc = _pools(wl)
    L = wl.layout
    rng = np.random.default_rng(5)
    rows = []
    for s in range(L.S):
        lo, hi = int(wl.cu_seqlens_q[s]), int(wl.cu_seqlens_q[s + 1])
        fixed = [lo, lo + 1, lo + 127, lo + 128, hi - 1]
        rows += [r for r in fixed if lo <= r < hi] + list(rng.integers(lo, hi, 4))
    rows = np.unique(np.array(rows))
    for causal in (True, False):
        say(f"prefill full P1 causal={causal}")
        o, lse = _run(wl, q, kc, vc, causal, gpu_device)
        want = paged_prefill_fp64(q, kc, vc, L.block_table, L.seq_lens, wl.cu_seqlens_q,
                                  causal=causal, scale=L.scale, rows=rows)
        _check(f"P1 causal={causal}", (o[rows], lse[rows]), want)


def test_prefill_deterministic(gpu_device):
    """The same inputs give the same bits."""
    wl = w.prefill_workload(641, S=3, H=2, d=128, ctx_lens=[0, 0, 0], new_lens=[300, 129, 64],
                            spare=4)
    q = w.prefill_q(wl)
    kc, vc = _pools(wl, poison=False)
    say("prefill determinism")
    a = _run(wl, q, kc, vc, True, gpu_device)
    b = _run(wl, q, kc, vc, True, gpu_device)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_rows_past_total_q_keep_positions(gpu_device, causal):
    """Device data whose last sequence runs past total_q (cu_seqlens_q[S] >
    total_q): the rows inside are computed at their true positions (the new
    tokens are still the last n_s cached ones) and nothing past total_q is
    touched."""
    import torch
    new = [30, 150]
    wl = w.prefill_workload(621, S=2, H=2, d=128, ctx_lens=[20, 60], new_lens=new, spare=4)
    q = w.prefill_q(wl)
    kc, vc = _pools(wl)
    L = wl.layout
    total_q = 30 + 100                         # 50 of sequence 1's rows lie past the end
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(gpu_device)  # noqa: E731
    qd = to_dev(q, "bf16", gpu_device)
    o = torch.full((wl.total_q, L.H, L.d), 7.0, dtype=torch.bfloat16, device=gpu_device)
    lse = torch.full((wl.total_q, L.H), 7.0, dtype=torch.float32, device=gpu_device)
    say(f"prefill rows past total_q causal={causal}")
    fa.fa_paged_prefill(qd[:total_q], to_dev(kc, "bf16", gpu_device),
                        to_dev(vc, "bf16", gpu_device), t(L.block_table), t(L.seq_lens),
                        t(wl.cu_seqlens_q), o[:total_q], lse[:total_q], wl.max_q_len, causal,
                        L.scale)
    torch.cuda.synchronize()
    o, lse = to_host(o), to_host(lse)
    want = paged_prefill_fp64(q, kc, vc, L.block_table, L.seq_lens, wl.cu_seqlens_q,
                              causal=causal, scale=L.scale)
    _check("rows inside total_q", (o[:total_q], lse[:total_q]),
           (want[0][:total_q], want[1][:total_q]))
    assert np.all(o[total_q:] == 7.0) and np.all(lse[total_q:] == 7.0)
