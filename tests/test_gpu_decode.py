"""Paged-KV decode parity: the HIP kernels through the C ABI against the fp64 oracle.

Every slot no sequence may read (tails past a sequence's length, spare pages,
the page unused table entries point to) holds NaN, so any stray read shows up
as NaN in the output.
"""
import math

import numpy as np
import pytest

import exact_attention_26_amd as fa
from exact_attention_26_amd import workloads as w
from gpu_util import LSE_ATOL, O_ATOL, assert_close, say, to_dev, to_host
from oracle import attention_fp64, paged_decode_fp64

pytestmark = pytest.mark.gpu


def _upload(layout, q, kc, vc, device):
    import torch
    return (to_dev(q, "bf16", device), to_dev(kc, "bf16", device), to_dev(vc, "bf16", device),
            torch.from_numpy(layout.block_table).to(device),
            torch.from_numpy(layout.seq_lens).to(device))


def _decode(layout, q, kc, vc, device, seq_lens=None, table=None, scale=None):
    import torch
    qd, kd, vd, bt, sl = _upload(layout, q, kc, vc, device)
    if seq_lens is not None:
        sl = torch.from_numpy(np.asarray(seq_lens, np.int32)).to(device)
    if table is not None:
        bt = torch.from_numpy(np.asarray(table, np.int32)).to(device)
    o, lse = fa.paged_decode(qd, kd, vd, bt, sl, scale=layout.scale if scale is None else scale)
    torch.cuda.synchronize()
    return to_host(o), to_host(lse)


def _small_layout(seed, lens, d=128, H=4, shared_prefix=48, max_blocks=None):
    L = w.decode_layout(seed, S=len(lens), H=H, d=d, lens=lens, shared_prefix=shared_prefix,
                        spare=3, max_blocks=max_blocks, len_range=(1, max(lens + [1])))
    q = w.decode_q(L)
    kc = w.decode_pool(L, "k", poison=True)
    vc = w.decode_pool(L, "v", poison=True)
    return L, q, kc, vc


@pytest.mark.parametrize("d", [64, 128])
def test_edge_lengths(gpu_device, d):
    lens = [1, 15, 16, 17, 31, 32, 33, 511, 512, 513, 600, 1025, 2, 100]
    L, q, kc, vc = _small_layout(81, lens, d=d)
    say(f"decode d={d} lens={lens}")
    o, lse = _decode(L, q, kc, vc, gpu_device)
    ro, rl = paged_decode_fp64(q, kc, vc, L.block_table, L.seq_lens, scale=L.scale)
    assert_close("o", o, ro, O_ATOL["bf16"])
    assert_close("lse", lse, rl, LSE_ATOL["bf16"])


@pytest.mark.parametrize("d", [64, 128])
def test_negative_and_zero_scale(gpu_device, d):
    lens = [1, 17, 300, 1025]
    L, q, kc, vc = _small_layout(83, lens, d=d, H=2)
    for scale in (-0.2, 0.0):
        say(f"decode d={d} scale={scale}")
        o, lse = _decode(L, q, kc, vc, gpu_device, scale=scale)
        ro, rl = paged_decode_fp64(q, kc, vc, L.block_table, L.seq_lens, scale=scale)
        assert_close(f"o scale={scale}", o, ro, O_ATOL["bf16"])
        assert_close(f"lse scale={scale}", lse, rl, LSE_ATOL["bf16"])


def test_long_sequence_many_chunks(gpu_device):
    """A 40 000-token sequence (2500 pages: 79 chunks of 32 pages in the
    grid's second dimension) beside very short ones, sharing a prefix with its
    neighbour; NaN-poisoned pools, every head against the oracle."""
    lens = [40000, 3, 16, 1, 40000 - 17, 511]
    L, q, kc, vc = _small_layout(84, lens, d=128, H=3, shared_prefix=1000)
    say(f"decode long sequences lens={lens} max_blocks={L.max_blocks}")
    o, lse = _decode(L, q, kc, vc, gpu_device)
    ro, rl = paged_decode_fp64(q, kc, vc, L.block_table, L.seq_lens, scale=L.scale)
    assert_close("o", o, ro, O_ATOL["bf16"])
    assert_close("lse", lse, rl, LSE_ATOL["bf16"])


def test_empty_and_clamped_and_bad_pages(gpu_device):
    lens = [0, 40, 64, 20]
    L, q, kc, vc = _small_layout(82, lens, H=2, shared_prefix=0, max_blocks=4)
    # seq 3 claims more tokens than its table can hold: clamped to 4 pages
    seq_lens = np.array([0, 40, 64, 10_000], np.int32)
    table = L.block_table.copy()
    table[3, :] = table[2, :]                   # 4 valid pages (those of seq 2)
    # seq 1: its last page (tokens 32..39) points outside the pool -> skipped
    table[1, 2] = L.num_blocks + 7
    say("decode empty / clamped / out-of-range page")
    o, lse = _decode(L, q, kc, vc, gpu_device, seq_lens=seq_lens, table=table)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))
    ro, rl = paged_decode_fp64(q, kc, vc, table, np.array([0, 32, 64, 64], np.int32),
                               scale=L.scale)
    assert_close("o", o[1:], ro[1:], O_ATOL["bf16"])
    assert_close("lse", lse[1:], rl[1:], LSE_ATOL["bf16"])


def test_decode_equals_last_causal_row(gpu_device):
    """Cross-path: decode over a paged copy == last row of the causal forward."""
    import torch
    n, H, d = 700, 4, 128
    q, k, v = w.fwd_inputs(1, H, n, d, seed=83)
    P = 16
    pages = -(-n // P)
    perm = np.random.default_rng(83).permutation(pages + 2).astype(np.int32)
    kc = np.full((pages + 2, H, P, d), np.nan, np.float32)
    vc = np.full((pages + 2, H, P, d), np.nan, np.float32)
    for p in range(pages):
        t0, t1 = p * P, min(n, p * P + P)
        kc[perm[p], :, : t1 - t0] = k[0, :, t0:t1]
        vc[perm[p], :, : t1 - t0] = v[0, :, t0:t1]
    say("decode vs causal forward last row")
    qd, kd, vd = (to_dev(x, "bf16", gpu_device) for x in (q, k, v))
    of, lf = fa.attention(qd, kd, vd, causal=True)
    od, ld = fa.paged_decode(qd[:, :, n - 1, :].contiguous(), to_dev(kc, "bf16", gpu_device),
                             to_dev(vc, "bf16", gpu_device),
                             torch.from_numpy(perm[None, :pages].copy()).to(gpu_device),
                             torch.tensor([n], dtype=torch.int32, device=gpu_device))
    torch.cuda.synchronize()
    assert_close("o", to_host(od)[0], to_host(of)[0, :, n - 1], O_ATOL["bf16"])
    assert_close("lse", to_host(ld)[0], to_host(lf)[0, :, n - 1], LSE_ATOL["bf16"])
    ro, rl = attention_fp64(q[0, :, n - 1:n], k[0], v[0], scale=1 / math.sqrt(d))
    assert_close("o vs oracle", to_host(od)[0], ro[:, 0], O_ATOL["bf16"])


def test_full_c4_sampled(gpu_device):
    """The full paged-decode workload (64 sequences, 128..8192 tokens, shared
    512-token prefixes, shuffled pool), NaN-poisoned; oracle on sampled pairs."""
    import torch
    L = w.decode_layout(**w.DECODE_C4)
    q = w.decode_q(L)
    say("decode full C4: generating pools")
    kc = w.decode_pool(L, "k", poison=True)
    vc = w.decode_pool(L, "v", poison=True)
    say("decode full C4: running")
    o, lse = _decode(L, q, kc, vc, gpu_device)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    rng = np.random.default_rng(4)
    order = np.argsort(L.seq_lens)
    seqs = sorted(set([int(order[0]), int(order[-1]), 0, 1, 2, 3]
                      + rng.choice(L.S, 10, replace=False).tolist()))
    pairs = [(s, int(h)) for s in seqs for h in rng.choice(L.H, 3, replace=False)]
    ro, rl = paged_decode_fp64(q, kc, vc, L.block_table, L.seq_lens, scale=L.scale, pairs=pairs)
    idx_s = [p[0] for p in pairs]
    idx_h = [p[1] for p in pairs]
    assert_close("o", o[idx_s, idx_h], ro, O_ATOL["bf16"])
    assert_close("lse", lse[idx_s, idx_h], rl, LSE_ATOL["bf16"])
    del kc, vc
    torch.cuda.empty_cache()


def test_deterministic(gpu_device):
    import torch
    lens = [900, 33, 4000, 17]
    L, q, kc, vc = _small_layout(84, lens)
    qd, kd, vd, bt, sl = _upload(L, q, kc, vc, gpu_device)
    say("decode determinism")
    o1, l1 = fa.paged_decode(qd, kd, vd, bt, sl)
    o2, l2 = fa.paged_decode(qd, kd, vd, bt, sl)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
