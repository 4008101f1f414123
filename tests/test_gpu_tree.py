"""Draft-tree verification parity: fa_tree_decode through the C ABI against the fp64 oracle."""
import numpy as np
import pytest

import exact_attention_26_amd as fa
from exact_attention_26_amd import workloads as w
from gpu_util import LSE_ATOL, O_ATOL, assert_close, say, to_dev, to_host
from oracle import tree_decode_fp64

pytestmark = pytest.mark.gpu


def _run(wl, parents, q, kc, vc, device, max_q_len=None, scale=None):
    import torch
    L = wl.layout
    scale = L.scale if scale is None else scale
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(device)  # noqa: E731
    o, lse = fa.tree_decode(to_dev(q, "bf16", device), to_dev(kc, "bf16", device),
                            to_dev(vc, "bf16", device), t(L.block_table), t(L.seq_lens),
                            t(wl.cu_seqlens_q), t(parents.astype(np.int32)),
                            max_q_len or wl.max_q_len, scale=scale)
    torch.cuda.synchronize()
    return to_host(o), to_host(lse)


def _check(tag, got, want):
    assert_close(f"{tag} o", got[0], want[0], O_ATOL["bf16"])
    assert_close(f"{tag} lse", got[1], want[1], LSE_ATOL["bf16"])


def _shapes():
    """(committed tokens, parents) per sequence: chains, stars, random trees,
    single nodes, 64 nodes, trees straddling tile and page edges."""
    rng = np.random.default_rng(70)
    rand = lambda n: [-1] + [int(rng.integers(-1, i)) for i in range(1, n)]  # noqa: E731
    return [
        (0, [-1]),
        (5, [-1, 0, 1, 2]),
        (100, [-1] * 7),
        (63, rand(17)),
        (64, rand(64)),
        (1000, [-1] + list(range(63))),
        (37, rand(33)),
        (200, [-1, 0, 0, 1, 1, 2, 2, 3]),
        (1, rand(64)),
        (512, rand(40)),
    ]


@pytest.mark.parametrize("d", [64, 128])
def test_tree_edge_batches(gpu_device, d):
    shapes = _shapes()
    ctx = [c for c, _ in shapes]
    new = [len(p) for _, p in shapes]
    parents = np.concatenate([np.array(p, dtype=np.int32) for _, p in shapes])
    wl, _ = w.tree_workload(701 + d, S=len(shapes), H=3, d=d, ctx_lens=ctx, new_lens=new,
                            shared_prefix=32, spare=4)
    q = w.prefill_q(wl)
    kc = w.decode_pool(wl.layout, "k", poison=True)
    vc = w.decode_pool(wl.layout, "v", poison=True)
    L = wl.layout
    say(f"tree edges d={d} S={len(shapes)}")
    got = _run(wl, parents, q, kc, vc, gpu_device)
    want = tree_decode_fp64(q, kc, vc, L.block_table, L.seq_lens, wl.cu_seqlens_q, parents,
                            scale=L.scale)
    _check(f"tree d={d}", got, want)


def test_tree_parents_out_of_range_are_roots(gpu_device):
    # a parent index not before the node (or below -1) hangs it off the context
    wl, _ = w.tree_workload(711, S=2, H=2, d=128, ctx_lens=[50, 0], new_lens=[6, 5], spare=4)
    parents = np.array([3, 0, 9, -5, 1, 4, -1, 0, 7, 2, 2], dtype=np.int32)
    q = w.prefill_q(wl)
    kc = w.decode_pool(wl.layout, "k", poison=True)
    vc = w.decode_pool(wl.layout, "v", poison=True)
    L = wl.layout
    say("tree out-of-range parents")
    got = _run(wl, parents, q, kc, vc, gpu_device)
    want = tree_decode_fp64(q, kc, vc, L.block_table, L.seq_lens, wl.cu_seqlens_q, parents,
                            scale=L.scale)
    _check("bad parents", got, want)


def test_tree_negative_scale(gpu_device):
    wl, _ = w.tree_workload(715, S=2, H=2, d=128, ctx_lens=[0, 90], new_lens=[7, 30], spare=4)
    parents = np.array([-1, 0, 0, 1, -1, 4, 2] + [-1] + list(range(29)), dtype=np.int32)
    q = w.prefill_q(wl)
    kc = w.decode_pool(wl.layout, "k", poison=True)
    vc = w.decode_pool(wl.layout, "v", poison=True)
    L = wl.layout
    say("tree scale=-0.2")
    got = _run(wl, parents, q, kc, vc, gpu_device, scale=-0.2)
    want = tree_decode_fp64(q, kc, vc, L.block_table, L.seq_lens, wl.cu_seqlens_q, parents,
                            scale=-0.2)
    _check("negative scale", got, want)


def test_tree_full_size(gpu_device):
    """The bench workload (64 sequences, 128..8192 committed tokens, 64-node
    trees, H=32, d=128), NaN-poisoned pools; every node of sampled sequences."""
    wl, parents = w.tree_workload(**w.TREE_T1)
    q = w.prefill_q(wl)
    kc = w.decode_pool(wl.layout, "k", poison=True)
    vc = w.decode_pool(wl.layout, "v", poison=True)
    L = wl.layout
    say("tree full T1")
    o, lse = _run(wl, parents, q, kc, vc, gpu_device)
    seqs = [0, 1, 17, 40, L.S - 1]
    rows = np.concatenate([np.arange(wl.cu_seqlens_q[s], wl.cu_seqlens_q[s + 1]) for s in seqs])
    # the oracle over the chosen sequences only (same tables and lengths)
    cu_sub = np.concatenate([[0], np.cumsum([wl.new_lens[s] for s in seqs])]).astype(np.int32)
    want = tree_decode_fp64(q[rows], kc, vc, L.block_table[seqs], L.seq_lens[seqs], cu_sub,
                            parents[rows], scale=L.scale)
    _check("T1", (o[rows], lse[rows]), want)


def test_tree_deterministic_and_rejects_big_trees(gpu_device):
    import torch
    wl, parents = w.tree_workload(721, S=3, H=2, d=64, ctx_lens=[10, 300, 70],
                                  new_lens=[64, 1, 20], spare=4)
    q = w.prefill_q(wl)
    kc = w.decode_pool(wl.layout, "k")
    vc = w.decode_pool(wl.layout, "v")
    say("tree determinism")
    a = _run(wl, parents, q, kc, vc, gpu_device)
    b = _run(wl, parents, q, kc, vc, gpu_device)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    with pytest.raises(fa.FaError) as e:
        _run(wl, parents, q, kc, vc, gpu_device, max_q_len=65)
    assert e.value.status == 2


def test_tree_more_nodes_than_the_limit_keeps_positions(gpu_device):
    """Device data with 70 nodes in a sequence (max_q_len says 64): nodes
    0..63 are computed at their true positions (the tree's K/V are still the
    last 70 cached tokens) and nodes 64..69 are not written."""
    import torch
    wl, parents = w.tree_workload(731, S=2, H=2, d=128, ctx_lens=[100, 40], new_lens=[70, 10],
                                  spare=4)
    q = w.prefill_q(wl)
    kc = w.decode_pool(wl.layout, "k", poison=True)
    vc = w.decode_pool(wl.layout, "v", poison=True)
    L = wl.layout
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(gpu_device)  # noqa: E731
    o = torch.full((wl.total_q, L.H, L.d), 7.0, dtype=torch.bfloat16, device=gpu_device)
    lse = torch.full((wl.total_q, L.H), 7.0, dtype=torch.float32, device=gpu_device)
    say("tree 70 nodes, max_q_len 64")
    fa.fa_tree_decode(to_dev(q, "bf16", gpu_device), to_dev(kc, "bf16", gpu_device),
                      to_dev(vc, "bf16", gpu_device), t(L.block_table), t(L.seq_lens),
                      t(wl.cu_seqlens_q), t(parents.astype(np.int32)), o, lse, 64, L.scale)
    torch.cuda.synchronize()
    o, lse = to_host(o), to_host(lse)
    want = tree_decode_fp64(q, kc, vc, L.block_table, L.seq_lens, wl.cu_seqlens_q, parents,
                            scale=L.scale)
    done = np.r_[0:64, 70:80]
    _check("first 64 nodes", (o[done], lse[done]), (want[0][done], want[1][done]))
    assert np.all(o[64:70] == 7.0) and np.all(lse[64:70] == 7.0), "nodes past 64 were written"
