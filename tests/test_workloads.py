"""The seeded input generators: rounding, determinism and the paged layout's structure."""
import numpy as np
import pytest

from exact_attention_26_amd import workloads as w


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(0).standard_normal(100_000).astype(np.float32) * 7
    # include exact ties to check ties-to-even
    ties = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)], dtype=np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(w.round_to_bf16(x), ref)


def test_fwd_inputs_are_seeded_and_bf16_exact():
    a = w.fwd_inputs(1, 2, 33, 64, seed=5)
    b = w.fwd_inputs(1, 2, 33, 64, seed=5)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
        np.testing.assert_array_equal(w.round_to_bf16(x), x)
    c = w.fwd_inputs(1, 2, 33, 64, seed=6)
    assert not np.array_equal(a[0], c[0])


def test_long_config_scales_qk_only():
    q, k, v = w.fwd_inputs(1, 1, 4096, 128, seed=3, sigma_qk=3.0)
    assert 2.8 < q.std() < 3.2 and 2.8 < k.std() < 3.2 and 0.9 < v.std() < 1.1


def test_configs_hold_16k_tokens():
    for name, cfg in w.FWD_CONFIGS.items():
        if name != "smoke":
            assert cfg.B * cfg.N == 16384, name


def _check_layout(L):
    P = L.page_size
    used_total = 0
    owners = {}
    for s in range(L.S):
        n = int(L.seq_lens[s])
        used = L.used_pages(s)
        assert used.size == -(-n // P)
        # at most page_size - 1 slots wasted per sequence
        assert used.size * P - n <= P - 1
        assert np.all(L.block_table[s, used.size:] == L.poison_page)
        assert L.poison_page not in set(used.tolist())
        for p, blk in enumerate(used.tolist()):
            owners.setdefault(blk, []).append((s, p))
        used_total += used.size
    # a page is referenced once, or twice as the same logical page of a pair
    for blk, refs in owners.items():
        assert len(refs) in (1, 2)
        if len(refs) == 2:
            (s0, p0), (s1, p1) = refs
            assert s1 == s0 + 1 and s0 % 2 == 0 and p0 == p1
    assert set(L.shared_pages.tolist()) == {b for b, r in owners.items() if len(r) == 2}
    assert len(owners) + len(L.spare_pages) == L.num_blocks


def test_decode_layout_structure_small():
    L = w.decode_layout(11, S=6, H=2, d=8, page_size=4, len_range=(1, 40), shared_prefix=12,
                        spare=3)
    _check_layout(L)


def test_decode_layout_c4():
    L = w.decode_layout(**w.DECODE_C4)
    _check_layout(L)
    assert L.seq_lens.min() >= 128 and L.seq_lens.max() <= 8192
    assert L.max_blocks == 512
    # pairs share whole pages of their common prefix (up to 512 tokens)
    for a in range(0, L.S, 2):
        sp = min(512, int(L.seq_lens[a]), int(L.seq_lens[a + 1])) // 16
        np.testing.assert_array_equal(L.block_table[a, :sp], L.block_table[a + 1, :sp])


def test_pool_pages_regenerate_exactly_and_poison():
    L = w.decode_layout(12, S=4, H=2, d=8, page_size=4, len_range=(3, 30), shared_prefix=8,
                        spare=2)
    full = w.decode_pool(L, "k", poison=True)
    part = w.decode_pool_pages(L, "k", [0, L.poison_page, L.num_blocks - 1], poison=True)
    for p, x in part.items():
        np.testing.assert_array_equal(np.isnan(x), np.isnan(full[p]))
        np.testing.assert_array_equal(np.nan_to_num(x), np.nan_to_num(full[p]))
    assert np.isnan(full[L.poison_page]).all()
    valid = w.page_valid_slots(L)
    for blk in range(L.num_blocks):
        assert not np.isnan(full[blk, :, :valid[blk]]).any()
        assert np.isnan(full[blk, :, valid[blk]:]).all()
    clean = w.decode_pool(L, "k", poison=False)
    assert not np.isnan(clean).any()
    np.testing.assert_array_equal(np.nan_to_num(full, nan=0.0)[~np.isnan(full)],
                                  clean[~np.isnan(full)])
