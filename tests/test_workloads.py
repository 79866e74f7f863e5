"""Seeded generator: determinism, poison placement and the page layout."""

import numpy as np

from workloads import bf16_bits_to_f32, make_config, make_workload


def test_deterministic():
    a = make_workload(seed=3, ctx_lens=[40, 7], q_lens=[5, 9], num_heads=2, num_kv_heads=1,
                      head_size=8, page_size=6, causal=True)
    b = make_workload(seed=3, ctx_lens=[40, 7], q_lens=[5, 9], num_heads=2, num_kv_heads=1,
                      head_size=8, page_size=6, causal=True)
    for f in ("q", "k_new", "v_new", "k_cache", "v_cache", "block_table"):
        assert np.array_equal(getattr(a, f), getattr(b, f))


def test_poison_and_unused_entries():
    w = make_workload(seed=4, ctx_lens=[13, 0, 6], q_lens=[3, 4, 5], num_heads=1,
                      num_kv_heads=1, head_size=4, page_size=4, causal=True)
    kc = bf16_bits_to_f32(w.k_cache)
    used = np.zeros(kc.shape[:2], dtype=bool)
    for s in range(3):
        c = int(w.ctx_lens[s])
        npg = -(-c // 4)
        assert (w.block_table[s, npg:] == -1).all()
        for j in range(c):
            used[w.block_table[s, j // 4], j % 4] = True
    assert np.isfinite(kc[used]).all()
    assert np.isnan(kc[~used]).all()
    assert w.num_pages == 4 + 2 + 1  # 13 and 6 cached tokens -> 4 + 2 pages, plus 10% spare


def test_config_shapes():
    w1 = make_config(1)
    assert w1.block_table.shape == (1, 8) and sorted(w1.block_table[0]) == list(range(8))
    assert (w1.ctx_lens[0], w1.q_lens[0]) == (32, 48)
    w4 = make_config(4, new_tokens=256)
    assert w4.num_pages == 1 and w4.max_pages_per_seq == 1 and int(w4.block_table[0, 0]) == -1
    w5 = make_config(5, heads=(2, 1), new_tokens=12454)
    st, en = w5.mm_ranges[0, :, 0], w5.mm_ranges[0, :, 1]
    assert w5.mm_ranges.shape == (1, 60, 2)
    assert ((en - st) == 255).all() and (st[1:] > en[:-1]).all()
    assert st[0] >= 0 and en[-1] <= 16549


def test_sigma_one_unchanged_draw():
    """qk_sigma = 1 gives the plain draw's bits (the benchmark inputs are unchanged);
    other values widen Q and K only."""
    kw = dict(seed=5, ctx_lens=[10], q_lens=[7], num_heads=2, num_kv_heads=1,
              head_size=64, page_size=16, causal=True)
    a = make_workload(**kw)
    b = make_workload(qk_sigma=1.0, **kw)
    c = make_workload(qk_sigma=3.0, **kw)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k_cache, b.k_cache)
    assert np.array_equal(a.v_new, c.v_new)
    ratio = np.abs(c.f32("q")).mean() / np.abs(a.f32("q")).mean()
    assert 2.9 < ratio < 3.1
