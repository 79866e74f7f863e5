"""Pin the oracle's mask variants and the split-KV merge.

Variants (vLLM PR #53147 report, "Key source snippets", compute_tile_loop_bounds,
and "Review highlights"): chunked local attention, a causal flag per
sequence, and multimodal ranges without the window clamp.  Split-KV: the
log-sum-exp merge of per-segment softmax results.

Pins, none of which re-types the oracle's own formula:

* a pure-Python brute force that builds each query's allowed key set from
  integer ranges (chunk start by ``divmod``, per-sequence flags looked up per
  sequence) and evaluates the softmax with ``math.exp`` / ``math.fsum``;
* identities: chunk size 1 with lookback k is the window ``window_left = k``;
  a lookback covering the whole sequence removes the left edge; per-sequence
  flags that are all equal give the scalar flag; without a left window the
  clamp makes no difference;
* tile bounds: every allowed key of a tile's rows lies in ``[lo, hi)`` KV
  tiles and the first and last of those tiles hold an allowed key (tight),
  checked by brute force; pruning to the bounds changes the fp64 output
  only by summation order;
* split-KV: merging any contiguous segmentation of the keys reproduces the
  unsplit output; a single segment is the identity; a segment with no
  allowed key carries zero weight.
"""

import math

import numpy as np
import pytest

import oracle
from workloads import make_workload


def brute_keys(a, L, causal, wl, wr, ranges, cs, lb, clamp):
    if cs > 0 and lb >= 0:
        chunk, _ = divmod(a, cs)
        left = (chunk - lb) * cs
    else:
        left = a - wl if wl >= 0 else 0
    right = a if causal else (a + wr if wr >= 0 else L - 1)
    keys = set(range(max(left, 0), min(right, L - 1) + 1))
    for st, en in ranges:
        if st < en and st <= a <= en:
            mleft = max(st, a - wl) if (clamp and wl >= 0) else st
            keys.update(range(max(mleft, 0), min(en, L - 1) + 1))
    return keys


def seq_flag(w, s):
    return bool(w.causal_per_seq[s]) if w.causal_per_seq is not None else w.causal


def brute_out(w, s, i, h):
    P = w.page_size
    c, n = int(w.ctx_lens[s]), int(w.q_lens[s])
    L, q0 = c + n, int(w.query_start_loc[s])
    g = h // (w.num_heads // w.num_kv_heads)
    qf, kn, vn = w.f32("q"), w.f32("k_new"), w.f32("v_new")
    kc, vc = w.f32("k_cache"), w.f32("v_cache")

    def row(j, new_arr, cache_arr):
        if j < c:
            pi, slot = divmod(j, P)
            return [float(x) for x in cache_arr[int(w.block_table[s][pi])][slot][g]]
        return [float(x) for x in new_arr[q0 + j - c][g]]

    keys = sorted(brute_keys(c + i, L, seq_flag(w, s), w.window_left, w.window_right,
                             w.mm_list(s), w.chunk_size, w.chunk_lookback, w.mm_clamp))
    qv = [float(x) for x in qf[q0 + i][h]]
    sc = [w.scale * math.fsum(x * y for x, y in zip(qv, row(j, kn, kc))) for j in keys]
    mx = max(sc)
    ex = [math.exp(x - mx) for x in sc]
    den = math.fsum(ex)
    vr = [row(j, vn, vc) for j in keys]
    return [math.fsum(e * v[d] for e, v in zip(ex, vr)) / den for d in range(w.head_size)]


def random_variant(rng, case):
    S = int(rng.integers(1, 4))
    Hkv = int(rng.choice([1, 2]))
    group = int(rng.choice([1, 2]))
    d = int(rng.choice([4, 8]))
    P = int(rng.choice([1, 3, 5, 16]))
    ctx = rng.integers(0, 40, size=S)
    new = rng.integers(1, 25, size=S)
    wl = int(rng.choice([-1, 0, 2, 7, 20]))
    wr = int(rng.choice([-1, 0, 3, 30]))
    cs = int(rng.choice([0, 1, 4, 7, 16]))
    lb = int(rng.choice([-1, 0, 1, 2]))
    per_seq = rng.integers(0, 2, size=S) if rng.random() < 0.5 else None
    R = int(rng.choice([0, 1, 2, 3]))
    mm = None
    if R:
        mm = np.zeros((S, R, 2), dtype=np.int32)
        for s in range(S):
            L = int(ctx[s] + new[s])
            for r in range(R):
                st = int(rng.integers(0, L + 3))
                mm[s, r] = (st, st + int(rng.choice([0, 1, 5, 14, 30])))
    return make_workload(seed=7000 + case, ctx_lens=ctx, q_lens=new, num_heads=Hkv * group,
                         num_kv_heads=Hkv, head_size=d, page_size=P,
                         causal=bool(rng.integers(0, 2)), window_left=wl, window_right=wr,
                         mm_ranges=mm, scale=float(rng.uniform(0.3, 1.0)),
                         causal_per_seq=per_seq, mm_clamp=bool(rng.integers(0, 2)),
                         chunk_size=cs, chunk_lookback=lb)


def full(w, **over):
    kw = w.mask_kwargs()
    kw.update({k: v for k, v in over.items() if k in kw})
    return oracle.reference_prefill(
        w.f32("q"), w.f32("k_new"), w.f32("v_new"), w.f32("k_cache"), w.f32("v_cache"),
        w.block_table, w.query_start_loc, w.ctx_lens, w.num_heads, w.num_kv_heads,
        w.head_size, w.page_size, over.get("window_left", w.window_left),
        w.window_right, over.get("causal", w.causal_arg), w.mm_ranges, w.scale, **kw)


@pytest.mark.parametrize("chunk", range(3))
def test_variants_match_bruteforce(chunk):
    rng = np.random.default_rng(880 + chunk)
    for case in range(40):
        w = random_variant(rng, chunk * 40 + case)
        ref = full(w)
        for s in range(w.num_seqs):
            q0 = int(w.query_start_loc[s])
            for i in range(int(w.q_lens[s])):
                for h in range(w.num_heads):
                    b = np.array(brute_out(w, s, i, h))
                    assert np.abs(ref[q0 + i, h] - b).max() < 2e-5, (case, s, i, h)


def _base(**kw):
    args = dict(seed=31, ctx_lens=[37, 0, 90], q_lens=[50, 23, 41], num_heads=4,
                num_kv_heads=2, head_size=8, page_size=7, causal=True)
    args.update(kw)
    return make_workload(**args)


def test_chunk_size_one_is_window():
    mm = np.array([[[10, 60], [70, 80]], [[0, 9], [3, 3]], [[40, 120], [0, 0]]], np.int32)
    for k in (0, 3, 11):
        w = _base(mm_ranges=mm, window_left=k, chunk_size=1, chunk_lookback=k)
        plain = full(w, chunk_size=0, chunk_lookback=-1)
        assert np.array_equal(full(w), plain)


def test_long_lookback_removes_left_edge():
    w = _base(chunk_size=16, chunk_lookback=100)
    assert np.array_equal(full(w), full(w, chunk_size=0, chunk_lookback=-1))


def test_chunk_without_lookback_is_local_and_differs():
    w = _base(chunk_size=16, chunk_lookback=0)
    mask = oracle.allowed_mask(37, 50, True, -1, -1, [], chunk_size=16, chunk_lookback=0)
    # row 0 (a = 37) sees keys 32..37 only
    assert np.flatnonzero(mask[0]).tolist() == list(range(32, 38))
    assert not np.allclose(full(w), full(w, chunk_size=0, chunk_lookback=-1))


def test_per_seq_flags_all_equal_give_scalar_flag():
    for flag in (0, 1):
        w = _base(causal=bool(flag), causal_per_seq=[flag] * 3, window_right=5)
        assert np.array_equal(full(w), full(w, causal=bool(flag)))


def test_per_seq_flags_mix_per_sequence():
    w = _base(causal=True, causal_per_seq=[1, 0, 1])
    out = full(w)
    nc = full(w, causal=False)
    c = full(w, causal=True)
    q = w.query_start_loc
    assert np.array_equal(out[q[0]:q[1]], c[q[0]:q[1]])
    assert np.array_equal(out[q[1]:q[2]], nc[q[1]:q[2]])
    assert np.array_equal(out[q[2]:q[3]], c[q[2]:q[3]])


def test_clamp_is_moot_without_left_window():
    mm = np.array([[[5, 70], [0, 0]], [[0, 20], [0, 0]], [[10, 100], [0, 0]]], np.int32)
    w = _base(mm_ranges=mm, window_left=-1, mm_clamp=False)
    assert np.array_equal(full(w), full(w, mm_clamp=True))
    w2 = _base(mm_ranges=mm, window_left=4, mm_clamp=False)
    assert not np.allclose(full(w2), full(w2, mm_clamp=True))


@pytest.mark.parametrize("block_q,block_n", [(4, 8), (16, 32), (64, 16)])
def test_variant_bounds_sound_tight_and_pruning_exact(block_q, block_n):
    rng = np.random.default_rng(4040 + block_q)
    for case in range(25):
        w = random_variant(rng, 300 + case)
        causal = w.causal_arg
        tb = oracle.tile_bounds_all(w.ctx_lens, w.q_lens, block_q, block_n, causal,
                                    w.window_left, w.window_right, w.mm_ranges,
                                    **w.mask_kwargs())
        for s in range(w.num_seqs):
            c, n = int(w.ctx_lens[s]), int(w.q_lens[s])
            L = c + n
            for t in range(tb.shape[1]):
                lo, hi = (int(x) for x in tb[s, t])
                rows = range(t * block_q, min((t + 1) * block_q, n))
                if not rows:
                    assert (lo, hi) == (0, 0)
                    continue
                keys = set()
                for i in rows:
                    keys |= brute_keys(c + i, L, seq_flag(w, s), w.window_left,
                                       w.window_right, w.mm_list(s), w.chunk_size,
                                       w.chunk_lookback, w.mm_clamp)
                assert min(keys) // block_n == lo and max(keys) // block_n + 1 == hi
                kw = w.mask_kwargs()
                args = (w.f32("q"), w.f32("k_new"), w.f32("v_new"), w.f32("k_cache"),
                        w.f32("v_cache"), w.block_table, w.query_start_loc, w.ctx_lens,
                        w.num_heads, w.num_kv_heads, w.head_size, w.page_size,
                        w.window_left, w.window_right, causal, w.mm_ranges, w.scale, s,
                        np.array(list(rows)))
                dense = oracle.reference_rows(*args, dtype=np.float64, **kw)
                pruned = oracle.reference_rows(*args, key_range=(lo * block_n,
                                                                 min(hi * block_n, L)),
                                               dtype=np.float64, **kw)
                # only masked keys are dropped: equal up to summation order
                assert np.abs(dense - pruned).max() < 1e-12


def test_variant_useful_pairs_equal_mask_count():
    rng = np.random.default_rng(99)
    for case in range(30):
        w = random_variant(rng, 600 + case)
        dense = 0
        for s in range(w.num_seqs):
            dense += int(oracle.allowed_mask(
                int(w.ctx_lens[s]), int(w.q_lens[s]), seq_flag(w, s), w.window_left,
                w.window_right, w.mm_list(s), **w.mask_kwargs()).sum())
        assert oracle.useful_pairs(w.ctx_lens, w.q_lens, w.causal_arg, w.window_left,
                                   w.window_right, w.mm_ranges, **w.mask_kwargs()) == dense


def _segments(L, k, rng):
    cuts = sorted(rng.choice(np.arange(1, L), size=min(k - 1, L - 1), replace=False)) \
        if L > 1 else []
    edges = [0] + [int(x) for x in cuts] + [L]
    return list(zip(edges[:-1], edges[1:]))


@pytest.mark.parametrize("k", [1, 2, 3, 7])
def test_split_merge_reproduces_unsplit(k):
    rng = np.random.default_rng(12 + k)
    for case in range(12):
        w = random_variant(rng, 900 + 20 * k + case)
        for s in range(w.num_seqs):
            c, n = int(w.ctx_lens[s]), int(w.q_lens[s])
            rows = np.arange(n)
            args = (w.f32("q"), w.f32("k_new"), w.f32("v_new"), w.f32("k_cache"),
                    w.f32("v_cache"), w.block_table, w.query_start_loc, w.ctx_lens,
                    w.num_heads, w.num_kv_heads, w.head_size, w.page_size, w.window_left,
                    w.window_right, w.causal_arg, w.mm_ranges, w.scale, s, rows)
            kw = w.mask_kwargs()
            whole = oracle.reference_rows(*args, dtype=np.float64, **kw)
            parts = [oracle.reference_rows(*args, key_range=seg, dtype=np.float64,
                                           return_stats=True, **kw)
                     for seg in _segments(c + n, k, rng)]
            merged = oracle.merge_partials([p[0] for p in parts], [p[1] for p in parts],
                                           [p[2] for p in parts])
            assert np.abs(merged - whole).max() < 1e-10
            if k == 1:
                assert np.array_equal(parts[0][0], whole)


def test_split_segment_without_allowed_key_has_zero_weight():
    w = _base(window_left=3)  # causal band of 4 keys: early keys are never allowed late
    args = (w.f32("q"), w.f32("k_new"), w.f32("v_new"), w.f32("k_cache"), w.f32("v_cache"),
            w.block_table, w.query_start_loc, w.ctx_lens, w.num_heads, w.num_kv_heads,
            w.head_size, w.page_size, w.window_left, w.window_right, w.causal_arg,
            w.mm_ranges, w.scale, 0, np.arange(40, 50))
    empty = oracle.reference_rows(*args, key_range=(0, 10), return_stats=True)
    assert np.all(empty[2] == 0) and np.all(np.isneginf(empty[1])) and np.all(empty[0] == 0)
    rest = oracle.reference_rows(*args, key_range=(10, 87), return_stats=True)
    merged = oracle.merge_partials([empty[0], rest[0]], [empty[1], rest[1]],
                                   [empty[2], rest[2]])
    assert np.abs(merged - oracle.reference_rows(*args)).max() < 1e-6
