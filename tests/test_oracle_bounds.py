"""Pin the oracle's tile bounds and useful-pair count.

* the two loop ranges printed on the vLLM PR #53147 report (golden fixture);
* soundness: no allowed (query, key) pair of a Q tile lies outside the
  returned KV-tile range (brute force over the dense mask);
* tightness: the range is exactly the tiles of the smallest and largest
  allowed key over the tile's rows (brute force);
* for full query blocks with no context, the loop limits of the vLLM
  PR #50776 report's windowed prefill (start rounded down to a key block,
  end = last needed key + 1) visit exactly the same tiles;
* restricting the oracle to the bounded keys changes nothing (pruned = dense);
* the per-row closed form of the allowed set equals the dense mask, and the
  useful-pair counts of the tiny and sliding-window configs equal their
  closed-form values.
"""

import os

import numpy as np
import pytest

import oracle
from workloads import make_config, make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tile_bounds_printed.txt")


def load_golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        f = line.split()
        ranges = [tuple(int(x) for x in r.split(":")) for r in f[8].split(";")]
        rows.append(dict(c=int(f[0]), L=int(f[1]), block_q=int(f[2]), t=int(f[3]),
                         block_n=int(f[4]), causal=bool(int(f[5])), wl=int(f[6]),
                         wr=int(f[7]), ranges=ranges, expect=(int(f[9]), int(f[10]))))
    return rows


@pytest.mark.parametrize("case", load_golden())
def test_printed_bounds(case):
    n = case["L"] - case["c"]
    got = oracle.tile_bounds_ref(case["c"], n, case["t"], case["block_q"], case["block_n"],
                                 case["causal"], case["wl"], case["wr"], case["ranges"])
    assert got == case["expect"]
    # the printed query rows of this block
    assert case["t"] * case["block_q"] == 1120
    # without pruning the loop would scan every tile
    assert case["L"] // case["block_n"] == 128


def brute_tile_range(c, n, t, block_q, block_n, causal, wl, wr, ranges):
    rows = np.arange(t * block_q, min((t + 1) * block_q, n))
    if rows.size == 0:
        return None
    m = oracle.allowed_mask(c, n, causal, wl, wr, ranges, rows=rows)
    js = np.nonzero(m.any(axis=0))[0]
    return js.min(), js.max()


def random_geometry(rng):
    c = int(rng.integers(0, 300))
    n = int(rng.integers(1, 300))
    causal = bool(rng.integers(0, 2))
    wl = int(rng.choice([-1, 0, 1, 5, 31, 64, 100, 1000]))
    wr = int(rng.choice([-1, 0, 3, 17, 64, 500]))
    R = int(rng.integers(0, 4))
    L = c + n
    ranges = []
    for _ in range(R):
        st = int(rng.integers(0, L + 5))
        ranges.append((st, st + int(rng.choice([0, 1, 7, 40, 150, 400]))))
    block_q = int(rng.choice([1, 8, 16, 32, 64, 128]))
    block_n = int(rng.choice([16, 32, 64, 128]))
    return c, n, causal, wl, wr, ranges, block_q, block_n


def test_bounds_sound_and_tight_bruteforce():
    rng = np.random.default_rng(2024)
    checked = 0
    for _ in range(400):
        c, n, causal, wl, wr, ranges, bq, bn = random_geometry(rng)
        for t in range(-(-n // bq) + 1):
            lo, hi = oracle.tile_bounds_ref(c, n, t, bq, bn, causal, wl, wr, ranges)
            br = brute_tile_range(c, n, t, bq, bn, causal, wl, wr, ranges)
            if br is None:
                assert (lo, hi) == (0, 0)
                continue
            jmin, jmax = br
            # sound: every allowed key lies in [lo*bn, hi*bn)
            assert lo * bn <= jmin and jmax < hi * bn
            # tight: exactly the tiles of the extreme allowed keys
            assert (lo, hi) == (jmin // bn, jmax // bn + 1)
            checked += 1
    assert checked > 1000


def test_matches_windowed_prefill_loop_limits_full_blocks():
    """vLLM PR #50776 report, "Key source snippets": full query blocks, no context."""
    for (bm, bn, swq, swk) in [(128, 64, 64, 64), (64, 32, 10, 0), (128, 64, 200, 7),
                               (32, 32, 1, 100)]:
        n = 4096
        for start_m in range(n // bm):
            first_needed = start_m * bm - swq
            start = max(0, (first_needed // bn) * bn)
            end = n
            last_needed = (start_m + 1) * bm - 1 + swk
            end = min(end, last_needed + 1)
            p2 = (start // bn, -(-end // bn))
            ours = oracle.tile_bounds_ref(0, n, start_m, bm, bn, False, swq, swk, [])
            assert ours == p2


@pytest.mark.parametrize("mode", [
    dict(causal=True, wl=-1, wr=-1, mm=None),
    dict(causal=False, wl=9, wr=4, mm=None),
    dict(causal=True, wl=12, wr=-1, mm=np.array([[[5, 60], [70, 71]], [[0, 0], [10, 30]]])),
    dict(causal=False, wl=-1, wr=-1, mm=None),
])
def test_pruned_equals_dense(mode):
    w = make_workload(seed=8, ctx_lens=[50, 13], q_lens=[40, 29], num_heads=2,
                      num_kv_heads=1, head_size=16, page_size=7, causal=mode["causal"],
                      window_left=mode["wl"], window_right=mode["wr"], mm_ranges=mode["mm"])
    bq, bn = 8, 16
    args = (w.f32("q"), w.f32("k_new"), w.f32("v_new"), w.f32("k_cache"), w.f32("v_cache"),
            w.block_table, w.query_start_loc, w.ctx_lens, 2, 1, 16, 7, w.window_left,
            w.window_right, w.causal, w.mm_ranges, w.scale)
    for s in range(2):
        n, c = int(w.q_lens[s]), int(w.ctx_lens[s])
        for t in range(-(-n // bq)):
            rows = np.arange(t * bq, min(n, (t + 1) * bq))
            lo, hi = oracle.tile_bounds_ref(c, n, t, bq, bn, w.causal, w.window_left,
                                            w.window_right, w.mm_list(s))
            dense = oracle.reference_rows(*args, s, rows)
            pruned = oracle.reference_rows(*args, s, rows,
                                           key_range=(lo * bn, min(hi * bn, c + n)))
            assert np.abs(dense - pruned).max() <= 1e-6


def test_row_intervals_equal_dense_mask():
    rng = np.random.default_rng(5)
    for _ in range(300):
        c, n, causal, wl, wr, ranges, _, _ = random_geometry(rng)
        lo, hi = oracle.row_intervals(c, n, causal, wl, wr, ranges)
        m = oracle.allowed_mask(c, n, causal, wl, wr, ranges)
        j = np.arange(c + n)[None, :]
        assert np.array_equal(m, (j >= lo[:, None]) & (j <= hi[:, None]))


def test_useful_pairs_closed_forms():
    # tiny config: causal, 32 cached + 48 new -> row i sees 33 + i keys
    w1 = make_config(1)
    assert oracle.useful_pairs(w1.ctx_lens, w1.q_lens, True, -1, -1, None) == \
        sum(33 + i for i in range(48)) == 2712
    # sliding window +-64 over 16384 tokens, non-causal: 129 keys per row
    # except 64 rows at each end, which lose 64..1 keys
    u4 = oracle.useful_pairs([0], [16384], False, 64, 64, None)
    assert u4 == 16384 * 129 - 2 * (64 * 65 // 2) == 2_109_376
    # brute count on random geometries
    rng = np.random.default_rng(9)
    for _ in range(200):
        c, n, causal, wl, wr, ranges, _, _ = random_geometry(rng)
        mm = np.array(ranges, dtype=np.int64).reshape(1, -1, 2) if ranges else None
        got = oracle.useful_pairs([c], [n], causal, wl, wr, mm)
        assert got == int(oracle.allowed_mask(c, n, causal, wl, wr, ranges).sum())


def test_tile_bounds_all_shape_and_padding():
    out = oracle.tile_bounds_all([5, 0, 9], [20, 3, 1], 8, 16, True, -1, -1, None)
    assert out.shape == (3, 3, 2)
    assert tuple(out[1, 1]) == (0, 0) and tuple(out[2, 1]) == (0, 0)
    assert tuple(out[0, 2]) == (0, (5 + 19) // 16 + 1)
