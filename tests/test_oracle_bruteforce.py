"""Pin the dense oracle against a pure-Python brute force on tiny inputs.

The brute force shares nothing with ``oracle/``: it walks the block table with
``divmod``, builds each query's allowed key set from explicit integer ranges
(window interval, then every image range holding the query, clamped on the
left to the window edge), and evaluates the softmax with ``math.exp`` and
``math.fsum`` in float64.  The oracle instead builds a boolean mask from
conjunctions and uses numpy in fp32.  A dropped term, a wrong sign, an
off-by-one window edge, a transposed operand or a wrong GQA map in either
shows up as a mismatch.
"""

import math

import numpy as np
import pytest

import oracle
from workloads import make_workload


def brute_allowed_keys(a, L, causal, wl, wr, ranges):
    keys = set()
    left = a - wl if wl >= 0 else 0
    if causal:
        right = a
    else:
        right = a + wr if wr >= 0 else L - 1
    keys.update(range(max(left, 0), min(right, L - 1) + 1))
    for st, en in ranges:
        if st < en and st <= a <= en:
            mleft = st if wl < 0 else max(st, a - wl)
            keys.update(range(max(mleft, 0), min(en, L - 1) + 1))
    return keys


def brute_row(w, s, i, h):
    """Output vector (list of floats) for local row i of sequence s, head h."""
    P = w.page_size
    c = int(w.ctx_lens[s])
    n = int(w.q_lens[s])
    L = c + n
    q0 = int(w.query_start_loc[s])
    kvh = h // (w.num_heads // w.num_kv_heads)
    qf, kn, vn = w.f32("q"), w.f32("k_new"), w.f32("v_new")
    kc, vc = w.f32("k_cache"), w.f32("v_cache")

    def key_row(j, new_arr, cache_arr):
        if j < c:
            page_idx, slot = divmod(j, P)
            page = int(w.block_table[s][page_idx])
            return [float(x) for x in cache_arr[page][slot][kvh]]
        return [float(x) for x in new_arr[q0 + (j - c)][kvh]]

    a = c + i
    keys = sorted(brute_allowed_keys(a, L, w.causal, w.window_left, w.window_right,
                                     w.mm_list(s)))
    qv = [float(x) for x in qf[q0 + i][h]]
    scores = []
    for j in keys:
        kv = key_row(j, kn, kc)
        scores.append(w.scale * math.fsum(qa * kb for qa, kb in zip(qv, kv)))
    mx = max(scores)
    ex = [math.exp(x - mx) for x in scores]
    den = math.fsum(ex)
    out = []
    vrows = [key_row(j, vn, vc) for j in keys]
    for dd in range(w.head_size):
        out.append(math.fsum(e * vr[dd] for e, vr in zip(ex, vrows)) / den)
    return out


def random_tiny_workload(rng, case):
    S = int(rng.integers(1, 4))
    Hkv = int(rng.choice([1, 2]))
    group = int(rng.choice([1, 2, 3]))
    d = int(rng.choice([4, 8, 16]))
    P = int(rng.choice([1, 3, 4, 5, 16, 40]))
    ctx = rng.integers(0, 40, size=S)
    new = rng.integers(1, 25, size=S)
    causal = bool(rng.integers(0, 2))
    wl = int(rng.choice([-1, 0, 1, 3, 7, 20]))
    wr = int(rng.choice([-1, 0, 2, 5, 30]))
    R = int(rng.choice([0, 1, 2, 3]))
    mm = None
    if R:
        mm = np.zeros((S, R, 2), dtype=np.int32)
        for s in range(S):
            L = int(ctx[s] + new[s])
            for r in range(R):
                st = int(rng.integers(0, L + 3))
                # widths up to beyond the window; some degenerate (st == en)
                en = st + int(rng.choice([0, 1, 4, 12, 30]))
                mm[s, r] = (st, en)
    return make_workload(seed=5000 + case, ctx_lens=ctx, q_lens=new, num_heads=Hkv * group,
                         num_kv_heads=Hkv, head_size=d, page_size=P, causal=causal,
                         window_left=wl, window_right=wr, mm_ranges=mm,
                         scale=float(rng.uniform(0.2, 1.0)))


def oracle_full(w):
    return oracle.reference_prefill(
        w.f32("q"), w.f32("k_new"), w.f32("v_new"), w.f32("k_cache"), w.f32("v_cache"),
        w.block_table, w.query_start_loc, w.ctx_lens, w.num_heads, w.num_kv_heads,
        w.head_size, w.page_size, w.window_left, w.window_right, w.causal, w.mm_ranges,
        w.scale)


@pytest.mark.parametrize("chunk", range(4))
def test_oracle_matches_bruteforce_random(chunk):
    """200 random tiny cases (50 per chunk) over every mask mode and page size."""
    rng = np.random.default_rng(77 + chunk)
    worst = 0.0
    for case in range(50):
        w = random_tiny_workload(rng, chunk * 50 + case)
        ref = oracle_full(w)
        assert np.isfinite(ref).all()
        for s in range(w.num_seqs):
            for i in range(int(w.q_lens[s])):
                for h in range(w.num_heads):
                    b = np.array(brute_row(w, s, i, h))
                    o = ref[int(w.query_start_loc[s]) + i, h]
                    err = float(np.abs(o - b).max())
                    worst = max(worst, err)
                    assert err <= 1e-5, (chunk, case, s, i, h, err)
    assert worst <= 1e-5


def test_oracle_matches_bruteforce_config1_shape():
    """The tiny benchmark shape (1 seq, 32 cached + 48 new, P=16, 4/2 heads, d=64)."""
    from workloads import make_config
    w = make_config(1)
    ref = oracle_full(w)
    for i in range(0, 48, 7):
        for h in range(4):
            b = np.array(brute_row(w, 0, i, h))
            assert np.abs(ref[i, h] - b).max() <= 1e-5
