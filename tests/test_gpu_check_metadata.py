"""GPU tests of prefill_attention_check_metadata, the device-side check of the
metadata preconditions that prefill_attention states but does not check.

Expected results come from the preconditions as the header states them,
evaluated here in plain Python, and from the corruption each case plants.  The
checker only reads the metadata arrays within their declared sizes, and no
attention launch ever sees corrupted metadata.
"""

import numpy as np
import pytest

from workloads import NAMED, make_config, make_named

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    import paged_kv_prefill_attention_amd as ppa
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    ppa.load_library()


def expected_flags(qsl, ctx, bt, page_size, num_pages, total, max_q_len, cache_only):
    import paged_kv_prefill_attention_amd as ppa
    f = 0
    S = len(ctx)
    if qsl[0] != 0 or qsl[S] != total:
        f |= ppa.BAD_QSL
    for s in range(S):
        n = int(qsl[s + 1]) - int(qsl[s])
        c = int(ctx[s])
        if n < 0:
            f |= ppa.BAD_QSL
        if n > max_q_len:
            f |= ppa.BAD_QLEN
        if c < 0:
            f |= ppa.BAD_CTX
        L = max(c, 0) + max(n, 0)
        if L > 1 << 24:
            f |= ppa.BAD_LENGTH
        cached = L if cache_only else max(c, 0)
        need = -(-cached // page_size)
        if need > bt.shape[1]:
            f |= ppa.BAD_PAGES
        for p in range(min(need, bt.shape[1])):
            if not 0 <= int(bt[s, p]) < num_pages:
                f |= ppa.BAD_PAGE_ID
    return f


def run_check(qsl, ctx, bt, page_size, num_pages, total, max_q_len, cache_only=False):
    import torch
    import paged_kv_prefill_attention_amd as ppa
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()  # noqa: E731
    got = ppa.check_metadata(i32(bt), i32(qsl), i32(ctx), page_size, num_pages, total,
                             max_q_len, cache_only=cache_only)
    want = expected_flags(np.asarray(qsl), np.asarray(ctx), np.asarray(bt), page_size,
                          num_pages, total, max_q_len, cache_only)
    assert got == want, (got, want)
    return got


def meta(w):
    return (w.query_start_loc.copy(), w.ctx_lens.copy(), w.block_table.copy(), w.page_size,
            int(w.k_cache.shape[0]), int(w.total_q_tokens), int(w.max_q_len))


@pytest.mark.parametrize("cid,P", [(1, None), (2, None), (3, 1040), (3, 1056), (4, None),
                                   (5, None)])
def test_benchmark_workloads_pass(cid, P):
    w = make_config(cid, page_size=P)
    assert run_check(*meta(w)) == 0


@pytest.mark.parametrize("name", NAMED)
def test_named_workloads_pass(name):
    assert run_check(*meta(make_named(name))) == 0


def test_each_precondition_sets_its_bit():
    import paged_kv_prefill_attention_amd as ppa
    w = make_config(2)
    qsl, ctx, bt, P, npages, T, mq = meta(w)
    S = len(ctx)

    def case(bit, qsl=qsl, ctx=ctx, bt=bt, total=T, max_q_len=mq):
        got = run_check(qsl, ctx, bt, P, npages, total, max_q_len)
        assert got & bit, (got, bit)
        return got

    q = qsl.copy(); q[0] = 1
    case(ppa.BAD_QSL, qsl=q)
    case(ppa.BAD_QSL, total=T + 1)
    q = qsl.copy(); q[3] = q[2] - 1                      # a decreasing step
    case(ppa.BAD_QSL, qsl=q, max_q_len=1 << 20)
    case(ppa.BAD_QLEN, max_q_len=int(np.diff(qsl).max()) - 1)
    c = ctx.copy(); c[3] = -5
    assert case(ppa.BAD_CTX, ctx=c) == ppa.BAD_CTX
    b = bt.copy(); b[2, 0] = npages
    assert case(ppa.BAD_PAGE_ID, bt=b) == ppa.BAD_PAGE_ID
    b = bt.copy(); b[2, 0] = -1
    assert case(ppa.BAD_PAGE_ID, bt=b) == ppa.BAD_PAGE_ID
    c = ctx.copy(); c[1] = bt.shape[1] * P + 1            # more pages than a table row holds
    case(ppa.BAD_PAGES, ctx=c)
    c = ctx.copy(); c[0] = (1 << 24) + 1 - int(qsl[1] - qsl[0])  # L just past 2^24
    case(ppa.BAD_LENGTH, ctx=c)
    # entries at or beyond cdiv(ctx, P) are never read: junk there is fine
    s = int(np.argmin(ctx))
    need = -(-int(ctx[s]) // P)
    if need < bt.shape[1]:
        b = bt.copy(); b[s, need:] = 123456789
        assert run_check(qsl, ctx, b, P, npages, T, mq) == 0
    assert S == 8


def test_cache_sourced_mode_counts_every_position():
    import paged_kv_prefill_attention_amd as ppa
    w = make_config(1)
    qsl, ctx, bt, P, npages, T, mq = meta(w)
    # the block table covers the cached context only: cache-sourced mode needs cdiv(L, P) pages
    got = run_check(qsl, ctx, bt[:, :-(-int(ctx[0]) // P)], P, npages, T, mq, cache_only=True)
    assert got == ppa.BAD_PAGES
    assert run_check(qsl, ctx, bt, P, npages, T, mq, cache_only=True) == 0


def test_random_metadata_against_the_stated_preconditions():
    rng = np.random.default_rng(77)
    for _ in range(40):
        S = int(rng.integers(0, 12))
        P = int(rng.choice([1, 3, 16, 544]))
        n = rng.integers(-2, 40, size=S)
        qsl = np.concatenate([[0], np.cumsum(n)]).astype(np.int64)
        if rng.random() < 0.2:
            qsl[0] = int(rng.integers(-3, 3))
        T = int(qsl[-1]) + int(rng.integers(-1, 2) if rng.random() < 0.2 else 0)
        ctx = rng.integers(-3, 200, size=S)
        maxp = int(rng.integers(0, 12))
        npages = int(rng.integers(1, 64))
        bt = rng.integers(-2, npages + 2, size=(S, maxp))
        mq = int(rng.integers(0, 45))
        run_check(qsl, ctx, bt, P, npages, T, mq, cache_only=bool(rng.random() < 0.3))
