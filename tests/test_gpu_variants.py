"""GPU parity of the mask variants and split-KV (prefill_attention_ex) against the oracle.

Bar as for the base path: |gpu - oracle| <= 2e-2 + 2e-2 * |oracle| elementwise;
tile bounds bit-exact against the oracle's integer formula.
"""

import numpy as np
import pytest

import oracle
from tests.harness import (compare, oracle_full, oracle_rows, out_to_f32, run_gpu,
                           sample_rows, to_device)
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    import paged_kv_prefill_attention_amd as ppa
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    ppa.load_library()


PAGES = [1, 7, 16, 544, 1040]
HEADS = [(4, 4), (8, 2), (8, 1), (6, 3), (16, 16)]


def variant_workload(rng, i, big=False):
    S = int(rng.integers(1, 5))
    H, Hkv = HEADS[int(rng.integers(0, len(HEADS)))]
    d = int(rng.choice([64, 128, 256]))
    P = int(rng.choice(PAGES))
    ctx = rng.integers(0, 1500 if big else 600, size=S)
    new = rng.integers(1, 700 if big else 300, size=S)
    wl = int(rng.choice([-1, 0, 40, 200]))
    wr = int(rng.choice([-1, 0, 64]))
    cs = int(rng.choice([0, 16, 64, 100, 256]))
    lb = int(rng.choice([-1, 0, 1, 3]))
    per_seq = rng.integers(0, 2, size=S) if rng.random() < 0.5 else None
    mm = None
    if rng.random() < 0.5:
        R = int(rng.integers(1, 5))
        mm = np.zeros((S, R, 2), dtype=np.int32)
        for s in range(S):
            L = int(ctx[s] + new[s])
            for r in range(R):
                st = int(rng.integers(0, L + 10))
                mm[s, r] = (st, st + int(rng.choice([0, 5, 60, 250, 500])))
    return make_workload(seed=12000 + i, ctx_lens=ctx, q_lens=new, num_heads=H,
                         num_kv_heads=Hkv, head_size=d, page_size=P,
                         causal=bool(rng.integers(0, 2)), window_left=wl, window_right=wr,
                         mm_ranges=mm, causal_per_seq=per_seq,
                         mm_clamp=bool(rng.integers(0, 2)), chunk_size=cs, chunk_lookback=lb,
                         name="variant%d" % i)


def describe(w):
    return ("%s d=%d H=%d/%d P=%d causal=%s per_seq=%s wl=%d wr=%d chunk=%d/%d clamp=%s R=%d" % (
        w.name, w.head_size, w.num_heads, w.num_kv_heads, w.page_size, w.causal,
        None if w.causal_per_seq is None else w.causal_per_seq.tolist(), w.window_left,
        w.window_right, w.chunk_size, w.chunk_lookback, w.mm_clamp, w.max_mm_ranges))


@pytest.mark.parametrize("chunk", range(4))
def test_mask_variants_full_outputs(chunk):
    """40 random ragged batches over chunked local attention, per-sequence causal flags
    and clamped / unclamped multimodal ranges."""
    rng = np.random.default_rng(6060 + chunk)
    for i in range(10):
        w = variant_workload(rng, chunk * 10 + i)
        print(describe(w), flush=True)
        compare(out_to_f32(run_gpu(w)), oracle_full(w), w.name)


def test_variant_tile_bounds_bitexact():
    import torch
    import paged_kv_prefill_attention_amd as ppa
    rng = np.random.default_rng(7171)
    for i in range(60):
        w = variant_workload(rng, 200 + i)
        dev = to_device(w)
        got = ppa.tile_bounds(dev["query_start_loc"], dev["ctx_lens"], w.num_heads,
                              w.num_kv_heads, w.head_size, w.window_left, w.window_right,
                              w.causal, dev["mm_ranges"], w.max_q_len,
                              causal_per_seq=dev["causal_per_seq"], mm_clamp=w.mm_clamp,
                              chunk_size=w.chunk_size, chunk_lookback=w.chunk_lookback)
        torch.cuda.synchronize()
        bq, bn = ppa.tile_config(w.head_size, w.num_heads, w.num_kv_heads, w.num_seqs,
                                 w.max_q_len,
                                 window_left=w.window_left, window_right=w.window_right,
                                 causal=w.causal)
        ref = oracle.tile_bounds_all(w.ctx_lens, w.q_lens, bq, bn, w.causal_arg,
                                     w.window_left, w.window_right, w.mm_ranges,
                                     **w.mask_kwargs())
        assert np.array_equal(got.cpu().numpy(), ref), describe(w)


@pytest.mark.parametrize("splits", [2, 3, 8, 0])
def test_split_kv_full_outputs(splits):
    """Split-KV segments merged by log-sum-exp match the oracle, including segments that
    are empty for some tiles (more splits than KV tiles)."""
    rng = np.random.default_rng(8080 + splits)
    for i in range(6):
        w = variant_workload(rng, 400 + 10 * splits + i, big=True)
        print(describe(w), "splits", splits, flush=True)
        compare(out_to_f32(run_gpu(w, kv_splits=splits)), oracle_full(w),
                "%s splits=%d" % (w.name, splits))


def test_split_kv_long_context_short_chunk():
    """The split-KV workload shape: two sequences with 32k cached tokens and a 256-token
    chunk (few Q tiles); sampled rows against the oracle, automatic split count."""
    import paged_kv_prefill_attention_amd as ppa
    w = make_workload(seed=515, ctx_lens=[32768, 30000], q_lens=[256, 200], num_heads=32,
                      num_kv_heads=8, head_size=128, page_size=16, causal=True,
                      name="long_ctx_short_chunk")
    k = ppa.split_count(w.head_size, w.num_heads, w.num_kv_heads, w.num_seqs,
                        w.total_q_tokens, w.max_q_len, 0,
                        window_left=w.window_left, window_right=w.window_right, causal=w.causal)
    assert k > 1
    out = out_to_f32(run_gpu(w, kv_splits=0))
    bq, _ = ppa.tile_config(w.head_size, w.num_heads, w.num_kv_heads)
    rng = np.random.default_rng(3)
    for s in range(w.num_seqs):
        rows = sample_rows(int(w.q_lens[s]), bq, rng)
        q0 = int(w.query_start_loc[s])
        compare(out[q0 + rows], oracle_rows(w, s, rows), "long ctx seq %d" % s)


def test_chunked_local_attention_long_sequence():
    """Chunked local attention at length: 12k new tokens after 4k cached, chunks of 2048
    with one chunk of lookback, plus clamped multimodal ranges that reach back over a
    chunk edge; sampled rows on every chunk edge."""
    import paged_kv_prefill_attention_amd as ppa
    mm = np.array([[[1500, 2600], [6000, 6100], [9000, 11000], [0, 0]]], dtype=np.int32)
    w = make_workload(seed=616, ctx_lens=[4096], q_lens=[12288], num_heads=8, num_kv_heads=2,
                      head_size=128, page_size=64, causal=True, window_left=1500,
                      mm_ranges=mm, chunk_size=2048, chunk_lookback=1, name="chunked_16k")
    out = out_to_f32(run_gpu(w))
    rows = np.unique(np.concatenate([
        np.arange(0, 12288, 397),
        np.array([e - 4096 + o for e in range(4096, 16384, 2048) for o in (-1, 0, 1)
                  if 0 <= e - 4096 + o < 12288])]))
    compare(out[rows], oracle_rows(w, 0, rows), w.name)
    bq, bn = ppa.tile_config(w.head_size, w.num_heads, w.num_kv_heads, w.num_seqs, w.max_q_len,
                             window_left=w.window_left, window_right=w.window_right,
                             causal=w.causal)
    dev = to_device(w)
    got = ppa.tile_bounds(dev["query_start_loc"], dev["ctx_lens"], w.num_heads, w.num_kv_heads,
                          w.head_size, w.window_left, w.window_right, w.causal,
                          dev["mm_ranges"], w.max_q_len, chunk_size=w.chunk_size,
                          chunk_lookback=w.chunk_lookback)
    ref = oracle.tile_bounds_all(w.ctx_lens, w.q_lens, bq, bn, w.causal, w.window_left,
                                 w.window_right, w.mm_ranges, **w.mask_kwargs())
    assert np.array_equal(got.cpu().numpy(), ref)


def test_variants_negative_controls():
    """Each variant changes the output where the pages say it should."""
    base = dict(seed=717, ctx_lens=[300, 80], q_lens=[200, 150], num_heads=4, num_kv_heads=2,
                head_size=64, page_size=16, causal=True)
    plain = out_to_f32(run_gpu(make_workload(**base)))
    chunked = out_to_f32(run_gpu(make_workload(**base, chunk_size=64, chunk_lookback=0)))
    assert np.abs(chunked - plain).max() > 0.05
    mixed = out_to_f32(run_gpu(make_workload(**base, causal_per_seq=[1, 0])))
    assert np.array_equal(mixed[:200], plain[:200])
    assert np.abs(mixed[200:] - plain[200:]).max() > 0.05
    mm = np.array([[[100, 400]], [[0, 0]]], dtype=np.int32)
    clamped = out_to_f32(run_gpu(make_workload(**base, window_left=20, mm_ranges=mm)))
    unclamped = out_to_f32(run_gpu(make_workload(**base, window_left=20, mm_ranges=mm,
                                                 mm_clamp=False)))
    assert np.abs(clamped - unclamped).max() > 0.05


def test_split_kv_rejects_missing_workspace():
    import torch
    import paged_kv_prefill_attention_amd as ppa
    w = make_workload(seed=1, ctx_lens=[100], q_lens=[10], num_heads=2, num_kv_heads=2,
                      head_size=64, page_size=16, causal=True)
    dev = to_device(w)
    lib = ppa.load_library()
    import ctypes
    out = torch.empty_like(dev["q"])
    P = ctypes.c_void_p
    rc = lib.prefill_attention_ex(
        P(dev["q"].data_ptr()), P(dev["k_new"].data_ptr()), P(dev["v_new"].data_ptr()),
        P(dev["k_cache"].data_ptr()), P(dev["v_cache"].data_ptr()),
        P(dev["block_table"].data_ptr()), P(dev["query_start_loc"].data_ptr()),
        P(dev["ctx_lens"].data_ptr()), 2, 2, 64, 16, -1, -1, 1, None, 0.125,
        P(out.data_ptr()), 1, 10, 10, int(w.num_pages), int(w.block_table.shape[1]), 0,
        None, 1, 0, -1, 4, None, 0, None)
    assert rc == ppa.ERR_INVALID_ARG


@pytest.mark.parametrize("d,heads", [(128, (4, 4)), (64, (4, 4)), (128, (2, 1)), (256, (4, 4))])
@pytest.mark.parametrize("splits", [1, 3])
def test_short_last_tiles_split_kv_tiles_between_halves(d, heads, splits):
    """Short last Q tiles (at most half the tile's rows valid, two or more KV tiles):
    the two halves of the workgroup take alternate KV tiles and are merged at the end.
    Lengths straddle the half- and quarter-tile boundaries and include one-token chunks;
    causal, windowed and bidirectional masks; whole outputs against the oracle."""
    import paged_kv_prefill_attention_amd as ppa
    H, Hkv = heads
    bq, _ = ppa.tile_config(d, H, Hkv)
    half = bq // 2
    qtr = bq // 4
    q_lens = [1, half - 1, half, half + 1, bq + half, 2 * bq + 7, qtr - 1, qtr, qtr + 1]
    ctx = [700, 64, 1, 333, 900, 0, 520, 3, 1200]
    for i, (causal, wl, wr) in enumerate([(True, -1, -1), (True, 100, -1), (False, 80, 40)]):
        w = make_workload(seed=9100 + 10 * i + splits, ctx_lens=ctx, q_lens=q_lens,
                          num_heads=H, num_kv_heads=Hkv, head_size=d, page_size=16,
                          causal=causal, window_left=wl, window_right=wr,
                          name="short_tiles_%d" % i)
        print(describe(w), "splits", splits, flush=True)
        compare(out_to_f32(run_gpu(w, kv_splits=splits)), oracle_full(w),
                "%s splits=%d" % (w.name, splits))


@pytest.mark.parametrize("d,n,causal,wl,wr,note", [
    (128, 256 * 66, True, 511, -1, "528 items: last 16 split"),
    (64, 128 * 258, False, 64, 64, "2064 items, four workgroups per CU: last 16 split"),
])
def test_tail_splitting_automatic(d, n, causal, wl, wr, note):
    """Automatic split count on batches of two to four rounds of items: the kernel cuts
    only the items of a short last round (the first Q tiles of the sequence, since the
    last Q tile goes first) into segments run by helper slots, merged by log-sum-exp.
    Every row of those first Q tiles is checked, plus sampled rows elsewhere."""
    import paged_kv_prefill_attention_amd as ppa
    w = make_workload(seed=7100 + d + n % 97, ctx_lens=[0], q_lens=[n], num_heads=8,
                      num_kv_heads=8, head_size=d, page_size=16, causal=causal,
                      window_left=wl, window_right=wr, name="tail_%d_%d" % (d, n))
    print(w.name, note, flush=True)
    assert ppa.split_count(d, 8, 8, 1, n, n, 0, window_left=wl, window_right=wr,
                           causal=causal) == 4
    out = out_to_f32(run_gpu(w, kv_splits=0))
    bq, _ = ppa.tile_config(d, 8, 8)
    first = np.arange(0, 2 * bq)
    compare(out[first], oracle_rows(w, 0, first), "%s first Q tiles" % w.name)
    rows = sample_rows(n, bq, np.random.default_rng(d), extra=24)
    compare(out[rows], oracle_rows(w, 0, rows), "%s sampled rows" % w.name)


def test_tail_splitting_config5():
    """The window-clamped multimodal prefix workload (784 items of near-equal length) in
    the automatic mode: its last 16 items, Q tiles 0 and 1 of every KV head, are split."""
    import paged_kv_prefill_attention_amd as ppa
    from workloads import make_config
    w = make_config(5)
    assert ppa.split_count(w.head_size, w.num_heads, w.num_kv_heads, w.num_seqs,
                           w.total_q_tokens, w.max_q_len, 0,
                           window_left=w.window_left, window_right=w.window_right,
                           causal=w.causal) == 4
    out = out_to_f32(run_gpu(w, kv_splits=0))
    bq, _ = ppa.tile_config(w.head_size, w.num_heads, w.num_kv_heads)
    first = np.arange(0, 2 * bq)
    compare(out[first], oracle_rows(w, 0, first), "config 5 first Q tiles")
    rows = sample_rows(int(w.q_lens[0]), bq, np.random.default_rng(5), extra=24)
    compare(out[rows], oracle_rows(w, 0, rows), "config 5 sampled rows")
