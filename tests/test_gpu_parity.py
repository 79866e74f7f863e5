"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bar: |gpu - oracle| <= 2e-2 + 2e-2 * |oracle| elementwise for bf16 outputs;
tile bounds bit-exact.  The full-size configurations run in the same launch
configuration as the benchmark: the headline ragged batch is compared on every
output element, the others on every head of every Q-tile edge row and every
multimodal-range boundary row; the small cases are compared on every output
element.
"""

import numpy as np
import pytest

import oracle
from tests.harness import (compare, edge_rows, oracle_full, oracle_rows, out_to_f32,
                           run_gpu, to_device)
from workloads import make_config, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    import paged_kv_prefill_attention_amd as ppa
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    ppa.load_library()


def tile_q(w):
    """(block_q, block_n) the library uses for this batch."""
    import paged_kv_prefill_attention_amd as ppa
    return ppa.tile_config(w.head_size, w.num_heads, w.num_kv_heads, w.num_seqs, w.max_q_len,
                           window_left=w.window_left, window_right=w.window_right, causal=w.causal)


def check_sampled(w, out, seed, cache_only=False, mm_ranges="default", rows_per_seq=None):
    """Compare every head of each sequence's edge rows (every Q-tile edge, every
    multimodal-range boundary, random rows) with the oracle."""
    bq, _ = tile_q(w)
    rng = np.random.default_rng(seed)
    worst = (0.0, 0.0)
    for s in range(w.num_seqs):
        n = int(w.q_lens[s])
        if n == 0:
            continue
        rows = edge_rows(w, s, bq, rng)
        q0 = int(w.query_start_loc[s])
        ref = oracle_rows(w, s, rows, cache_only=cache_only, mm_ranges=mm_ranges)
        e = compare(out[q0 + rows], ref, "%s seq %d" % (w.name, s))
        worst = (max(worst[0], e[0]), max(worst[1], e[1]))
    return worst


def test_config1_tiny_full():
    w = make_config(1)
    out = out_to_f32(run_gpu(w))
    compare(out, oracle_full(w), w.name)


def test_config2_full_outputs():
    """The headline ragged batch (8 sequences, 544-token pages, 64/64 heads, d=128),
    in the benchmark's launch configuration: every one of its 3317 x 64 output rows
    against the oracle."""
    w = make_config(2)
    out = out_to_f32(run_gpu(w))
    err = compare(out, oracle_full(w), w.name)
    print("%s (all rows) max_abs=%.3g max_rel=%.3g" % (w.name, err[0], err[1]), flush=True)


@pytest.mark.parametrize("cid,P", [(3, 1040), (3, 1056), (4, None), (5, None)],
                         ids=["c3_page1040", "c3_page1056", "c4_window", "c5_mm_prefix"])
def test_full_size_configs_edge_rows(cid, P):
    """Full-size configurations: every Q-tile edge row and, on the multimodal
    workload, the rows at st-1, st, en, en+1 of each of its 60 ranges."""
    w = make_config(cid, page_size=P)
    out = out_to_f32(run_gpu(w))
    assert np.isfinite(out).all()
    err = check_sampled(w, out, seed=cid)
    print("%s max_abs=%.3g max_rel=%.3g" % (w.name, err[0], err[1]), flush=True)


def test_config3_automatic_split_sampled():
    """The d=256 GQA batch under the automatic split count (two segments: its token count
    bounds it to 332 Q-tile items), in the launch configuration the suite times."""
    import paged_kv_prefill_attention_amd as ppa
    w = make_config(3, page_size=1040)
    k = ppa.split_count(w.head_size, w.num_heads, w.num_kv_heads, w.num_seqs,
                        w.total_q_tokens, w.max_q_len, 0,
                        window_left=w.window_left, window_right=w.window_right, causal=w.causal)
    assert k == 2
    out = out_to_f32(run_gpu(w, kv_splits=0))
    err = check_sampled(w, out, seed=33)
    print("%s auto split max_abs=%.3g max_rel=%.3g" % (w.name, err[0], err[1]), flush=True)


def test_config3_page_sizes_bitwise_equal():
    """Tiles never depend on pages: 1040 and 1056 give the same bits."""
    import torch
    a = run_gpu(make_config(3, page_size=1040))
    b = run_gpu(make_config(3, page_size=1056))
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_config5_negative_control_mm_ranges_matter():
    w = make_config(5)
    with_mm = out_to_f32(run_gpu(w))
    without = out_to_f32(run_gpu(w, mm_ranges=None))
    rows = np.arange(0, int(w.q_lens[0]), 97)
    assert np.abs(with_mm[rows] - without[rows]).max() > 0.05
    ref = oracle_rows(w, 0, rows, mm_ranges=None)
    compare(without[rows], ref, "config5 without ranges")


def test_deterministic_bitwise():
    import torch
    w = make_config(2)
    dev = to_device(w)
    a = run_gpu(w, dev=dev).clone()
    b = run_gpu(w, dev=dev)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


FUZZ_PAGES = [1, 7, 16, 128, 512, 544, 1040, 1056, 2048]
FUZZ_HEADS = [(4, 4), (8, 2), (8, 1), (6, 2), (16, 16), (12, 4), (64, 1), (3, 3)]


FUZZ_SIGMAS = [1.0, 1.0, 2.0, 3.0, 4.0]
FUZZ_SCALES = [1.0, 1.0, 0.5, 2.0]  # times 1/sqrt(d)


def fuzz_workload(rng, i, cache_only=False):
    """Random ragged batch ``i``: 1-4 sequences, page sizes 1..2048 (powers of two and
    not), head sizes 64/128/256, MHA/GQA/MQA, causal or not, windows, multimodal
    ranges.  Input magnitude (Q, K ~ N(0, sigma^2), sigma in 1..4) and the scale
    (0.5, 1 or 2 over sqrt(d)) come from a second stream seeded by ``i``."""
    S = int(rng.integers(1, 5))
    H, Hkv = FUZZ_HEADS[int(rng.integers(0, len(FUZZ_HEADS)))]
    d = int(rng.choice([64, 128, 256]))
    P = int(rng.choice(FUZZ_PAGES))
    ctx = rng.integers(0, 700, size=S)
    if rng.random() < 0.3:
        ctx[int(rng.integers(0, S))] = 0
    new = rng.integers(1, 300, size=S)
    causal = bool(rng.integers(0, 2))
    wl = int(rng.choice([-1, -1, 0, 5, 63, 64, 200]))
    wr = int(rng.choice([-1, 0, 17, 64, 300]))
    mm = None
    if rng.random() < 0.4:
        R = int(rng.integers(1, 5))
        mm = np.zeros((S, R, 2), dtype=np.int32)
        for s in range(S):
            L = int(ctx[s] + new[s])
            for r in range(R):
                st = int(rng.integers(0, L + 10))
                mm[s, r] = (st, st + int(rng.choice([0, 3, 40, 150, 400])))
    mrng = np.random.default_rng(50000 + i)
    sigma = float(mrng.choice(FUZZ_SIGMAS))
    scale = float(mrng.choice(FUZZ_SCALES)) / np.sqrt(d)
    return make_workload(seed=9000 + i, ctx_lens=ctx, q_lens=new, num_heads=H,
                         num_kv_heads=Hkv, head_size=d, page_size=P, causal=causal,
                         window_left=wl, window_right=wr, mm_ranges=mm,
                         new_in_cache=cache_only, name="fuzz%d" % i, qk_sigma=sigma,
                         scale=scale)


@pytest.mark.parametrize("chunk", range(60))
def test_fuzz_full_outputs(chunk):
    """600 random ragged batches (10 per chunk), whole outputs against the oracle:
    page sizes, head sizes, MHA/GQA/MQA, windows, ranges, input magnitudes and
    scales; every fourth batch in the cache-sourced mode (k_new = v_new = NULL)."""
    rng = np.random.default_rng(31337 + chunk)
    for i in range(10):
        idx = chunk * 10 + i
        cache_only = idx % 4 == 3
        w = fuzz_workload(rng, idx, cache_only=cache_only)
        print("fuzz case", idx, w.head_size, w.num_heads, w.num_kv_heads,
              w.page_size, w.causal, w.window_left, w.window_right,
              w.max_mm_ranges, "cache_only" if cache_only else "split",
              "scale=%.4g" % w.scale, flush=True)
        out = out_to_f32(run_gpu(w, cache_only=cache_only))
        compare(out, oracle_full(w, cache_only=cache_only), w.name)


@pytest.mark.parametrize("chunk", range(2))
def test_cache_sourced_mode(chunk):
    """k_new = v_new = NULL: every position comes through the block table; the bits
    equal those of the split mode on the same logical K/V."""
    import torch
    rng = np.random.default_rng(777 + chunk)
    for i in range(6):
        w = fuzz_workload(rng, 100 + chunk * 6 + i, cache_only=True)
        out = run_gpu(w, cache_only=True)
        compare(out_to_f32(out), oracle_full(w, cache_only=True), w.name + " cache-only")
        split = run_gpu(w)
        assert torch.equal(out.view(torch.int16), split.view(torch.int16))


def test_paging_invariance_bitwise():
    import torch
    outs = []
    for P, ts in [(16, 1), (16, 2), (544, 3), (1056, 4), (7, 5), (1, 6)]:
        w = make_workload(seed=4242, table_seed=ts, ctx_lens=[1500, 0, 613, 97],
                          q_lens=[300, 129, 64, 1], num_heads=8, num_kv_heads=2,
                          head_size=128, page_size=P, causal=True)
        outs.append(run_gpu(w).view(torch.int16).clone())
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_edge_cases():
    import torch
    # empty sequences between non-empty ones, a single-token sequence, context
    # that ends mid-page, page size 1
    for P in (1, 5, 16):
        w = make_workload(seed=17, ctx_lens=[33, 50, 0, 7, 0], q_lens=[0, 1, 130, 0, 2],
                          num_heads=4, num_kv_heads=2, head_size=64, page_size=P, causal=True)
        compare(out_to_f32(run_gpu(w)), oracle_full(w), "edge P=%d" % P)
    # zero windows, right-only window, degenerate and out-of-sequence ranges
    mm = np.array([[[5, 5], [40, 300], [2, 9]]], dtype=np.int32)
    for causal, wl, wr in [(False, 0, 0), (False, -1, 0), (False, 0, -1), (True, 0, -1),
                           (True, 3, -1), (False, 2, 1)]:
        w = make_workload(seed=18, ctx_lens=[20], q_lens=[150], num_heads=2, num_kv_heads=1,
                          head_size=128, page_size=16, causal=causal, window_left=wl,
                          window_right=wr, mm_ranges=mm)
        compare(out_to_f32(run_gpu(w)), oracle_full(w), "edge window %s" % ((causal, wl, wr),))
    # empty batch: nothing launched, output untouched
    import paged_kv_prefill_attention_amd as ppa
    dev = "cuda"
    q = torch.empty((0, 4, 64), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((1, 16, 2, 64), dtype=torch.bfloat16, device=dev)
    out = ppa.prefill_attention(q, q[:, :2], q[:, :2], kc, kc,
                                torch.zeros((0, 1), dtype=torch.int32, device=dev),
                                torch.zeros((1,), dtype=torch.int32, device=dev),
                                torch.zeros((0,), dtype=torch.int32, device=dev),
                                4, 2, 64, 16, -1, -1, True, None, 0.125, max_q_len=0)
    assert out.shape == (0, 4, 64)


def test_tile_bounds_bitexact():
    import torch
    import paged_kv_prefill_attention_amd as ppa
    cases = [make_config(c) for c in (1, 2, 4, 5)] + [make_config(3, page_size=1040)]
    rng = np.random.default_rng(55)
    for i in range(40):
        cases.append(fuzz_workload(rng, 500 + i))
    for w in cases:
        dev = to_device(w)
        got = ppa.tile_bounds(dev["query_start_loc"], dev["ctx_lens"], w.num_heads,
                              w.num_kv_heads, w.head_size, w.window_left, w.window_right,
                              w.causal, dev["mm_ranges"], w.max_q_len)
        torch.cuda.synchronize()
        bq, bn = tile_q(w)
        ref = oracle.tile_bounds_all(w.ctx_lens, w.q_lens, bq, bn, w.causal, w.window_left,
                                     w.window_right, w.mm_ranges)
        assert np.array_equal(got.cpu().numpy(), ref), w.name


@pytest.mark.parametrize("d", [64, 128])
def test_large_batch_without_sequence_sort(d):
    """More sequences than the workgroup sorts in LDS (256): the work decode reads the
    sequence table from memory and pads each (sequence, KV head) group to the
    longest tile count.  300 short ragged sequences, whole outputs."""
    rng = np.random.default_rng(4400 + d)
    S = 300
    ctx = rng.integers(0, 200, size=S)
    ctx[rng.integers(0, S, size=20)] = 0
    new = rng.integers(1, 60, size=S)
    w = make_workload(seed=4401 + d, ctx_lens=ctx, q_lens=new, num_heads=4, num_kv_heads=2,
                      head_size=d, page_size=16, causal=True, window_left=100,
                      name="batch300_d%d" % d)
    compare(out_to_f32(run_gpu(w)), oracle_full(w), w.name)


@pytest.mark.parametrize("d,ctx,page,bn", [(64, 5000, 1, 64), (128, 9000, 1, 64),
                                           (64, 7000, 3, 64), (64, 2000, 1, 64),
                                           (64, 2100, 1, 64), (64, 480, 1, 32),
                                           (64, 560, 1, 32)])
def test_block_table_beyond_lds_cache(d, ctx, page, bn):
    """A work item whose cached KV range covers more pages than the LDS block-table
    cache holds (4096 entries at d=128; at d=64, 2048 for the 64-key shape and 512 for
    the 32-key one; the cases at 2000/2100 and 480/560 cached tokens sit on either side
    of those limits): pages are read on the scalar unit, with copies that straddle
    page boundaries and the cache/new-token edge.  The 32-key cases use a batch of
    1024 Q-tile items under a 600-key window, which selects that shape.  Whole
    outputs, plain and split-KV."""
    if bn == 32:
        w = make_workload(seed=4600 + ctx, ctx_lens=[ctx, 40], q_lens=[1024, 1024],
                          num_heads=64, num_kv_heads=64, head_size=d, page_size=page,
                          causal=True, window_left=600, name="bt_fallback_many_%d" % ctx)
    else:
        w = make_workload(seed=4500 + d + page + ctx, ctx_lens=[ctx, 40], q_lens=[200, 30],
                          num_heads=2, num_kv_heads=1, head_size=d, page_size=page,
                          causal=True, name="bt_fallback_d%d_P%d_%d" % (d, page, ctx))
    assert tile_q(w)[1] == bn
    ref = oracle_full(w)
    compare(out_to_f32(run_gpu(w)), ref, w.name)
    compare(out_to_f32(run_gpu(w, kv_splits=3)), ref, w.name + " splits=3")


def d64_shape_case(name):
    """Batches on either side of the d=64 shape rule (32-key tiles for a window of at
    most 2048 keys per row with at least 1024 Q-tile items, or for 4096 items)."""
    rng = np.random.default_rng(4700 + len(name))
    if name == "four_rounds_causal":      # 32 x 8 tiles x 16 KV heads = 4096 items
        S = 32
        return make_workload(seed=4701, ctx_lens=rng.integers(0, 400, size=S),
                             q_lens=rng.integers(900, 1025, size=S), num_heads=16,
                             num_kv_heads=16, head_size=64, page_size=16, causal=True,
                             name=name), 32
    if name == "three_rounds_causal":     # 3072 items: long-loop shape
        S = 24
        return make_workload(seed=4702, ctx_lens=rng.integers(0, 400, size=S),
                             q_lens=rng.integers(900, 1025, size=S), num_heads=16,
                             num_kv_heads=16, head_size=64, page_size=16, causal=True,
                             name=name), 64
    if name == "window_one_round":        # 2 x 64 tiles x 8 = 1024 items, 1501 keys
        return make_workload(seed=4703, ctx_lens=[300, 0], q_lens=[8192, 8100], num_heads=8,
                             num_kv_heads=8, head_size=64, page_size=32, causal=True,
                             window_left=1500, name=name), 32
    if name == "window_below_round":      # 2 x 63 x 8 = 1008 items
        return make_workload(seed=4704, ctx_lens=[300, 0], q_lens=[8064, 8000], num_heads=8,
                             num_kv_heads=8, head_size=64, page_size=32, causal=True,
                             window_left=1500, name=name), 64
    if name == "window_past_span":        # 1024 items, 2049 keys per row
        return make_workload(seed=4705, ctx_lens=[300, 0], q_lens=[8192, 8100], num_heads=8,
                             num_kv_heads=8, head_size=64, page_size=32, causal=True,
                             window_left=2048, name=name), 64
    if name == "bidirectional_window":    # GQA 16/8 (64-token tiles): 2 x 64 x 8 items
        return make_workload(seed=4706, ctx_lens=[0, 77], q_lens=[4096, 4001], num_heads=16,
                             num_kv_heads=8, head_size=64, page_size=16, causal=False,
                             window_left=300, window_right=200, name=name), 32
    raise KeyError(name)


@pytest.mark.parametrize("name", ["four_rounds_causal", "three_rounds_causal",
                                  "window_one_round", "window_below_round",
                                  "window_past_span", "bidirectional_window"])
def test_d64_shape_choice(name):
    """Both d=64 tile shapes on batches at the edges of the rule that picks them: the
    library reports the expected block_n, and every head of every Q-tile edge row and
    of random rows matches the oracle, unsplit and under the automatic split count."""
    w, bn = d64_shape_case(name)
    assert tile_q(w)[1] == bn, (name, tile_q(w))
    print(describe_case(w), "block_n", bn, flush=True)
    dev = to_device(w)
    plain = out_to_f32(run_gpu(w, dev=dev))
    auto = out_to_f32(run_gpu(w, dev=dev, kv_splits=0))
    rng = np.random.default_rng(4710)
    for s in range(w.num_seqs):
        rows = edge_rows(w, s, tile_q(w)[0], rng)
        q0 = int(w.query_start_loc[s])
        ref = oracle_rows(w, s, rows)
        compare(plain[q0 + rows], ref, "%s seq %d" % (w.name, s))
        compare(auto[q0 + rows], ref, "%s seq %d automatic split" % (w.name, s))


def describe_case(w):
    return "%s S=%d H=%d/%d tokens=%d causal=%s window=(%d,%d)" % (
        w.name, w.num_seqs, w.num_heads, w.num_kv_heads, w.total_q_tokens, w.causal,
        w.window_left, w.window_right)
