"""Pin the oracle with invariants, closed forms and a library routine.

* softmax rows sum to one and put zero weight outside the mask;
* constant V returns the constant;
* with no paging and no context, causal / windowed / GQA attention equals
  torch's CPU ``scaled_dot_product_attention`` with masks built by
  ``torch.tril``/``torch.triu`` and heads expanded by ``repeat_interleave``;
* the output does not depend on the page size or the physical page order;
* windows wider than the sequence equal no window;
* negative controls: dropping the multimodal ranges changes the output,
  perturbing a used page changes it, perturbing an unused page does not.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_bits_to_f32, f32_to_bf16_bits, make_config, make_workload


def run(w, **over):
    args = dict(q=w.f32("q"), k_new=w.f32("k_new"), v_new=w.f32("v_new"),
                k_cache=w.f32("k_cache"), v_cache=w.f32("v_cache"),
                block_table=w.block_table, query_start_loc=w.query_start_loc,
                ctx_lens=w.ctx_lens, num_heads=w.num_heads, num_kv_heads=w.num_kv_heads,
                head_size=w.head_size, page_size=w.page_size, window_left=w.window_left,
                window_right=w.window_right, causal=w.causal, mm_ranges=w.mm_ranges,
                scale=w.scale)
    args.update(over)
    return oracle.reference_prefill(**args)


def small(seed=1, S=2, ctx=(20, 0), new=(30, 17), H=4, Hkv=2, d=16, P=8, causal=True,
          wl=-1, wr=-1, mm=None, **kw):
    return make_workload(seed=seed, ctx_lens=ctx[:S], q_lens=new[:S], num_heads=H,
                         num_kv_heads=Hkv, head_size=d, page_size=P, causal=causal,
                         window_left=wl, window_right=wr, mm_ranges=mm, **kw)


MODES = [
    dict(causal=True, wl=-1, wr=-1),
    dict(causal=True, wl=5, wr=-1),
    dict(causal=False, wl=-1, wr=-1),
    dict(causal=False, wl=4, wr=9),
    dict(causal=False, wl=-1, wr=3),
    dict(causal=True, wl=6, wr=-1, mm=np.array([[[3, 18], [25, 40]], [[0, 9], [0, 0]]])),
]


@pytest.mark.parametrize("mode", range(len(MODES)))
def test_softmax_rows_sum_to_one_and_respect_mask(mode):
    w = small(**MODES[mode])
    for s in range(w.num_seqs):
        n, c = int(w.q_lens[s]), int(w.ctx_lens[s])
        rows = np.arange(n)
        _, probs = oracle.reference_rows(
            w.f32("q"), w.f32("k_new"), w.f32("v_new"), w.f32("k_cache"), w.f32("v_cache"),
            w.block_table, w.query_start_loc, w.ctx_lens, w.num_heads, w.num_kv_heads,
            w.head_size, w.page_size, w.window_left, w.window_right, w.causal,
            w.mm_ranges, w.scale, s, rows, return_probs=True)
        mask = oracle.allowed_mask(c, n, w.causal, w.window_left, w.window_right,
                                   w.mm_list(s))
        for p in probs:
            assert np.abs(p.sum(axis=1) - 1.0).max() <= 1e-6
            assert (p[~mask] == 0).all()
            assert (p[mask] > 0).all()


@pytest.mark.parametrize("mode", range(len(MODES)))
def test_constant_v_returns_constant(mode):
    w = small(**MODES[mode])
    cval = np.float32(0.71875)  # exactly representable in bf16
    vn = np.full_like(w.f32("v_new"), cval)
    vc = np.full_like(w.f32("v_cache"), cval)
    out = run(w, v_new=vn, v_cache=vc)
    assert np.abs(out - cval).max() <= 1e-6


def sdpa_ref(q, k, v, mask, scale):
    """torch CPU fp32 SDPA; q [n,H,d], k/v [L,H,d], mask [n,L] bool."""
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None].contiguous()
    vt = torch.from_numpy(v).permute(1, 0, 2)[None].contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.from_numpy(mask) if mask is not None else None,
        scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def logical_kv(w, s=0):
    # identity paging with one page that holds the whole sequence -> new rows only
    q0, q1 = int(w.query_start_loc[s]), int(w.query_start_loc[s + 1])
    return w.f32("q")[q0:q1], w.f32("k_new")[q0:q1], w.f32("v_new")[q0:q1]


@pytest.mark.parametrize("H,Hkv", [(4, 4), (4, 2), (6, 1)])
def test_causal_no_context_equals_sdpa(H, Hkv):
    w = small(S=1, ctx=(0,), new=(37,), H=H, Hkv=Hkv, d=32, P=64)
    q, k, v = logical_kv(w)
    G = H // Hkv
    k = np.repeat(k, G, axis=1)
    v = np.repeat(v, G, axis=1)
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None].contiguous()
    vt = torch.from_numpy(v).permute(1, 0, 2)[None].contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, is_causal=True, scale=w.scale)[0].permute(1, 0, 2).numpy()
    out = run(w)
    assert np.abs(out - ref).max() <= 1e-5


def test_causal_with_context_equals_sdpa_bottom_right():
    """Context c>0: row i sits at position c+i (mask = tril with diagonal c)."""
    w = make_workload(seed=9, ctx_lens=[23], q_lens=[19], num_heads=2, num_kv_heads=2,
                      head_size=16, page_size=5, causal=True, new_in_cache=True)
    # the cache holds every position (new_in_cache) so the logical K/V is
    # available from pages; read it back independently of the oracle
    L = 42
    kc, vc = w.f32("k_cache"), w.f32("v_cache")
    k = np.stack([kc[w.block_table[0][j // 5], j % 5] for j in range(L)])
    v = np.stack([vc[w.block_table[0][j // 5], j % 5] for j in range(L)])
    mask = torch.ones(19, L, dtype=torch.bool).tril(23).numpy()
    ref = sdpa_ref(w.f32("q"), k, v, mask, w.scale)
    out = run(w)
    assert np.abs(out - ref).max() <= 1e-5
    # cache-sourced mode (no k_new/v_new) reads the same values from pages
    out2 = run(w, k_new=None, v_new=None)
    assert np.abs(out2 - ref).max() <= 1e-5


@pytest.mark.parametrize("wl,wr", [(3, 3), (0, 5), (7, 0), (2, 11)])
def test_noncausal_band_equals_sdpa(wl, wr):
    w = small(S=1, ctx=(0,), new=(41,), H=2, Hkv=1, d=16, P=64, causal=False, wl=wl, wr=wr)
    q, k, v = logical_kv(w)
    k = np.repeat(k, 2, axis=1)
    v = np.repeat(v, 2, axis=1)
    mask = torch.ones(41, 41, dtype=torch.bool).tril(wr).triu(-wl).numpy()
    ref = sdpa_ref(q, k, v, mask, w.scale)
    assert np.abs(run(w) - ref).max() <= 1e-5


def test_causal_window_equals_sdpa():
    w = small(S=1, ctx=(0,), new=(33,), H=2, Hkv=2, d=16, P=64, causal=True, wl=4)
    q, k, v = logical_kv(w)
    mask = torch.ones(33, 33, dtype=torch.bool).tril(0).triu(-4).numpy()
    assert np.abs(run(w) - sdpa_ref(q, k, v, mask, w.scale)).max() <= 1e-5


def test_paging_invariance_bitwise():
    """Same logical K/V at page sizes 16/544/1040/1056 and two table seeds."""
    outs = []
    for P, ts in [(16, 1), (16, 2), (544, 3), (1040, 4), (1056, 5), (7, 6)]:
        w = make_workload(seed=42, table_seed=ts, ctx_lens=[1200, 0, 613], q_lens=[5, 9, 4],
                          num_heads=2, num_kv_heads=1, head_size=16, page_size=P, causal=True)
        outs.append(run(w))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_config3_page_sizes_hold_same_logical_tensors():
    a = make_config(3, heads=(2, 1), page_size=1040)
    b = make_config(3, heads=(2, 1), page_size=1056)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k_new, b.k_new)
    assert not np.array_equal(a.block_table, b.block_table)
    rows = np.array([0, 5, 100])
    for s in (0, 3):
        oa = oracle.reference_rows(a.f32("q"), a.f32("k_new"), a.f32("v_new"),
                                   a.f32("k_cache"), a.f32("v_cache"), a.block_table,
                                   a.query_start_loc, a.ctx_lens, 2, 1, 256, 1040, -1, -1,
                                   True, None, a.scale, s, rows)
        ob = oracle.reference_rows(b.f32("q"), b.f32("k_new"), b.f32("v_new"),
                                   b.f32("k_cache"), b.f32("v_cache"), b.block_table,
                                   b.query_start_loc, b.ctx_lens, 2, 1, 256, 1056, -1, -1,
                                   True, None, b.scale, s, rows)
        assert np.array_equal(oa, ob)


def test_window_wider_than_sequence_equals_no_window():
    base = small(causal=False, wl=-1, wr=-1)
    wide = small(causal=False, wl=500, wr=500)
    assert np.array_equal(run(base), run(wide))
    cbase = small(causal=True, wl=-1)
    cwide = small(causal=True, wl=500)
    assert np.array_equal(run(cbase), run(cwide))
    # non-causal with only a left window == right window unbounded
    a = small(causal=False, wl=4, wr=-1)
    b = small(causal=False, wl=4, wr=10_000)
    assert np.array_equal(run(a), run(b))


def test_negative_control_mm_ranges_matter():
    mm = np.array([[[2, 40]], [[0, 12]]])
    w = small(causal=True, wl=3, mm=mm)
    with_mm = run(w)
    without = run(w, mm_ranges=None)
    assert np.abs(with_mm - without).max() > 0.05


def test_negative_control_mm_ranges_matter_config5_shape():
    """Config-5-like geometry at a small size: window 1023 rows, 256-wide images."""
    rng = np.random.default_rng(3)
    offs = np.sort(rng.integers(0, 300, size=6))
    st = offs + 256 * np.arange(6)
    mm = np.stack([st, st + 255], -1)[None]
    w = make_workload(seed=11, ctx_lens=[300], q_lens=[1500], num_heads=2, num_kv_heads=1,
                      head_size=16, page_size=16, causal=True, window_left=1023,
                      mm_ranges=mm)
    rows = np.arange(0, 1500, 37)
    args = (w.f32("q"), w.f32("k_new"), w.f32("v_new"), w.f32("k_cache"), w.f32("v_cache"),
            w.block_table, w.query_start_loc, w.ctx_lens, 2, 1, 16, 16, 1023, -1, True)
    a = oracle.reference_rows(*args, w.mm_ranges, w.scale, 0, rows)
    b = oracle.reference_rows(*args, None, w.scale, 0, rows)
    assert np.abs(a - b).max() > 0.05


def test_negative_control_page_perturbation():
    w = small(S=2, ctx=(37, 11), new=(9, 6), P=8)
    ref = run(w)
    assert np.isfinite(ref).all()  # poison (NaN) slots are never read
    used = set(int(p) for p in w.block_table.reshape(-1) if p >= 0)
    unused = [p for p in range(w.num_pages) if p not in used]
    assert unused, "pool should have spare pages"
    kc = w.f32("k_cache").copy()
    kc[unused[0]] = 123.0
    assert np.array_equal(run(w, k_cache=kc), ref)
    kc = w.f32("k_cache").copy()
    kc[int(w.block_table[0][1]), 3, 0, 0] += 4.0
    assert np.abs(run(w, k_cache=kc) - ref).max() > 0.0


def test_bf16_rounding_matches_torch():
    vals = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, -2.5, 3.3e-5, 65504.0, 1e30, -0.0,
                     np.inf, 1.00000012], dtype=np.float32)
    rng = np.random.default_rng(0)
    vals = np.concatenate([vals, rng.standard_normal(10000, dtype=np.float32) * 100])
    ours = f32_to_bf16_bits(vals)
    theirs = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    assert np.array_equal(bf16_bits_to_f32(ours), torch.from_numpy(vals).to(
        torch.bfloat16).float().numpy())
