"""Shared helpers for the GPU tests: move a seeded workload to the device, call
the HIP library through its binding, and compare with the oracle."""

import numpy as np

import oracle
from workloads import bf16_bits_to_f32

ATOL = 2e-2
RTOL = 2e-2


def to_device(w, cache_only=False, device="cuda"):
    import torch

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(
            torch.bfloat16)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)

    return dict(q=bf(w.q), k_new=None if cache_only else bf(w.k_new),
                v_new=None if cache_only else bf(w.v_new), k_cache=bf(w.k_cache),
                v_cache=bf(w.v_cache), block_table=i32(w.block_table),
                query_start_loc=i32(w.query_start_loc), ctx_lens=i32(w.ctx_lens),
                mm_ranges=None if w.mm_ranges is None else i32(w.mm_ranges),
                causal_per_seq=None if w.causal_per_seq is None else i32(w.causal_per_seq))


def variant_kwargs(w, dev, kv_splits=1):
    """Keyword arguments of the binding for the workload's mask variant."""
    return dict(causal_per_seq=dev["causal_per_seq"], mm_clamp=w.mm_clamp,
                chunk_size=w.chunk_size, chunk_lookback=w.chunk_lookback, kv_splits=kv_splits)


def run_gpu(w, dev=None, cache_only=False, out=None, mm_ranges="default", kv_splits=1):
    import paged_kv_prefill_attention_amd as ppa
    if dev is None:
        dev = to_device(w, cache_only=cache_only)
    mm = dev["mm_ranges"] if isinstance(mm_ranges, str) else mm_ranges
    return ppa.prefill_attention(
        dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
        dev["block_table"], dev["query_start_loc"], dev["ctx_lens"], w.num_heads,
        w.num_kv_heads, w.head_size, w.page_size, w.window_left, w.window_right, w.causal,
        mm, w.scale, out=out, max_q_len=w.max_q_len, **variant_kwargs(w, dev, kv_splits))


def out_to_f32(out):
    import torch
    return bf16_bits_to_f32(out.view(torch.int16).cpu().numpy().view(np.uint16))


def oracle_rows(w, s, rows, heads=None, cache_only=False, mm_ranges="default"):
    mm = w.mm_ranges if isinstance(mm_ranges, str) else mm_ranges
    return oracle.reference_rows(
        w.f32("q"), None if cache_only else w.f32("k_new"),
        None if cache_only else w.f32("v_new"), w.f32("k_cache"), w.f32("v_cache"),
        w.block_table, w.query_start_loc, w.ctx_lens, w.num_heads, w.num_kv_heads,
        w.head_size, w.page_size, w.window_left, w.window_right, w.causal_arg, mm, w.scale, s,
        rows, heads=heads, **w.mask_kwargs())


def oracle_full(w, cache_only=False):
    return oracle.reference_prefill(
        w.f32("q"), None if cache_only else w.f32("k_new"),
        None if cache_only else w.f32("v_new"), w.f32("k_cache"), w.f32("v_cache"),
        w.block_table, w.query_start_loc, w.ctx_lens, w.num_heads, w.num_kv_heads,
        w.head_size, w.page_size, w.window_left, w.window_right, w.causal_arg, w.mm_ranges,
        w.scale, **w.mask_kwargs())


def compare(gpu, ref, what=""):
    """Assert |gpu - ref| <= ATOL + RTOL*|ref| elementwise; return (max_abs, max_rel)."""
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), "non-finite GPU output " + what
    err = np.abs(gpu.astype(np.float64) - ref.astype(np.float64))
    bound = ATOL + RTOL * np.abs(ref.astype(np.float64))
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d elements out of tolerance, max err %.4g, first %s" % (
            what, int(bad.sum()), float(err.max()), idx.tolist()))
    rel = err / np.maximum(np.abs(ref), 1e-6)
    return float(err.max()), float(rel[np.abs(ref) > 0.05].max() if (np.abs(ref) > 0.05).any()
                                   else 0.0)


def sample_rows(n, block_q, rng, extra=8):
    """Rows that span tiles and tails: first/last rows, tile edges, random ones."""
    cand = {0, n - 1, n // 2}
    for t in range(0, n, block_q):
        cand.update({t, min(n - 1, t + block_q - 1)})
    rows = sorted(r for r in cand if 0 <= r < n)
    if len(rows) > 24:
        rows = sorted(set(rng.choice(rows, 24, replace=False).tolist()) | {0, n - 1})
    rnd = rng.integers(0, n, size=min(extra, n)).tolist()
    return np.array(sorted(set(rows) | set(rnd)), dtype=np.int64)


def edge_rows(w, s, block_q, rng, extra=8):
    """Rows of sequence ``s`` to compare at full size, with no cap: the first,
    middle and last row, both edges (and the row after the first edge) of every
    Q tile, the rows at absolute positions st-1, st, en and en+1 of every
    multimodal range [st, en] that fall among the new tokens, and ``extra``
    random rows."""
    n, c = int(w.q_lens[s]), int(w.ctx_lens[s])
    cand = {0, n - 1, n // 2}
    for t in range(0, n, block_q):
        cand.update({t, t + 1, t + block_q - 1})
    for st, en in w.mm_list(s):
        cand.update(a - c for a in (st - 1, st, en, en + 1))
    cand.update(rng.integers(0, n, size=min(extra, n)).tolist())
    return np.array(sorted(r for r in cand if 0 <= r < n), dtype=np.int64)
