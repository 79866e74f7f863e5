"""Dense reference for paged-KV prefill attention (test infrastructure only).

What is computed, for each sequence ``s`` with ``c = ctx_lens[s]`` cached
tokens and ``n = qsl[s+1] - qsl[s]`` new tokens (``L = c + n``), each query
head ``h`` and each new-token row ``i`` whose absolute position is
``a = c + i``:

1. Gather (vLLM PR #54194 report, "Features and motivation" and
   "Implementation breakdown" item 4): key position ``j < c`` lives in page
   ``block_table[s][j // P]`` at slot ``j % P`` of the cache; key position
   ``j >= c`` is new-token row ``qsl[s] + (j - c)`` of ``k_new``/``v_new``.
2. GQA/MQA: query head ``h`` reads KV head ``h // (H / Hkv)`` (contiguous
   groups; the pages name ``num_queries_per_kv`` without printing the map).
3. Scores ``scale * <q, k_j>`` in fp32.
4. Mask (vLLM PR #50776 report, "Features and motivation": keys within the
   distances ``window_left`` before and ``window_right`` after the query;
   vLLM PR #53147 report, "Implementation breakdown" item 2 and "Review
   highlights": the multimodal mask is ORed onto the base mask, a query inside
   an inclusive image range sees the whole range, clamped on the left to the
   window's left edge, and only ranges with start < end count).
5. Softmax over the allowed keys (max subtracted first), then the weighted sum
   of the gathered V rows.

Mask variants (vLLM PR #53147 report, "Key source snippets",
compute_tile_loop_bounds, and "Review highlights"):

* chunked local attention: with ``chunk_size > 0`` and ``chunk_lookback >= 0``
  the base window's left edge is the start of the chunk ``chunk_lookback``
  chunks before the query's own chunk, ``(a // chunk_size - chunk_lookback) *
  chunk_size``, in place of ``a - window_left``; a multimodal range is still
  clamped by ``window_left`` and so may re-admit keys before that edge;
* a causal flag per sequence (``causal`` given as a sequence of flags);
* unclamped multimodal ranges (``mm_clamp=False``): a query inside a range sees
  the whole range, with no left clamp by the window.

Split-KV (vLLM PR #53147 report, "Key source snippets": the segment arguments
of the tile-bound helper): the keys of a query are cut into contiguous
segments; each segment yields its own softmax statistics and normalised
partial output, and ``merge_partials`` combines them by the log-sum-exp rule.
"""

from __future__ import annotations

import numpy as np


def gather_kv(cache: np.ndarray, new, block_table: np.ndarray,
              query_start_loc: np.ndarray, ctx_lens: np.ndarray, s: int,
              page_size: int) -> np.ndarray:
    """Logical K (or V) of sequence ``s``: [L, Hkv, d], cached part then new part.

    With ``new=None`` (the cache-sourced mode, vLLM PR #54194 report,
    "Implementation breakdown" item 4) all ``L`` positions come from the cache.
    """
    c = int(ctx_lens[s])
    q0, q1 = int(query_start_loc[s]), int(query_start_loc[s + 1])
    from_cache = c if new is not None else c + (q1 - q0)
    rows = []
    for j in range(from_cache):
        page = int(block_table[s][j // page_size])
        rows.append(cache[page, j % page_size])
    cached = np.stack(rows) if rows else np.zeros((0,) + cache.shape[2:], cache.dtype)
    if new is None:
        return cached
    return np.concatenate([cached, new[q0:q1]], axis=0)


def chunked(chunk_size: int, chunk_lookback: int) -> bool:
    return chunk_size > 0 and chunk_lookback >= 0


def allowed_mask(c: int, n: int, causal: bool, window_left: int, window_right: int,
                 ranges, rows=None, chunk_size: int = 0, chunk_lookback: int = -1,
                 mm_clamp: bool = True) -> np.ndarray:
    """Boolean [len(rows), L] mask: row i (absolute position c+i) may attend key j.

    ``rows`` defaults to every new-token row ``0..n-1``.
    """
    L = c + n
    if rows is None:
        rows = np.arange(n, dtype=np.int64)
    a = (c + np.asarray(rows, dtype=np.int64))[:, None]
    j = np.arange(L, dtype=np.int64)[None, :]
    base = np.ones((a.shape[0], L), dtype=bool)
    if causal:
        base &= j <= a
    if chunked(chunk_size, chunk_lookback):
        base &= j >= (a // chunk_size - chunk_lookback) * chunk_size
    elif window_left >= 0:
        base &= j >= a - window_left
    if (not causal) and window_right >= 0:
        base &= j <= a + window_right
    mm = np.zeros((a.shape[0], L), dtype=bool)
    for st, en in ranges:
        if not st < en:
            continue  # a range counts only when start < end
        r = (st <= a) & (a <= en) & (st <= j) & (j <= en)
        if mm_clamp and window_left >= 0:
            r &= j >= a - window_left
        mm |= r
    return base | mm


def seq_causal(causal, s: int) -> bool:
    """The causal flag of sequence ``s``: one flag for all, or one per sequence."""
    if np.ndim(causal) == 0:
        return bool(causal)
    return bool(np.asarray(causal)[s])


def _seq_ranges(mm_ranges, s):
    if mm_ranges is None:
        return []
    return [(int(x), int(y)) for x, y in np.asarray(mm_ranges)[s]]


def reference_rows(q, k_new, v_new, k_cache, v_cache, block_table, query_start_loc,
                   ctx_lens, num_heads, num_kv_heads, head_size, page_size, window_left,
                   window_right, causal, mm_ranges, scale, s, rows, heads=None,
                   key_range=None, dtype=np.float32, return_probs=False, kv=None,
                   chunk_size=0, chunk_lookback=-1, mm_clamp=True, return_stats=False):
    """Attention output of sequence ``s`` for local query ``rows`` (indices into
    the sequence's new tokens) and query ``heads``: [len(rows), len(heads), d].

    ``key_range=(lo, hi)`` restricts the keys considered to ``[lo, hi)`` (used
    to show that pruning to the tile bounds changes nothing, and to form
    split-KV segments); the mask is still the full dense mask.  A row with no
    allowed key in the range gets output 0 (only possible for a segment).
    ``return_stats`` also returns, per row and head, the max scaled score ``m``
    (-inf when no key is allowed) and ``l = sum exp(score - m)``.
    """
    H, Hkv = num_heads, num_kv_heads
    group = H // Hkv
    c = int(ctx_lens[s])
    n = int(query_start_loc[s + 1] - query_start_loc[s])
    rows = np.asarray(rows, dtype=np.int64)
    if heads is None:
        heads = range(H)
    heads = list(heads)
    if kv is None:
        kv = (gather_kv(k_cache, k_new, block_table, query_start_loc, ctx_lens, s,
                        page_size).astype(dtype),
              gather_kv(v_cache, v_new, block_table, query_start_loc, ctx_lens, s,
                        page_size).astype(dtype))
    K, V = kv
    mask = allowed_mask(c, n, seq_causal(causal, s), window_left, window_right,
                        _seq_ranges(mm_ranges, s), rows=rows, chunk_size=chunk_size,
                        chunk_lookback=chunk_lookback, mm_clamp=mm_clamp)
    if key_range is not None:
        lo, hi = key_range
        keep = np.zeros(mask.shape[1], dtype=bool)
        keep[lo:hi] = True
        K, V, mask = K[keep], V[keep], mask[:, keep]
    qs = q[int(query_start_loc[s]) + rows].astype(dtype)
    out = np.zeros((len(rows), len(heads), head_size), dtype=dtype)
    m_out = np.full((len(rows), len(heads)), -np.inf, dtype=dtype)
    l_out = np.zeros((len(rows), len(heads)), dtype=dtype)
    probs = []
    any_key = mask.any(axis=1)
    for hi_, h in enumerate(heads):
        g = h // group
        scores = (qs[:, h, :] @ K[:, g, :].T) * dtype(scale)
        scores = np.where(mask, scores, -np.inf)
        m = np.where(any_key, scores.max(axis=1, initial=-np.inf), 0.0).astype(dtype)
        p = np.exp(scores - m[:, None])
        l = p.sum(axis=1)
        p = p / np.where(any_key, l, 1.0)[:, None]
        out[:, hi_, :] = p @ V[:, g, :]
        m_out[:, hi_] = np.where(any_key, m, -np.inf)
        l_out[:, hi_] = l
        if return_probs:
            probs.append(p)
    if return_stats:
        return out, m_out, l_out
    if return_probs:
        return out, probs
    return out


def merge_partials(outs, ms, ls):
    """Combine split-KV segments: each segment k holds its normalised output
    ``O_k``, max ``m_k`` and sum ``l_k``.  The whole-range result is
    ``sum_k w_k O_k / sum_k w_k`` with ``w_k = l_k * exp(m_k - M)``,
    ``M = max_k m_k`` (segments with no allowed key have ``l_k = 0``)."""
    outs = np.asarray(outs, dtype=np.float64)
    ms = np.asarray(ms, dtype=np.float64)
    ls = np.asarray(ls, dtype=np.float64)
    M = ms.max(axis=0)
    w = np.where(ls > 0, ls * np.exp(ms - np.where(np.isfinite(M), M, 0.0)), 0.0)
    return (w[..., None] * outs).sum(axis=0) / w.sum(axis=0)[..., None]


def reference_prefill(q, k_new, v_new, k_cache, v_cache, block_table, query_start_loc,
                      ctx_lens, num_heads, num_kv_heads, head_size, page_size,
                      window_left, window_right, causal, mm_ranges, scale,
                      dtype=np.float32, row_chunk=512, chunk_size=0, chunk_lookback=-1,
                      mm_clamp=True):
    """Full output [T, H, d] (fp32): every new-token row of every sequence."""
    T = int(query_start_loc[-1])
    out = np.zeros((T, num_heads, head_size), dtype=dtype)
    for s in range(len(ctx_lens)):
        n = int(query_start_loc[s + 1] - query_start_loc[s])
        q0 = int(query_start_loc[s])
        kv = (gather_kv(k_cache, k_new, block_table, query_start_loc, ctx_lens, s,
                        page_size).astype(dtype),
              gather_kv(v_cache, v_new, block_table, query_start_loc, ctx_lens, s,
                        page_size).astype(dtype))
        for r0 in range(0, n, row_chunk):
            rows = np.arange(r0, min(n, r0 + row_chunk))
            out[q0 + rows] = reference_rows(
                q, k_new, v_new, k_cache, v_cache, block_table, query_start_loc,
                ctx_lens, num_heads, num_kv_heads, head_size, page_size, window_left,
                window_right, causal, mm_ranges, scale, s, rows, dtype=dtype, kv=kv,
                chunk_size=chunk_size, chunk_lookback=chunk_lookback, mm_clamp=mm_clamp)
    return out
