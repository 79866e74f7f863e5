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


def allowed_mask(c: int, n: int, causal: bool, window_left: int, window_right: int,
                 ranges, rows=None) -> np.ndarray:
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
    if window_left >= 0:
        base &= j >= a - window_left
    if (not causal) and window_right >= 0:
        base &= j <= a + window_right
    mm = np.zeros((a.shape[0], L), dtype=bool)
    for st, en in ranges:
        if not st < en:
            continue  # a range counts only when start < end
        r = (st <= a) & (a <= en) & (st <= j) & (j <= en)
        if window_left >= 0:
            r &= j >= a - window_left
        mm |= r
    return base | mm


def _seq_ranges(mm_ranges, s):
    if mm_ranges is None:
        return []
    return [(int(x), int(y)) for x, y in np.asarray(mm_ranges)[s]]


def reference_rows(q, k_new, v_new, k_cache, v_cache, block_table, query_start_loc,
                   ctx_lens, num_heads, num_kv_heads, head_size, page_size, window_left,
                   window_right, causal, mm_ranges, scale, s, rows, heads=None,
                   key_range=None, dtype=np.float32, return_probs=False, kv=None):
    """Attention output of sequence ``s`` for local query ``rows`` (indices into
    the sequence's new tokens) and query ``heads``: [len(rows), len(heads), d].

    ``key_range=(lo, hi)`` restricts the keys considered to ``[lo, hi)`` (used
    to show that pruning to the tile bounds changes nothing); the mask is still
    the full dense mask.
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
    mask = allowed_mask(c, n, causal, window_left, window_right,
                        _seq_ranges(mm_ranges, s), rows=rows)
    if key_range is not None:
        lo, hi = key_range
        keep = np.zeros(mask.shape[1], dtype=bool)
        keep[lo:hi] = True
        K, V, mask = K[keep], V[keep], mask[:, keep]
    qs = q[int(query_start_loc[s]) + rows].astype(dtype)
    out = np.zeros((len(rows), len(heads), head_size), dtype=dtype)
    probs = []
    for hi_, h in enumerate(heads):
        g = h // group
        scores = (qs[:, h, :] @ K[:, g, :].T) * dtype(scale)
        scores = np.where(mask, scores, -np.inf)
        scores = scores - scores.max(axis=1, keepdims=True)
        p = np.exp(scores)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, hi_, :] = p @ V[:, g, :]
        if return_probs:
            probs.append(p)
    if return_probs:
        return out, probs
    return out


def reference_prefill(q, k_new, v_new, k_cache, v_cache, block_table, query_start_loc,
                      ctx_lens, num_heads, num_kv_heads, head_size, page_size,
                      window_left, window_right, causal, mm_ranges, scale,
                      dtype=np.float32, row_chunk=512):
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
                window_right, causal, mm_ranges, scale, s, rows, dtype=dtype, kv=kv)
    return out
