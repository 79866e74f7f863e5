"""Tile-loop bounds and useful-work count (test infrastructure only).

``tile_bounds_ref`` gives, for Q tile ``t`` of sequence ``s`` (``block_q``
query tokens per tile), the half-open range ``[lo, hi)`` of KV tiles of
``block_n`` keys that can hold an allowed key.  Steps, in the pages' order:

* query rows of the tile: from ``t * block_q`` up to the last row of the tile
  that exists (the last tile of a sequence is partial);
* base window: left edge ``a_lo - window_left`` when a left window is set, else
  key 0 (vLLM PR #50776 report, "Key source snippets": the first needed key is
  the tile's first query minus the left window, rounded down to a whole key
  block); right edge is the last query itself when causal, the last query plus
  ``window_right`` when a right window is set, otherwise the last key
  (same snippet, and vLLM PR #53147 report, "Review highlights": the
  non-causal right window must survive the multimodal branch);
* union with every valid multimodal range (start < end) that overlaps the
  tile's query positions: the left edge may move down to
  ``max(start, a_lo - window_left)`` and the right edge up to the range's
  inclusive end (vLLM PR #53147 report, "Key source snippets",
  compute_tile_loop_bounds, and "Implementation breakdown" item 2);
* clamp to ``[0, L-1]`` and convert to KV tiles: ``lo = first // block_n``,
  ``hi = last // block_n + 1``.

Variants (same report, same snippet): with chunked local attention the base
left edge is the chunk start ``(a_lo // chunk_size - chunk_lookback) *
chunk_size`` and a clamped multimodal range may still lower it (the
``minimum`` of the review fix); with unclamped multimodal ranges the range
start itself is the candidate left edge; with a causal flag per sequence the
right edge follows each sequence's flag.

Reading of the pages where they are loose: the left window edge (and the
chunk start) is taken from the tile's *lowest* query row (the printed helper
takes it from the highest row, which would drop keys that lower rows need);
the last, partial tile uses its last existing row; windows are inclusive
distances with -1 meaning unbounded.

``useful_pairs`` counts allowed (query, key) pairs with a per-row closed form:
every allowed set is one interval that contains the query's own position,
because the base window always holds ``j = a`` and every multimodal interval
of a query contains that query (``start <= a <= end``).
"""

from __future__ import annotations

import numpy as np


def _valid_ranges(ranges):
    return [(int(st), int(en)) for st, en in ranges if int(st) < int(en)]


def _is_chunked(chunk_size: int, chunk_lookback: int) -> bool:
    return chunk_size > 0 and chunk_lookback >= 0


def _causal_of(causal, s: int) -> bool:
    return bool(causal) if np.ndim(causal) == 0 else bool(np.asarray(causal)[s])


def tile_bounds_ref(c: int, n: int, t: int, block_q: int, block_n: int, causal: bool,
                    window_left: int, window_right: int, ranges, chunk_size: int = 0,
                    chunk_lookback: int = -1, mm_clamp: bool = True) -> tuple:
    """``(lo, hi)`` KV-tile range of Q tile ``t``; ``(0, 0)`` for a tile past the rows."""
    i_lo = t * block_q
    if i_lo >= n:
        return (0, 0)
    i_hi = min(i_lo + block_q - 1, n - 1)
    L = c + n
    a_lo, a_hi = c + i_lo, c + i_hi
    if _is_chunked(chunk_size, chunk_lookback):
        first = (a_lo // chunk_size - chunk_lookback) * chunk_size
    else:
        first = a_lo - window_left if window_left >= 0 else 0
    if causal:
        last = a_hi
    elif window_right >= 0:
        last = a_hi + window_right
    else:
        last = L - 1
    for st, en in _valid_ranges(ranges):
        if st <= a_hi and en >= a_lo:
            clamp = mm_clamp and window_left >= 0
            first = min(first, max(st, a_lo - window_left) if clamp else st)
            last = max(last, en)
    first = max(first, 0)
    last = min(last, L - 1)
    return (first // block_n, last // block_n + 1)


def tile_bounds_all(ctx_lens, q_lens, block_q: int, block_n: int, causal,
                    window_left: int, window_right: int, mm_ranges, num_q_tiles=None,
                    chunk_size: int = 0, chunk_lookback: int = -1, mm_clamp: bool = True):
    """int32 [S, num_q_tiles, 2]; tiles past a sequence's rows are (0, 0).
    ``causal`` is one flag or one flag per sequence."""
    ctx_lens = np.asarray(ctx_lens)
    q_lens = np.asarray(q_lens)
    S = len(ctx_lens)
    if num_q_tiles is None:
        mx = int(q_lens.max()) if S else 0
        num_q_tiles = -(-mx // block_q)
    out = np.zeros((S, num_q_tiles, 2), dtype=np.int32)
    for s in range(S):
        ranges = [] if mm_ranges is None else [tuple(r) for r in np.asarray(mm_ranges)[s]]
        for t in range(num_q_tiles):
            out[s, t] = tile_bounds_ref(int(ctx_lens[s]), int(q_lens[s]), t, block_q,
                                        block_n, _causal_of(causal, s), window_left,
                                        window_right, ranges, chunk_size, chunk_lookback,
                                        mm_clamp)
    return out


def row_intervals(c: int, n: int, causal: bool, window_left: int, window_right: int,
                  ranges, chunk_size: int = 0, chunk_lookback: int = -1,
                  mm_clamp: bool = True):
    """Closed form of each row's allowed keys: int64 arrays ``lo, hi`` (inclusive)."""
    L = c + n
    a = c + np.arange(n, dtype=np.int64)
    if _is_chunked(chunk_size, chunk_lookback):
        lo = (a // chunk_size - chunk_lookback) * chunk_size
    else:
        lo = a - window_left if window_left >= 0 else np.zeros(n, dtype=np.int64)
    if causal:
        hi = a.copy()
    elif window_right >= 0:
        hi = a + window_right
    else:
        hi = np.full(n, L - 1, dtype=np.int64)
    lo = np.asarray(lo, dtype=np.int64).copy()
    for st, en in _valid_ranges(ranges):
        inside = (st <= a) & (a <= en)
        clamp = mm_clamp and window_left >= 0
        mm_lo = np.maximum(st, a - window_left) if clamp else np.full(n, st)
        lo = np.where(inside, np.minimum(lo, mm_lo), lo)
        hi = np.where(inside, np.maximum(hi, en), hi)
    return np.maximum(lo, 0), np.minimum(hi, L - 1)


def useful_pairs(ctx_lens, q_lens, causal, window_left: int, window_right: int,
                 mm_ranges, chunk_size: int = 0, chunk_lookback: int = -1,
                 mm_clamp: bool = True) -> int:
    """Allowed (query row, key) pairs summed over sequences, for ONE query head."""
    total = 0
    for s in range(len(ctx_lens)):
        ranges = [] if mm_ranges is None else [tuple(r) for r in np.asarray(mm_ranges)[s]]
        lo, hi = row_intervals(int(ctx_lens[s]), int(q_lens[s]), _causal_of(causal, s),
                               window_left, window_right, ranges, chunk_size,
                               chunk_lookback, mm_clamp)
        total += int(np.maximum(hi - lo + 1, 0).sum())
    return total


def useful_flops(ctx_lens, q_lens, num_heads: int, head_size: int, causal,
                 window_left: int, window_right: int, mm_ranges, chunk_size: int = 0,
                 chunk_lookback: int = -1, mm_clamp: bool = True) -> int:
    """4 * head_size FLOP per allowed pair per query head (QK^T and PV, 2 each)."""
    return 4 * head_size * num_heads * useful_pairs(ctx_lens, q_lens, causal, window_left,
                                                    window_right, mm_ranges, chunk_size,
                                                    chunk_lookback, mm_clamp)
