/*
 * paged_prefill.h — C ABI of the MI355X (gfx950) paged-KV prefill attention library.
 *
 * What the library computes (vLLM PR #54194 report, "Features and motivation"
 * and "Implementation breakdown"; vLLM PR #50776 report, "Features and
 * motivation"; vLLM PR #53147 report, "Implementation breakdown"):
 * for every sequence s of a ragged prefill batch, every query head h and every
 * new-token row i, the query at absolute position a = ctx_lens[s] + i attends
 * over the sequence's keys j in [0, L), L = ctx_lens[s] + n_s, where keys
 * j < ctx_lens[s] are read from a paged KV cache through the block table and
 * keys j >= ctx_lens[s] are the chunk's new K/V rows.  Scores are
 * scale * <q, k_j>; a key is allowed when j < L and
 *   (causal => j <= a) and (window_left >= 0 => j >= a - window_left) and
 *   (!causal and window_right >= 0 => j <= a + window_right),
 * or when some multimodal range [st, en] (inclusive, counted only if st < en)
 * holds both a and j and (window_left >= 0 => j >= a - window_left).
 * The output row is the softmax-weighted sum of the allowed V rows.
 * Query head h reads KV head h / (num_heads / num_kv_heads).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates no device memory and keeps no state between calls.  Every call
 *    is re-entrant and thread-safe (prefill_attention_ex_noalloc excepted: it
 *    uses the library's static scratch, see there).
 *  - bf16 tensors are passed as raw 16-bit patterns, dense, row-major.
 *  - Work is enqueued on `stream` (NULL = the default stream) and the call
 *    returns without synchronising.  A fault during execution surfaces at the
 *    caller's next synchronisation on that stream.
 *  - Scalar arguments are checked on the host; device-resident contents
 *    (lengths, page ids, ranges) are preconditions stated per argument and
 *    are not checked.  No C++ exception crosses this boundary.
 *  - Return value: PAGED_PREFILL_OK or one of the negative error codes below.
 */
#ifndef PAGED_PREFILL_H
#define PAGED_PREFILL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

#define PAGED_PREFILL_OK 0
#define PAGED_PREFILL_ERR_INVALID_ARG (-1) /* a null required pointer or an out-of-range scalar */
#define PAGED_PREFILL_ERR_UNSUPPORTED (-2) /* head_size not in {64, 128, 256}, or a size this build does not handle */
#define PAGED_PREFILL_ERR_HIP (-3)         /* the HIP runtime refused the launch */
#define PAGED_PREFILL_ERR_SCRATCH (-4)     /* split-KV partials beyond the static scratch (noalloc entry) */

/*
 * prefill_attention — one launch of paged-KV prefill attention over a ragged batch.
 *
 * Tensors (T = total_q_tokens, H = num_heads, Hkv = num_kv_heads, d = head_size,
 * P = page_size, S = num_seqs):
 *   q               bf16 [T][H][d]            queries of the new tokens, sequences packed
 *   k_new, v_new    bf16 [T][Hkv][d]          the chunk's new keys/values; row query_start_loc[s] + i
 *                                             is position ctx_lens[s] + i of sequence s.
 *                                             Both NULL selects the cache-sourced mode: every
 *                                             position j < L of a sequence is read from the cache
 *                                             (the new tokens are already written there), as in
 *                                             the k=None path of vLLM PR #54194 report,
 *                                             "Implementation breakdown" item 4.
 *   k_cache, v_cache bf16 [num_pages][P][Hkv][d]  paged cache; position j of sequence s lives in
 *                                             page block_table[s][j / P], slot j % P.  P may be
 *                                             any positive size, including non-powers of two
 *                                             (544, 1040, 1056; vLLM PR #54194 report, "Features
 *                                             and motivation"): tiles never depend on pages.
 *   block_table     int32 [S][max_pages_per_seq]; entry p must be a page id in [0, num_pages) for
 *                   p < cdiv(ctx_lens[s], P) (cdiv(L, P) in cache-sourced mode).  Entries at or
 *                   beyond that count are NEVER read and may hold anything (e.g. -1); pages not
 *                   named by a read entry are never touched (vLLM PR #54194 report, "Review
 *                   highlights": the unmasked block-table load hazard).
 *   query_start_loc int32 [S+1]; query_start_loc[0] = 0, non-decreasing, query_start_loc[S] = T.
 *   ctx_lens        int32 [S]; cached tokens per sequence, >= 0.
 *   mm_ranges       int32 [S][max_mm_ranges][2]; absolute, inclusive [start, end] multimodal
 *                   ranges (vLLM PR #53147 report, "Key source snippets": [seq][range][start,end]
 *                   layout, [0, 0] padding, valid only if start < end).  NULL iff max_mm_ranges==0.
 *   out             bf16 [T][H][d]; written for every new-token row (round-to-nearest-even from
 *                   fp32).  Must not alias an input.
 * Scalars:
 *   window_left     keys j >= a - window_left are allowed; -1 = unbounded.  Inclusive distance,
 *                   as the windowed-prefill report uses (vLLM PR #50776 report, "Features and
 *                   motivation"); a width-W window of the multimodal report is W - 1 here.
 *   window_right    keys j <= a + window_right are allowed when !causal; -1 = unbounded;
 *                   ignored when causal.
 *   causal          0 or 1; causal rows sit at their absolute position (bottom-right alignment).
 *   scale           softmax scale applied to q.k (e.g. 1/sqrt(d)); must be finite and > 0.
 *   max_q_len       >= every n_s = query_start_loc[s+1] - query_start_loc[s].
 *   num_pages, max_pages_per_seq, max_mm_ranges  sizes of the tensors above.
 * Errors: INVALID_ARG for a null required pointer, num_heads % num_kv_heads != 0, non-positive
 * sizes (page_size, num_heads, num_kv_heads; negative num_seqs/total_q_tokens/max_q_len),
 * window < -1, causal not 0/1, bad scale, exactly one of k_new/v_new NULL, max_mm_ranges < 0 or
 * > 4096, max_mm_ranges > 0 with NULL mm_ranges, or a geometry whose positions exceed the
 * library's 2^24-token limit per sequence; UNSUPPORTED for head_size not in {64, 128, 256};
 * HIP_ERROR if the launch fails.  An empty batch (num_seqs, total_q_tokens or max_q_len == 0)
 * returns OK without launching.
 */
int prefill_attention(const void* q, const void* k_new, const void* v_new,
                      const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* query_start_loc,
                      const int32_t* ctx_lens,
                      int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                      int32_t page_size, int32_t window_left, int32_t window_right,
                      int32_t causal, const int32_t* mm_ranges, float scale, void* out,
                      int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len,
                      int32_t num_pages, int32_t max_pages_per_seq, int32_t max_mm_ranges,
                      hipStream_t stream);

/*
 * prefill_attention_validate — the host-side argument checks of prefill_attention, alone.
 * Takes the same arguments, reads no pointer, launches nothing, needs no GPU.  Returns the
 * code prefill_attention would return before launching.
 */
int prefill_attention_validate(const void* q, const void* k_new, const void* v_new,
                               const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* query_start_loc,
                               const int32_t* ctx_lens,
                               int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                               int32_t page_size, int32_t window_left, int32_t window_right,
                               int32_t causal, const int32_t* mm_ranges, float scale,
                               const void* out, int32_t num_seqs, int32_t total_q_tokens,
                               int32_t max_q_len, int32_t num_pages, int32_t max_pages_per_seq,
                               int32_t max_mm_ranges);

/*
 * prefill_attention_tile_config — the tile geometry prefill_attention uses for this head
 * configuration: *block_q query tokens per Q tile (all heads of a GQA group share a tile) and
 * *block_n keys per KV tile.  The tile bounds below are expressed in these units.  Host-only.
 * The geometry never depends on the page size: query rows and KV columns of a tile never index
 * the paged cache, each key is resolved to its page on its own (vLLM PR #54194 report,
 * "Features and motivation", "Implementation breakdown" items 1-2 and "Key source snippets":
 * the tile selection of context_attention_fwd decoupled from pages).  The shapes themselves
 * are chosen per head size by measurement on gfx950, not the report's 128/64.  At head size 64
 * block_n also depends on the batch (prefill_attention_tile_config_ex); this form gives the
 * geometry of a small batch, exact for every other head size.
 * Errors: INVALID_ARG (null outputs, bad head counts), UNSUPPORTED (head_size).
 */
int prefill_attention_tile_config(int32_t head_size, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t* block_q, int32_t* block_n);

/*
 * prefill_attention_tile_config_ex — the tile geometry for a batch of num_seqs sequences of at
 * most max_q_len new tokens under the window (window_left, window_right, causal as for
 * prefill_attention), as prefill_attention, prefill_attention_tile_bounds and
 * prefill_attention_kv_splits choose it.  Only head size 64 depends on the batch: with I the
 * Q-tile work items (num_seqs * cdiv(max_q_len, block_q) per KV head and head block) and S the
 * workgroups the GPU holds of the 32-key shape (four per CU), block_n is 32 when the window
 * alone limits a query row to at most 2048 keys (window_left + 1 when causal, window_left + 1
 * + window_right otherwise) and I >= S, or when I >= 4 S; otherwise block_n is 64.  Multimodal
 * ranges and the mask options of prefill_attention_ex do not enter the choice.  block_q is the
 * same either way.  num_seqs = max_q_len = 0 gives prefill_attention_tile_config's answer.
 * Host-only (it asks the runtime for the current device's CU count).  Errors as for
 * prefill_attention_tile_config, plus INVALID_ARG for negative sizes, a window below -1 or
 * causal not 0/1.
 */
int prefill_attention_tile_config_ex(int32_t head_size, int32_t num_heads, int32_t num_kv_heads,
                                     int32_t num_seqs, int32_t max_q_len, int32_t window_left,
                                     int32_t window_right, int32_t causal, int32_t* block_q,
                                     int32_t* block_n);

/*
 * prefill_attention_tile_bounds — the KV-tile loop range [lo, hi) of every Q tile, computed on
 * the GPU by the same device function the attention kernel loops with (the helper-kernel test
 * pattern of vLLM PR #53147 report, "Key source snippets").  The range unions the base window
 * with every valid multimodal range that overlaps the tile's query positions, clamps to the
 * sequence, and converts to tiles of block_n keys (vLLM PR #50776 report, "Key source
 * snippets"; vLLM PR #53147 report, "Implementation breakdown" item 2).
 *   bounds_out  device int32 [num_seqs][cdiv(max_q_len, block_q)][2], written (lo, hi); tiles
 *               past a sequence's last row get (0, 0).  block_q and block_n are those of
 *               prefill_attention_tile_config_ex(head_size, num_heads, num_kv_heads,
 *               num_seqs, max_q_len, window_left, window_right, causal).
 * Other arguments as for prefill_attention.  Errors as for prefill_attention.
 */
int prefill_attention_tile_bounds(const int32_t* query_start_loc, const int32_t* ctx_lens,
                                  int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                  int32_t window_left, int32_t window_right, int32_t causal,
                                  const int32_t* mm_ranges, int32_t num_seqs, int32_t max_q_len,
                                  int32_t max_mm_ranges, int32_t* bounds_out, hipStream_t stream);

/*
 * prefill_attention_ex — prefill_attention with the mask variants and split-KV.  The first 24
 * arguments are those of prefill_attention; prefill_attention(...) equals
 * prefill_attention_ex(..., NULL, 1, 0, -1, 1, NULL, 0, stream).
 *   causal_per_seq  device int32 [num_seqs] of 0/1, the causal flag of each sequence; NULL =
 *                   `causal` for every sequence.  Contents are a precondition (0 or 1).
 *   mm_clamp        1: a multimodal range admits keys j >= a - window_left only (the window-
 *                   clamped prefix mask); 0: a query inside a range sees the whole range
 *                   (vLLM PR #53147 report, "Implementation breakdown" item 1: the
 *                   MM_PREFIX_CLAMP_SW switch).  Tile bounds stay tight in both modes.
 *   chunk_size, chunk_lookback
 *                   chunked local attention when chunk_size > 0 and chunk_lookback >= 0: the base
 *                   window's left edge becomes (a / chunk_size - chunk_lookback) * chunk_size,
 *                   the start of the chunk chunk_lookback chunks before the query's own; a
 *                   multimodal range may still admit earlier keys, clamped by window_left when
 *                   mm_clamp is 1 (vLLM PR #53147 report, "Key source snippets",
 *                   compute_tile_loop_bounds, and "Review highlights").  chunk_size = 0 or
 *                   chunk_lookback = -1: off.
 *   kv_splits       split-KV (vLLM PR #53147 report, "Key source snippets": the segment
 *                   arguments of the tile-bound helper): each Q tile's KV-tile range is cut into
 *                   kv_splits contiguous segments handled by separate workgroups, whose partial
 *                   results (unnormalised O, running max, running sum) are merged by the
 *                   log-sum-exp rule in a second kernel on the same stream.  1 = no split,
 *                   0 = automatic (prefill_attention_kv_splits tells the count), at most 64.
 *   workspace, workspace_bytes
 *                   device scratch owned by the caller, used when the split count is > 1; at
 *                   least prefill_attention_workspace_size(num_heads, head_size, total_q_tokens,
 *                   count) bytes, 256-byte aligned.  Unused (may be NULL) when the count is 1.
 *                   Two calls in flight must not share a workspace.
 * Errors: as prefill_attention, plus INVALID_ARG for mm_clamp not 0/1, chunk_size < 0,
 * chunk_lookback < -1, kv_splits outside [0, 64], or a missing/short workspace.
 */
int prefill_attention_ex(const void* q, const void* k_new, const void* v_new,
                         const void* k_cache, const void* v_cache,
                         const int32_t* block_table, const int32_t* query_start_loc,
                         const int32_t* ctx_lens,
                         int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                         int32_t page_size, int32_t window_left, int32_t window_right,
                         int32_t causal, const int32_t* mm_ranges, float scale, void* out,
                         int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len,
                         int32_t num_pages, int32_t max_pages_per_seq, int32_t max_mm_ranges,
                         const int32_t* causal_per_seq, int32_t mm_clamp, int32_t chunk_size,
                         int32_t chunk_lookback, int32_t kv_splits, void* workspace,
                         uint64_t workspace_bytes, hipStream_t stream);

/*
 * prefill_attention_ex_noalloc — prefill_attention_ex for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, arguments and results as prefill_attention_ex without its workspace
 * arguments.  The split-KV partials live in the library's static scratch, a file-scope device
 * array of PAGED_PREFILL_NOALLOC_SCRATCH_BYTES bytes that every GPU the library runs on holds
 * from module load until the process ends; its device address is looked up once per device, on
 * that device's first call.  The call allocates nothing: no hipMalloc, no hipFree, no allocating
 * library routine.
 *   kv_splits  as for prefill_attention_ex.  An explicit count whose partials
 *              (prefill_attention_workspace_size) exceed the scratch fails with
 *              PAGED_PREFILL_ERR_SCRATCH before anything is launched; the automatic count (0)
 *              falls back to no split when its partials would not fit.
 * Every call on one GPU shares that GPU's scratch, which keeps the last call's contents (no part
 * of it needs clearing: every partial the merge reads is written by the same call).  Calls that
 * overlap on one GPU, on different streams or from different threads, race on the scratch; the
 * caller serialises them (one stream at a time per device).  Errors: as prefill_attention_ex,
 * plus PAGED_PREFILL_ERR_SCRATCH; HIP_ERROR if the scratch cannot be located on the device.
 */
#define PAGED_PREFILL_NOALLOC_SCRATCH_BYTES (64ull << 20)
int prefill_attention_ex_noalloc(const void* q, const void* k_new, const void* v_new,
                                 const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* query_start_loc,
                                 const int32_t* ctx_lens,
                                 int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                 int32_t page_size, int32_t window_left, int32_t window_right,
                                 int32_t causal, const int32_t* mm_ranges, float scale, void* out,
                                 int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len,
                                 int32_t num_pages, int32_t max_pages_per_seq,
                                 int32_t max_mm_ranges, const int32_t* causal_per_seq,
                                 int32_t mm_clamp, int32_t chunk_size, int32_t chunk_lookback,
                                 int32_t kv_splits, hipStream_t stream);

/*
 * prefill_attention_kv_splits — the split count prefill_attention_ex uses for kv_splits,
 * and so the workspace it needs, for a batch under the window (window_left, window_right,
 * causal as for prefill_attention; they pick the head-size-64 geometry).  kv_splits > 0:
 * kv_splits itself.  kv_splits = 0 (automatic), with W the workgroups the GPU runs at once (CUs
 * times the workgroups that one CU holds of the shape prefill_attention_tile_config_ex names:
 * 256, 512 or 1024 on MI355X) and the Q-tile work items bounded from the sizes alone (at most
 * num_seqs * cdiv(max_q_len, block_q) Q tiles, and at most
 * (total_q_tokens + num_seqs * (block_q - 1)) / block_q, times the KV heads):
 *   - a whole number of rounds (a multiple of W, at least W items): 1;
 *   - at most W/2 items: k = floor(W / items), one round of segments, or k + 1 when k
 *     segments per item would leave more than a quarter of the round idle; at most 16;
 *   - otherwise fewer than 2W items: enough segments for about 2W workgroups, at most 16;
 *   - in both cases every item longer than its share is cut; but 1 when the window alone
 *     limits a query row to at most 2048 keys (then no item outgrows the share and a split
 *     would cut nothing);
 *   - 2W to 4W items whose last round is at most a quarter full (num_seqs <= 256): 4, and
 *     only the items of that last round are cut, by workgroups appended to the grid (the
 *     kernel counts those items exactly from the device-side lengths);
 *   - otherwise 1.
 * Host-only (it asks the runtime for the current device's CU count).  Returns the count
 * (>= 1) or a negative error code (INVALID_ARG for negative sizes, kv_splits outside
 * [0, 64], a window below -1 or causal not 0/1; UNSUPPORTED as for tile_config).
 */
int prefill_attention_kv_splits(int32_t head_size, int32_t num_heads, int32_t num_kv_heads,
                                int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len,
                                int32_t window_left, int32_t window_right, int32_t causal,
                                int32_t kv_splits);

/*
 * prefill_attention_workspace_size — bytes of workspace prefill_attention_ex needs with
 * `splits` segments (0 when splits <= 1, or for invalid sizes): fp32 partial outputs
 * [splits][total_q_tokens][num_heads][head_size] then fp32 (max, sum) pairs
 * [splits][total_q_tokens][num_heads].  Host-only.
 */
uint64_t prefill_attention_workspace_size(int32_t num_heads, int32_t head_size,
                                          int32_t total_q_tokens, int32_t splits);

/*
 * prefill_attention_tile_bounds_ex — prefill_attention_tile_bounds under the mask variants of
 * prefill_attention_ex (causal_per_seq, mm_clamp, chunk_size, chunk_lookback as there).  The
 * chunked left edge is taken at the tile's lowest query row.  Split-KV does not change the
 * bounds: a split only partitions [lo, hi).
 */
int prefill_attention_tile_bounds_ex(const int32_t* query_start_loc, const int32_t* ctx_lens,
                                     int32_t num_heads, int32_t num_kv_heads,
                                     int32_t head_size, int32_t window_left,
                                     int32_t window_right, int32_t causal,
                                     const int32_t* mm_ranges, int32_t num_seqs,
                                     int32_t max_q_len, int32_t max_mm_ranges,
                                     const int32_t* causal_per_seq, int32_t mm_clamp,
                                     int32_t chunk_size, int32_t chunk_lookback,
                                     int32_t* bounds_out, hipStream_t stream);

/*
 * prefill_attention_check_metadata — checks on the GPU the device-resident preconditions that
 * prefill_attention states but does not check (a debug aid for callers and tests; the attention
 * entry points never call it).  It reads query_start_loc [S+1], ctx_lens [S] and, of
 * block_table [S][max_pages_per_seq], exactly the entries prefill_attention would read (entry p
 * of sequence s when p * page_size < ctx_lens[s], or < L in cache-sourced mode, cache_only = 1:
 * the k_new = v_new = NULL mode).  It writes one int32 to the device pointer flags_out: 0 when
 * every precondition holds, else the OR of
 *   PAGED_PREFILL_BAD_QSL      query_start_loc[0] != 0, query_start_loc[S] != total_q_tokens, or
 *                              a decreasing step;
 *   PAGED_PREFILL_BAD_QLEN     some n_s > max_q_len;
 *   PAGED_PREFILL_BAD_CTX      some ctx_lens[s] < 0;
 *   PAGED_PREFILL_BAD_LENGTH   some L = ctx_lens[s] + n_s above 2^24 positions;
 *   PAGED_PREFILL_BAD_PAGES    some sequence needs more than max_pages_per_seq pages;
 *   PAGED_PREFILL_BAD_PAGE_ID  a block-table entry that would be read lies outside [0, num_pages).
 * One workgroup; enqueued on `stream` like the attention call, so the result is valid after the
 * caller synchronises.  All pointers are device pointers owned by the caller.  Errors:
 * INVALID_ARG for a null query_start_loc or flags_out, a null ctx_lens with num_seqs > 0, a null
 * block_table with a non-empty table, page_size <= 0, negative sizes, or cache_only not 0/1;
 * HIP_ERROR if the launch fails.
 */
#define PAGED_PREFILL_BAD_QSL 1
#define PAGED_PREFILL_BAD_QLEN 2
#define PAGED_PREFILL_BAD_CTX 4
#define PAGED_PREFILL_BAD_LENGTH 8
#define PAGED_PREFILL_BAD_PAGES 16
#define PAGED_PREFILL_BAD_PAGE_ID 32
int prefill_attention_check_metadata(const int32_t* block_table,
                                     const int32_t* query_start_loc, const int32_t* ctx_lens,
                                     int32_t cache_only, int32_t page_size, int32_t num_seqs,
                                     int32_t total_q_tokens, int32_t max_q_len,
                                     int32_t num_pages, int32_t max_pages_per_seq,
                                     int32_t* flags_out, hipStream_t stream);

/* prefill_attention_strerror — static description of an error code (never NULL).  No passage
 * of the pages defines it: it names this library's own error codes. */
const char* prefill_attention_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_PREFILL_H */
