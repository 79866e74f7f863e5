// Paged-KV prefill attention for MI355X (gfx950, CDNA4).
//
// One workgroup owns one Q tile: `block_q` query tokens of one sequence times
// the `heads_per_tile` query heads of one GQA group, packed into 32 MFMA rows
// per wavefront (256 rows for 8 wavefronts), so one K/V gather serves every
// head of the group.  Sequences are ranked heavy-first; a sequence's work
// items go in blocks of 8 (KV head, head block) columns, the Q tiles of one
// column on consecutive slots of one XCD (slot k of XCD x is item 8k + x).
// The workgroup walks the KV tiles
// [lo, hi) given by the tile bound calculator (the window unioned with every
// multimodal range that overlaps the tile's queries; vLLM PR #50776 report,
// "Key source snippets"; vLLM PR #53147 report, "Implementation breakdown"
// item 2).  Per KV tile:
//
//   1. page-offset resolver: key position j < ctx_len is slot j % P of page
//      block_table[j / P] (division by an invariant integer with a
//      Granlund-Montgomery multiply-shift, PLDI 1994; the block-table entries
//      an item reads are staged in LDS once, or read on the scalar unit when
//      there are too many), j >= ctx_len is a row of the chunk's new K/V,
//      j >= L reads a zero row; tiles never depend on pages, so any page size
//      works (vLLM PR #54194 report, "Features and motivation");
//   2. coalesced gather: 16-byte global->LDS DMA (global_load_lds_dwordx4)
//      into a 4-stage ring, two tiles per barrier with the next two in
//      flight.  K and V rows are stored row-major with XOR-swizzled 16-byte
//      chunks (conflict-free reads);
//   3. S^T = K Q^T on v_mfma_f32_32x32x16_bf16: every lane holds one query
//      row's scores, so softmax row reductions are in-lane plus one
//      v_permlane32_swap with the lane 32 away;
//   4. the element mask, only on tiles that are not provably all-allowed;
//   5. online softmax in the exp2 domain (Milakov & Gimelshein 2018, with the
//      scale folded into exp2 as in FlashAttention-2, Dao 2023);
//   6. O^T += V^T P^T on the same MFMA: P rounded to bf16 (round-to-nearest-
//      even, v_cvt_pk_bf16_f32); the V^T operand comes straight from the
//      row-major V tile through ds_read_b64_tr_b16.
// A Q tile with at most half its rows valid splits its KV tiles between the
// two halves of the workgroup and merges them by log-sum-exp.  The epilogue
// divides by the row sum and stores bf16 (or, under split-KV, the unnormalised
// partial with its max and sum for merge_splits_kernel).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "paged_prefill.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) float lds_f32;

constexpr int kMaxTokens = 1 << 24; // positions per sequence the resolver handles exactly
constexpr int kMaxMmRanges = 4096;
constexpr int kNumXcd = 8;         // MI355X: 8 accelerator complex dies, one L2 each
constexpr int kSortMaxSeqs = 256;  // batches up to this size get heavy-first ordering

// Tile shape per head size: wavefronts per workgroup, keys per KV tile, depth
// of the LDS ring, wavefronts per SIMD, and 32-row query blocks per wavefront.
// Overridable at build time (-DPREFILL_TILE_D128=4,64,4,1,2) for sweeps.  Head
// size 64 has two, picked per call by choose_tiles: PREFILL_TILE_D64 (longer
// tiles, for long KV loops) and PREFILL_TILE_D64_MANY (more workgroups per CU,
// shorter tiles, for short windows and batches of many work items).
#ifndef PREFILL_TILE_D64
#define PREFILL_TILE_D64 4, 64, 4, 2, 1
#endif
#ifndef PREFILL_TILE_D64_MANY
#define PREFILL_TILE_D64_MANY 4, 32, 4, 4, 1
#endif
#ifndef PREFILL_TILE_D128
#define PREFILL_TILE_D128 8, 64, 4, 2, 1
#endif
#ifndef PREFILL_TILE_D256
#define PREFILL_TILE_D256 8, 32, 4, 2, 1
#endif

// Rows past the end of a sequence are gathered from here: exact zeros.
__device__ __attribute__((aligned(16))) uint16_t g_zero_row[256];

// Split-KV partials of the allocation-free entry point (prefill_attention_ex_noalloc).
// Host code never passes this name to a kernel: it is a host-side stand-in, not a device
// address.  The device address comes from hipGetSymbolAddress, once per device
// (scratch_for_current_device below).
__device__ __attribute__((aligned(256))) unsigned char scratch[PAGED_PREFILL_NOALLOC_SCRATCH_BYTES];

struct KernelArgs {
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_table;
  const int32_t* qsl;
  const int32_t* ctx_lens;
  const int32_t* mm_ranges;
  uint16_t* out;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t group;           // query heads per KV head
  int32_t heads_per_tile;  // query heads of one group packed into a workgroup
  int32_t head_blocks;     // group / heads_per_tile
  int32_t block_q;         // query tokens per Q tile = rows / heads_per_tile
  int32_t page_size;
  uint32_t page_magic;     // ceil(2^(24+l) / page_size), l = ceil(log2(page_size))
  int32_t page_shift;      // 24 + l
  int32_t window_left;
  int32_t window_right;
  int32_t causal;
  float scale_log2;        // scale * log2(e)
  int32_t num_seqs;
  int32_t max_pages_per_seq;
  int32_t max_mm_ranges;
  int32_t cache_only;      // 1: every position comes from the cache
  int32_t num_q_tiles;     // cdiv(max_q_len, block_q)
  const int32_t* causal_per_seq;  // [num_seqs] or null (then `causal`)
  int32_t mm_clamp;
  int32_t chunk_size;
  int32_t chunk_lookback;
  int32_t kv_splits;       // KV segments per Q tile (1: no split)
  int32_t total_q_tokens;
  float* part_o;           // [kv_splits][T][H][d] unnormalised partial O (kv_splits > 1)
  float2* part_ml;         // [kv_splits][T][H] (m, l) of each partial, log2 units
  // Tail splitting (kv_splits segments for the items of the last partial round
  // only): main_slots item slots, then helper slots; round_slots workgroups
  // run at once.  tail_mode = 0: the segment-cap rule above applies instead.
  int32_t tail_mode;
  int32_t main_slots;
  int32_t round_slots;
};

// ---------------------------------------------------------------------------
// Mask of one sequence.  A key j < L is allowed for the query at absolute
// position a when the base window admits it:
//   causal => j <= a;  left edge: the chunk start (a / chunk_size -
//   chunk_lookback) * chunk_size in chunked local attention, else a -
//   window_left when window_left >= 0;  !causal and window_right >= 0 =>
//   j <= a + window_right;
// or when a valid multimodal range [st, en] (st < en) holds both a and j and,
// with the window clamp on, j >= a - window_left.  (vLLM PR #53147 report,
// "Key source snippets", compute_tile_loop_bounds; "Review highlights".)
// ---------------------------------------------------------------------------
struct MaskSpec {
  int causal;
  int wl, wr;
  int chunk_size, chunk_lookback;  // chunked when chunk_size > 0 and chunk_lookback >= 0
  int mm_clamp;                    // 1: a range is clamped on the left by window_left
};

__device__ __forceinline__ int base_left(int a, const MaskSpec& m) {
  if (m.chunk_size > 0 && m.chunk_lookback >= 0)
    return (a / m.chunk_size - m.chunk_lookback) * m.chunk_size;
  return m.wl >= 0 ? a - m.wl : 0;
}
__device__ __forceinline__ int range_left(int st, int a, const MaskSpec& m) {
  return (m.mm_clamp && m.wl >= 0) ? max(st, a - m.wl) : st;
}

// Tile bound calculator.  Query rows of tile t are [t*block_q, min(..., n)-1];
// the base window runs from base_left(a_lo) to a_hi (causal), a_hi +
// window_right, or the last key; every valid range [st, en] overlapping
// [a_lo, a_hi] may lower the left edge to range_left(st, a_lo) and raise the
// right edge to en; the result is clamped to [0, L-1] and converted to KV
// tiles of `block_n` keys.  Left edges are taken at the tile's lowest row,
// where they are smallest.
__device__ __forceinline__ int2 kv_tile_range(int c, int n, int t, int block_q, int block_n,
                                              const MaskSpec& m, const int32_t* ranges,
                                              int num_ranges) {
  const int i_lo = t * block_q;
  if (i_lo >= n) return make_int2(0, 0);
  const int i_hi = min(i_lo + block_q - 1, n - 1);
  const int L = c + n;
  const int a_lo = c + i_lo;
  const int a_hi = c + i_hi;
  int first = base_left(a_lo, m);
  int last = m.causal ? a_hi : (m.wr >= 0 ? a_hi + min(m.wr, L) : L - 1);
  for (int r = 0; r < num_ranges; ++r) {
    const int st = ranges[2 * r];
    const int en = ranges[2 * r + 1];
    if (st < en && st <= a_hi && en >= a_lo) {
      first = min(first, range_left(st, a_lo, m));
      last = max(last, en);
    }
  }
  first = max(first, 0);
  last = min(last, L - 1);
  return make_int2(first / block_n, last / block_n + 1);
}

// Allowed keys of the query at absolute position a: one interval [lo, hi].
// The base window always contains j = a, and every multimodal range that
// admits the query contains a as well, so their union is a single interval.
__device__ __forceinline__ void row_interval(int a, int L, const MaskSpec& m,
                                             const int32_t* ranges, int num_ranges,
                                             int& lo, int& hi) {
  lo = base_left(a, m);
  hi = m.causal ? a : (m.wr >= 0 ? a + min(m.wr, L) : L - 1);
  for (int r = 0; r < num_ranges; ++r) {
    const int st = ranges[2 * r];
    const int en = ranges[2 * r + 1];
    if (st < en && st <= a && a <= en) {
      lo = min(lo, range_left(st, a, m));
      hi = max(hi, en);
    }
  }
  lo = max(lo, 0);
  hi = min(hi, L - 1);
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}

// max over the lane pair (l, l ^ 32): v_permlane32_swap exchanges the two
// halves of the wave, so both lanes of a pair see both values.
__device__ __forceinline__ float pair_max(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// 16-byte asynchronous global->LDS copy: lane i writes lds_base + 16 i.  The
// compiler does not track these copies; completion is awaited explicitly with
// vm_wait<>() before the barrier that publishes a stage.  The LDS base goes
// through M0, which the compiler reserves: the copy saves M0 and puts it back,
// and leaves one wait state between the M0 write and the copy that reads it.
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
               "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(gaddr), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}
// Same copy from a wave-uniform base plus a 32-bit per-lane byte offset.
__device__ __forceinline__ void dma16s(uint32_t voff, const void* sbase, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
               "global_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}
// Page index of position j: floor(j / page_size) by Granlund-Montgomery
// multiply-shift (exact for j < 2^24).
__device__ __forceinline__ int page_of(int j, uint32_t magic, int shift) {
  return (int)(((uint64_t)(uint32_t)j * magic) >> shift);
}

// Block-table entry read on the scalar unit (s_load, counted by lgkmcnt), so a
// lookup never waits on the vector-memory counter that tracks the copies in
// flight.  `ptr` must be wave-uniform.
__device__ __forceinline__ int scalar_load_i32(const int32_t* ptr) {
  const uint64_t a = (uint64_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint64_t ua = ((uint64_t)hi << 32) | lo;
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ua) : "memory");
  return v;
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ void block_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS tile layout: rows of D bf16 (one key each), 16-byte chunks XOR-swizzled
// per row so that the MFMA operand reads hit distinct banks.
template <int D>
struct TileLayout {
  static constexpr int CHUNKS = D / 8;
  static constexpr int ROWS_PER_DMA = 512 / D;  // key rows per 1-KB DMA instruction
  // K: 16 lanes read the same chunk of 16 consecutive rows.
  __device__ static __forceinline__ int kswz(int row) {
    return D == 64 ? ((row >> 1) & 7) : (row & 15);
  }
  __device__ static __forceinline__ int kslot(int row, int chunk) { return chunk ^ kswz(row); }
  // V: a 16-lane group reads 4 consecutive rows x 4 chunks (transpose read).
  __device__ static __forceinline__ int vswz(int row) {
    return D == 64 ? ((((row >> 1) & 1)) << 2) : ((row & 3) << 2);
  }
  __device__ static __forceinline__ int vslot(int row, int chunk) { return chunk ^ vswz(row); }
  // The swizzle only touches address bits below the row stride (2D bytes), so
  // the byte offset of chunk (2ks + half) in row r is
  //   (r*2D + 16*(half ^ kswz(r))) ^ (32*ks)
  // and the transpose-read offset of dim block db is (base) ^ (64*db): one
  // lane-invariant base per operand, one XOR per read.
};

// ---------------------------------------------------------------------------
// Work decode.  The dispatcher deals workgroup ids to the 8 XCDs round-robin
// (id b runs on XCD b % 8 as its (b / 8)-th workgroup), and each XCD has its
// own L2.  A work item is (sequence s, KV head g, Q tile t, head block); all
// items of one (s, g) group read the same K/V stream, so they get consecutive
// slots on one XCD and share its L2.  For up to kSortMaxSeqs sequences the
// sequences are ranked heavy-first by their key count L; within a sequence,
// blocks of 8 (KV head, head block) columns deal each column's Q tiles to
// consecutive slots of one XCD, the tile order turned by one per block (see
// below).  Larger batches deal g-major contiguous chunks.
// ---------------------------------------------------------------------------
struct WorkItem {
  int s, g, hblk, t;
  bool valid;
  bool split;  // tail splitting: this item is cut into kv_splits segments
  int piece;   // the segment this slot computes
};

__device__ __forceinline__ int seq_ntiles(const int32_t* qsl, int s, int block_q) {
  return (qsl[s + 1] - qsl[s] + block_q - 1) / block_q;
}

// Per-sequence fields staged in LDS by decode_work for batches of up to
// kSortMaxSeqs sequences (one round trip to memory for all of them).
struct SeqTable {
  int order[kSortMaxSeqs];           // sequence of rank r (heaviest first)
  int ntiles_by_rank[kSortMaxSeqs];  // its Q tile count
  int key[kSortMaxSeqs];             // context + new tokens
  int q0[kSortMaxSeqs];              // query_start_loc
  int ctx[kSortMaxSeqs];             // cached tokens
};

template <typename Args>
__device__ WorkItem decode_work(const Args& p, int b, int tid, int nthreads, SeqTable& st) {
  int* order = st.order;
  int* ntiles_by_rank = st.ntiles_by_rank;
  const int S = p.num_seqs;
  const int Hkv = p.num_kv_heads;
  const int HBLK = p.head_blocks;
  const int x = b % kNumXcd;
  int k = b / kNumXcd;
  WorkItem w{0, 0, 0, 0, false, false, 0};
  if (S <= kSortMaxSeqs) {
    for (int i = tid; i < S; i += nthreads) {
      const int a = p.qsl[i], e = p.qsl[i + 1], cl = p.ctx_lens[i];
      st.key[i] = cl + e - a;
      st.q0[i] = a;
      st.ctx[i] = cl;
    }
    __syncthreads();
    for (int i = tid; i < S; i += nthreads) {
      const int key_i = st.key[i];
      int rank = 0;
      for (int j = 0; j < S; ++j) {
        const int key_j = st.key[j];
        rank += (key_j > key_i) || (key_j == key_i && j < i);
      }
      order[rank] = i;
      ntiles_by_rank[rank] = (key_i - st.ctx[i] + p.block_q - 1) / p.block_q;
    }
    __syncthreads();
    // Items in heavy-first order of their sequences are dealt round-robin over
    // the XCDs: slot k of XCD x is item 8k + x.  The order within a sequence
    // (its Q tiles by column blocks) is set in the enumeration below.
    int j = k * kNumXcd + x;
    if (p.tail_mode) {
      // Tail splitting.  The items past the last whole round (total mod
      // round_slots of them: the last in the order below, so those of the
      // lightest sequences, though within a column block the tile order is
      // rotated and they need not be the lightest tiles) would run alone at
      // the end; when they fill at most a quarter of a round, the last m of
      // them are cut into kv_splits segments: segment 0 in the item's own
      // slot, the others in the helper slots that follow the main ones.
      int total = 0;
      for (int sr = 0; sr < S; ++sr) total += ntiles_by_rank[sr];
      total *= Hkv * HBLK;
      const int ks = p.kv_splits;
      const int helpers = (int)gridDim.x - p.main_slots;
      const int tail = total % p.round_slots;
      const int m = tail <= p.round_slots / 4 ? min(tail, helpers / (ks - 1)) : 0;
      if (j >= p.main_slots) {  // helper slot: segment 1 + h % (ks - 1) of tail item h / (ks - 1)
        const int h = j - p.main_slots;
        if (h / (ks - 1) >= m) return w;
        w.piece = 1 + h % (ks - 1);
        j = total - m + h / (ks - 1);
      }
      w.split = j >= total - m && j < total;
    }
    for (int sr = 0; sr < S; ++sr) {
      const int per_tile = Hkv * HBLK;  // (KV head, head block) columns of a Q tile
      const int nt = ntiles_by_rank[sr];
      const int per_seq = per_tile * nt;
      if (j < per_seq) {
        // Columns go in blocks of 8; within a block, the Q tiles of each column
        // take consecutive slots of one XCD (item 8 zz + c of the block), so
        // they stream the column's K/V together and share it in L2.  The tile
        // order turns by one per block, so that the XCD's four shader engines,
        // which take its slots in strict rotation, see every tile length.  A
        // last block of wdt < 8 columns (columns per Q tile not a multiple of
        // 8) lays its items out as wdt zz + c: there a column's Q tiles are
        // spread over XCDs and do not share L2.
        const int cb = j / (8 * nt);
        const int wdt = min(8, per_tile - cb * 8);
        const int jj = j - cb * 8 * nt;
        const int zz = jj / wdt;
        const int col = cb * 8 + (jj - zz * wdt);
        const int z = (zz + cb) % nt;
        w.s = order[sr];
        w.g = col / HBLK;
        w.hblk = col - w.g * HBLK;
        w.t = nt - 1 - z;
        w.valid = true;
        return w;
      }
      j -= per_seq;
    }
    return w;
  }
  // Large batches: XCD x owns a contiguous g-major range of (g, s) groups,
  // each padded to the largest tile count (padding items exit).
  const int groups = S * Hkv;
  const int gper = (groups + kNumXcd - 1) / kNumXcd;
  const int per_group = p.num_q_tiles * HBLK;
  const int gidx = x * gper + k / per_group;
  if (gidx >= groups || k >= gper * per_group) return w;
  const int rem = k % per_group;
  const int s = gidx % S;
  const int nt = seq_ntiles(p.qsl, s, p.block_q);
  const int z = rem / HBLK;
  if (z >= nt) return w;
  w.s = s;
  w.g = gidx / S;
  w.hblk = rem - z * HBLK;
  w.t = nt - 1 - z;
  w.valid = true;
  return w;
}

template <int D_, int NW_, int BN_, int NSTAGE_, int WPE_, int RB_>
struct TileShape {
  static constexpr int D = D_;
  static constexpr int NW = NW_;
  static constexpr int BN = BN_;          // keys per KV tile
  static constexpr int NSTAGE = NSTAGE_;  // LDS ring depth (NSTAGE - 1 tiles in flight)
  static constexpr int WPE = WPE_;        // wavefronts per SIMD
  static constexpr int RB = RB_;          // 32-row query blocks per wavefront
  static constexpr int THREADS = 64 * NW;
  static constexpr int ROWS = 32 * RB * NW;
  static constexpr int DMA_PER_TENSOR = BN * D * 2 / 1024;  // 1-KB copies per tile per tensor
  static constexpr int DMA_PER_WAVE = DMA_PER_TENSOR / NW;
  static constexpr int LDS_BYTES = NSTAGE * 2 * BN * D * 2;
  // Block-table entries staged in LDS per workgroup: sized so that the
  // workgroups a CU holds (one with a large ring, two with a medium one, four
  // with a 32 KiB ring at four wavefronts per SIMD) fit its 160 KiB.
  static constexpr int BT_CACHE = WPE_ >= 4 ? 512 : (LDS_BYTES >= 96 * 1024 ? 4096 : 2048);
  // KV-pair mode (short Q tiles): the two halves of the workgroup exchange
  // their partial results through the ring, NW/2 x 64 lanes x (O, m, l).
  static constexpr int XREGS = RB * (D / 32 * 16 + 2);
  static constexpr bool PAIR = NW % 2 == 0 && NW / 2 * 64 * XREGS * 4 <= LDS_BYTES;
  // The output tile (ROWS x D bf16) is staged through the ring for row-wise stores.
  static constexpr bool STAGE_OUT = ROWS * D * 2 <= LDS_BYTES;
  // Workgroups resident per CU: four SIMDs of WPE wavefronts, 160 KiB of LDS
  // (ring, block-table cache, sequence table and a little slack).
  static constexpr int LDS_TOTAL = LDS_BYTES + BT_CACHE * 4 + 6 * 1024;
  static constexpr int WG_PER_CU = (4 * WPE / NW) < (160 * 1024 / LDS_TOTAL)
                                       ? (4 * WPE / NW) : (160 * 1024 / LDS_TOTAL);
  static_assert(WG_PER_CU >= 1, "a workgroup must fit a CU");
  static_assert(DMA_PER_TENSOR % NW == 0, "copies must split evenly over the wavefronts");
  static_assert(BN % 32 == 0 && D % 32 == 0, "MFMA blocking");
  static_assert(NSTAGE >= 2 && NSTAGE <= 6, "ring depth");

  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};
template <int D> struct ShapeFor;
template <> struct ShapeFor<64> { using T = TileShape<64, PREFILL_TILE_D64>; };
struct ShapeD64Many { using T = TileShape<64, PREFILL_TILE_D64_MANY>; };
template <> struct ShapeFor<128> { using T = TileShape<128, PREFILL_TILE_D128>; };
template <> struct ShapeFor<256> { using T = TileShape<256, PREFILL_TILE_D256>; };

template <typename C>
__global__ __attribute__((amdgpu_flat_work_group_size(C::THREADS, C::THREADS),
                          amdgpu_waves_per_eu(C::WPE, C::WPE)))
void prefill_attention_kernel(const KernelArgs p) {
  constexpr int D = C::D;
  constexpr int NW = C::NW;
  constexpr int RB = C::RB;
  constexpr int NSTAGE = C::NSTAGE;
  using Lay = TileLayout<D>;
  constexpr int BN = C::BN;
  constexpr int KSTEPS = D / 16;   // QK^T contraction steps of 16 dims
  constexpr int NKB = BN / 32;     // 32-key blocks per KV tile
  constexpr int PSTEPS = BN / 16;  // PV contraction steps of 16 keys
  // Operand fragments in flight ahead of the MFMAs that consume them (each
  // fragment feeds RB MFMAs).
  constexpr int QK_DEPTH = RB == 1 ? 4 : 3;
  constexpr int PV_DEPTH = RB == 1 ? 3 : 2;
  constexpr int NDB = D / 32;      // 32-dim blocks of the output
  constexpr int TILE_ELEMS = BN * D;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[NSTAGE][2][TILE_ELEMS];

  __shared__ SeqTable seqs;
  const int tid = threadIdx.x;
  // Split-KV: the kv_splits segments of one work item take consecutive slots
  // of the same XCD.  Items that stay whole use only their segment-0 slot, and
  // the hardware hands an XCD's workgroups to its 4 shader engines in strict
  // rotation, so the segment-0 slot is placed per item such that those slots
  // fall on every engine in turn.
  // Under tail splitting every slot is one item (or a helper segment), and
  // decode_work says which segment.
  const int ks = p.tail_mode ? 1 : p.kv_splits;
  const int pos = (int)((blockIdx.x / kNumXcd) % ks);
  const int item_idx = (int)((blockIdx.x / kNumXcd) / ks);
  const int pos0 = ks % 2 ? 0 : (ks % 4 == 2 ? (item_idx / 2) % 2 : item_idx % 4);
  const int bitem = (int)((blockIdx.x / kNumXcd) / ks) * kNumXcd + blockIdx.x % kNumXcd;
  const WorkItem wi = decode_work(p, bitem, tid, C::THREADS, seqs);
  if (!wi.valid) return;  // padding slot
  const int split = p.tail_mode ? wi.piece : (pos + ks - pos0) % ks;
  const int s = wi.s;
  const int g = wi.g;
  const int hblk = wi.hblk;
  const int t = wi.t;
  // workgroup-uniform: scalar registers (the copy bases are built from them)
  const bool staged = p.num_seqs <= kSortMaxSeqs;
  const int q0 = __builtin_amdgcn_readfirstlane(staged ? seqs.q0[s] : p.qsl[s]);
  const int n = __builtin_amdgcn_readfirstlane(staged ? seqs.key[s] - seqs.ctx[s]
                                                      : p.qsl[s + 1] - p.qsl[s]);
  const int c = __builtin_amdgcn_readfirstlane(staged ? seqs.ctx[s] : p.ctx_lens[s]);
  const int L = c + n;
  const int cache_end = p.cache_only ? L : c;
  const int R = p.max_mm_ranges;
  const int32_t* ranges = R > 0 ? p.mm_ranges + (int64_t)s * R * 2 : nullptr;
  const int32_t* bt = p.block_table + (int64_t)s * p.max_pages_per_seq;

  const MaskSpec mspec{p.causal_per_seq != nullptr ? p.causal_per_seq[s] : p.causal,
                       p.window_left, p.window_right, p.chunk_size, p.chunk_lookback,
                       p.mm_clamp};
  int2 tb = kv_tile_range(c, n, t, p.block_q, BN, mspec, ranges, R);
  // Split-KV: an item of at most `cap` KV tiles stays whole (its segment 0
  // writes the output; the item's other slots exit).  Longer items are cut into
  // segments of max(cap, ceil(tiles / kv_splits)) tiles, merged afterwards.
  // cap = ceil(tiles of the longest sequence / kv_splits), so only the items
  // that would hold back the tail are split and pay for partial results.
  bool whole = true;
  if (p.tail_mode) {
    if (wi.split) {  // segment `split` of kv_splits equal runs (possibly empty)
      const int k = p.kv_splits;
      const int per = (tb.y - tb.x + k - 1) / k;
      const int x0 = min(tb.x + split * per, tb.y);
      tb = make_int2(x0, min(x0 + per, tb.y));
      whole = false;
    }
  } else if (p.kv_splits > 1) {
    const int k = p.kv_splits;
    const int n_item = tb.y - tb.x;
    const int lmax = staged ? seqs.key[seqs.order[0]] : 0;  // heaviest sequence first
    const int cap = ((lmax + BN - 1) / BN + k - 1) / k;
    const int per = max(cap, (n_item + k - 1) / k);
    whole = __builtin_amdgcn_readfirstlane(n_item <= per ? 1 : 0) != 0;
    if (whole) {
      if (split > 0) return;
    } else {  // this item's segment of the tile range (possibly empty)
      const int x0 = min(tb.x + split * per, tb.y);
      tb = make_int2(x0, min(x0 + per, tb.y));
    }
  }
  // wave-uniform: keeps the loop bounds and copy bases in scalar registers
  tb.x = __builtin_amdgcn_readfirstlane(tb.x);
  tb.y = __builtin_amdgcn_readfirstlane(tb.y);

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;

  // ---- KV-pair mode.  When every valid row of the Q tile lies in the first
  // half of the tile (the short last tile of a sequence), both halves of the
  // workgroup take those rows and split the KV tiles between them, even tiles
  // to the first half and odd to the second: half the loop steps, with all
  // wavefronts busy.  The halves' partial results are merged at the end.
  const int vtok = min(n - t * p.block_q, p.block_q);
  const int rows_used = (p.heads_per_tile - 1) * p.block_q + vtok;
  const bool pair = __builtin_amdgcn_readfirstlane(
                        C::PAIR && rows_used <= C::ROWS / 2 && tb.y - tb.x >= 2 ? 1 : 0) != 0;
  // Wavefront w runs on SIMD w % 4.  The second half's row blocks are rotated
  // by a quarter of the workgroup, so that when only one or two row blocks
  // hold valid rows, their two halves run on different SIMDs rather than
  // sharing one.
  const int khalf = pair ? wave / (NW / 2) : 0;  // KV half: tiles with index % 2 == khalf
  const int wrow = pair ? (wave + khalf * (NW / 4)) % (NW / 2) : wave;  // row block of the tile

  // ---- this lane's query rows, one per row block (both lane halves hold the
  // same rows): tile row wrow*32*RB + 32*rb + col
  int tok[RB], head[RB], lo_a[RB], hi_a[RB];
  bool valid[RB];
  int lo_max = INT_MIN, hi_min = INT_MAX, lo_min = INT_MAX, hi_max = INT_MIN;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = (wrow * RB + rb) * 32 + col;
    const int hb = row / p.block_q;
    tok[rb] = t * p.block_q + (row - hb * p.block_q);
    valid[rb] = tok[rb] < n;
    head[rb] = g * p.group + hblk * p.heads_per_tile + hb;
    lo_a[rb] = 1;
    hi_a[rb] = 0;
    if (valid[rb]) {
      row_interval(c + tok[rb], L, mspec, ranges, R, lo_a[rb], hi_a[rb]);
      lo_max = max(lo_max, lo_a[rb]);
      hi_min = min(hi_min, hi_a[rb]);
      lo_min = min(lo_min, lo_a[rb]);
      hi_max = max(hi_max, hi_a[rb]);
    }
  }
  // wave-uniform summaries of the rows' key intervals (scalar registers)
  const int w_lo_max = __builtin_amdgcn_readfirstlane(wave_max(lo_max));
  const int w_hi_min = __builtin_amdgcn_readfirstlane(wave_min(hi_min));
  const int w_lo_min = __builtin_amdgcn_readfirstlane(wave_min(lo_min));
  const int w_hi_max = __builtin_amdgcn_readfirstlane(wave_max(hi_max));
  const bool wave_active = w_hi_max != INT_MIN;

  // ---- gather: wave `wave` issues copies id = wave*DMA_PER_WAVE + q of each
  // tensor; copy id fills key rows [id*ROWS_PER_DMA, +ROWS_PER_DMA), lane ->
  // (row, 16-byte slot).
  const uint32_t smem_base =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_u16*)&smem[0][0][0]);
  const int lane_row = lane / Lay::CHUNKS;
  const int lane_slot = lane % Lay::CHUNKS;
  const int64_t kv_row_stride = (int64_t)p.num_kv_heads * D;
  const int64_t lane_row_off = (int64_t)lane_row * kv_row_stride;
  // Wavefront `wave` fills tile rows [wave*WROWS, +WROWS) with DMA_PER_WAVE
  // copies per tensor; byte offsets of this lane's 16 bytes from the first
  // row's source, when those rows are consecutive in memory.
  constexpr int WROWS = C::DMA_PER_WAVE * Lay::ROWS_PER_DMA;
  // Source bases held in scalar registers (otherwise the compiler re-reads
  // them from the argument block inside the loop to pick one).
  const uint16_t* kc_ptr = p.k_cache;
  const uint16_t* vc_ptr = p.v_cache;
  const uint16_t* kn_ptr = p.k_new;
  const uint16_t* vn_ptr = p.v_new;
  const uint16_t* zero_row = g_zero_row;
  asm volatile("" : "+s"(kc_ptr), "+s"(vc_ptr), "+s"(kn_ptr), "+s"(vn_ptr), "+s"(zero_row));
  uint32_t voff_k[C::DMA_PER_WAVE], voff_v[C::DMA_PER_WAVE];
#pragma unroll
  for (int qi = 0; qi < C::DMA_PER_WAVE; ++qi) {
    const int rr = qi * Lay::ROWS_PER_DMA + lane_row;  // row within the wavefront's rows
    const int r = wave * WROWS + rr;                    // tile row
    voff_k[qi] = (uint32_t)((rr * kv_row_stride + 8 * Lay::kslot(r, lane_slot)) * 2);
    voff_v[qi] = (uint32_t)((rr * kv_row_stride + 8 * Lay::vslot(r, lane_slot)) * 2);
  }
  // ---- Q rows, loaded here so that their latency overlaps the block-table
  // staging below (lane: row `col`, dims 16ks + 8half..+8).  Rows past the
  // sequence read its first token (always present) and are zeroed after the
  // loads: a conditional load would be waited for one at a time.
  u32x4 qraw[RB][KSTEPS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const uint16_t* qrow =
        p.q + ((int64_t)(q0 + (valid[rb] ? tok[rb] : 0)) * p.num_heads + head[rb]) * D;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qraw[rb][ks] = *(const u32x4*)(qrow + 16 * ks + 8 * half);
  }
  // Block-table entries of every page the tile loop reads, staged in LDS once,
  // so the loop resolves pages with one LDS read per lane.  Workgroups that
  // touch more than BT_CACHE pages fall back to scalar-unit block-table reads.
  __shared__ int bt_cache[C::BT_CACHE];
  const uint32_t page_magic = p.page_magic;
  const int page_shift = p.page_shift;
  const int cache_lo = tb.x * BN;
  const int cache_hi = min(tb.y * BN, cache_end);
  const int pg_base = cache_hi > cache_lo ? page_of(cache_lo, page_magic, page_shift) : 0;
  const int pg_count = cache_hi > cache_lo ? page_of(cache_hi - 1, page_magic, page_shift) - pg_base + 1 : 0;
  const bool bt_in_lds = pg_count <= C::BT_CACHE;
  if (bt_in_lds) {
    for (int i = tid; i < pg_count; i += C::THREADS) bt_cache[i] = bt[pg_base + i];
  }
  // The Q loads complete here, before any tile copy is issued: a wait for
  // them later would also wait for copies in flight.  (The builtin form lets
  // the compiler see it: vmcnt(0), expcnt and lgkmcnt unconstrained.)
  __builtin_amdgcn_s_waitcnt(0x0F70);
  block_barrier();

  int cached_pg = -1;        // page index whose element base is cached_base (wave-uniform)
  int64_t cached_base = 0;
  auto issue_tile = [&](int tile, int stage) __attribute__((always_inline)) {
    const int j0 = tile * BN;
    const uint32_t kst = smem_base + (uint32_t)(stage * 2 * TILE_ELEMS * 2);
    const uint32_t vst = kst + (uint32_t)(TILE_ELEMS * 2);
    const int ws = j0 + wave * WROWS;  // first key of this wavefront's rows
    if (bt_in_lds) {
      // Usual case, decided per wavefront: its WROWS keys are consecutive rows
      // of one source (one cache page, or the new-token buffer).  The row base
      // is then scalar and each lane adds its fixed offset.
      const int pg = page_of(ws, page_magic, page_shift);
      const int slot = ws - pg * p.page_size;
      const uint16_t* kb = nullptr;
      const uint16_t* vb = nullptr;
      if (ws + WROWS <= cache_end && slot + WROWS <= p.page_size) {
        // Consecutive tiles mostly stay in the same page: look the page up
        // only when it changes.
        if (pg != cached_pg) {
          const int page = __builtin_amdgcn_readfirstlane(bt_cache[pg - pg_base]);
          cached_base = (int64_t)page * p.page_size * kv_row_stride + (int64_t)g * D;
          cached_pg = pg;
        }
        const int64_t off = cached_base + (int64_t)slot * kv_row_stride;
        kb = kc_ptr + off;
        vb = vc_ptr + off;
      } else if (ws >= cache_end && ws + WROWS <= L) {
        const int64_t off = (int64_t)(q0 + ws - c) * kv_row_stride + (int64_t)g * D;
        kb = kn_ptr + off;
        vb = vn_ptr + off;
      }
      if (kb != nullptr) {
#pragma unroll
        for (int qi = 0; qi < C::DMA_PER_WAVE; ++qi) {
          const uint32_t dst = (uint32_t)((wave * C::DMA_PER_WAVE + qi) * 1024);
          dma16s(voff_k[qi], kb, kst + dst);
          dma16s(voff_v[qi], vb, vst + dst);
        }
        return;
      }
      // Otherwise per lane: cached position, new row, or past the end.
#pragma unroll
      for (int qi = 0; qi < C::DMA_PER_WAVE; ++qi) {
        const int id = wave * C::DMA_PER_WAVE + qi;
        const int r = id * Lay::ROWS_PER_DMA + lane_row;  // tile row of this lane
        const int j = j0 + r;
        const uint16_t* kp = zero_row;
        const uint16_t* vp = zero_row;
        if (j < cache_end) {
          const int pgl = page_of(j, page_magic, page_shift);
          const int slotl = j - pgl * p.page_size;
          const int page = bt_cache[pgl - pg_base];
          const int64_t off = ((int64_t)page * p.page_size + slotl) * kv_row_stride + (int64_t)g * D;
          kp = p.k_cache + off;
          vp = p.v_cache + off;
        } else if (j < L) {
          const int64_t off = (int64_t)(q0 + j - c) * kv_row_stride + (int64_t)g * D;
          kp = p.k_new + off;
          vp = p.v_new + off;
        }
        dma16(kp + 8 * Lay::kslot(r, lane_slot), kst + (uint32_t)(id * 1024));
        dma16(vp + 8 * Lay::vslot(r, lane_slot), vst + (uint32_t)(id * 1024));
      }
      return;
    }
#pragma unroll
    for (int qi = 0; qi < C::DMA_PER_WAVE; ++qi) {
      const int id = wave * C::DMA_PER_WAVE + qi;
      const int rbase = id * Lay::ROWS_PER_DMA;
      const int js = j0 + rbase;             // first key of this copy (wave-uniform)
      const int r = rbase + lane_row;         // tile row of this lane
      const int j = js + lane_row;
      const int je = js + Lay::ROWS_PER_DMA;  // one past the copy's last key
      const uint16_t* kp = zero_row;
      const uint16_t* vp = zero_row;
      // Common cases, decided per wave: every key of the copy in one cache
      // page, every key a new row, or every key past the sequence.  The row
      // base is then computed on the scalar unit.
      const uint32_t pg0 = (uint32_t)(((uint64_t)(uint32_t)js * p.page_magic) >> p.page_shift);
      const int slot0 = js - (int)pg0 * p.page_size;
      if (je <= cache_end && slot0 + Lay::ROWS_PER_DMA <= p.page_size) {
        const int page = scalar_load_i32(bt + pg0);
        const int64_t base = ((int64_t)page * p.page_size + slot0) * kv_row_stride + (int64_t)g * D;
        kp = p.k_cache + base + lane_row_off;
        vp = p.v_cache + base + lane_row_off;
      } else if (js >= cache_end && je <= L) {
        const int64_t base = (int64_t)(q0 + js - c) * kv_row_stride + (int64_t)g * D;
        kp = p.k_new + base + lane_row_off;
        vp = p.v_new + base + lane_row_off;
      } else if (js >= L) {
        // zero rows
      } else if (js < cache_end) {
        // block-table entries of the pages this copy touches, on the scalar unit
        const int jl = min(js + Lay::ROWS_PER_DMA, cache_end) - 1;
        const uint32_t pg_first = (uint32_t)(((uint64_t)(uint32_t)js * p.page_magic) >> p.page_shift);
        const uint32_t pg_last = (uint32_t)(((uint64_t)(uint32_t)jl * p.page_magic) >> p.page_shift);
        const uint32_t pg_l = (uint32_t)(((uint64_t)(uint32_t)j * p.page_magic) >> p.page_shift);
        int page_l = 0;
        for (uint32_t pg = pg_first; pg <= pg_last; ++pg) {
          const int page = scalar_load_i32(bt + pg);
          page_l = pg_l == pg ? page : page_l;
        }
        if (j < cache_end) {
          const int slot = j - (int)pg_l * p.page_size;
          const int64_t off = ((int64_t)page_l * p.page_size + slot) * kv_row_stride + (int64_t)g * D;
          kp = p.k_cache + off;
          vp = p.v_cache + off;
        }
      }
      if (js < L && !(je <= cache_end && slot0 + Lay::ROWS_PER_DMA <= p.page_size) &&
          !(js >= cache_end && je <= L) && j >= cache_end && j < L) {
        const int64_t off = (int64_t)(q0 + j - c) * kv_row_stride + (int64_t)g * D;
        kp = p.k_new + off;
        vp = p.v_new + off;
      }
      dma16(kp + 8 * Lay::kslot(r, lane_slot), kst + (uint32_t)(id * 1024));
      dma16(vp + 8 * Lay::vslot(r, lane_slot), vst + (uint32_t)(id * 1024));
    }
  };

  f32x16 oacc[RB][NDB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[rb][i] = f32x16{};
  // Scores s = q.k are accumulated exactly as the MFMA gives them (Q is the
  // unscaled bf16 input).  The softmax works in log2 units against a per-row
  // reference max m_run: p = exp2(s * c - m_run) with c = scale * log2(e), one
  // fp32 FMA per score feeding exp2 (the folding FlashAttention-2 describes,
  // Dao 2023).  m_run only moves when a row's max exceeds it by more than
  // kLazy (factor 2^kLazy), so the O rescale is rare; numerator and
  // denominator share the reference, and p <= 2^kLazy stays far from
  // overflow.  A row's m_run is -inf until its first unmasked key; meanwhile
  // its offset mi is 0.
  constexpr float kLazy = 8.f;
  const float c_log2 = p.scale_log2;
  float m_run[RB], mi[RB], l_run[RB];  // mi = -m_run once the row has one, else 0
  // A tile's row max (relative to m_run) above thr moves m_run: any key at all
  // while the row has none (thr = -inf), else a growth beyond 2^kLazy.
  float thr[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    thr[rb] = -INFINITY;
    mi[rb] = 0.f;
    l_run[rb] = 0.f;                   // running row sum (this lane half's keys)
  }

  // Lane-invariant LDS byte offsets of the operand reads (stage 0).
  // K (A operand of S^T): row `col` of each 32-key block, chunk 2ks + half.
  const uint32_t k_lane = smem_base + (uint32_t)(col * 2 * D + 16 * (half ^ Lay::kswz(col)));
  // V^T (A operand of O^T) via the transpose read: 16-lane group G reads rows
  // 16ks2 + 8r + 4(G/2) + j16/4 and dims 32db + 16(G%2) + 4(j16%4).
  const int grp = lane >> 4;
  const int j16 = lane & 15;
  const int v_row_in = 4 * (grp >> 1) + (j16 >> 2);
  const int v_dim_in = 16 * (grp & 1) + 4 * (j16 & 3);
  const uint32_t v_lane = smem_base + (uint32_t)(v_row_in * 2 * D +
                                                 16 * Lay::vslot(v_row_in, v_dim_in >> 3) +
                                                 2 * (v_dim_in & 7));

  // Ring protocol (NSTAGE = 4): tiles go in pairs, one pair per barrier.  The
  // pair of step i + 1 is copied while step i computes, into the stages of
  // step i - 1, which every wavefront left before the barrier of step i.
  static_assert(NSTAGE == 4, "ring protocol assumes four stages");
  const int ntile = tb.y - tb.x;
  if (ntile > 0) issue_tile(tb.x, 0);
  if (ntile > 1) issue_tile(tb.x + 1, 1);

  // ---- Q fragments: B operand of S^T = K Q^T, the exact bf16 input (rows
  // past the sequence are zero)
  bf16x8 qf[RB][KSTEPS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qf[rb][ks] = __builtin_bit_cast(bf16x8, valid[rb] ? qraw[rb][ks] : u32x4{0, 0, 0, 0});

  // ---- per-tile pieces
  auto tile_active = [&](int it) __attribute__((always_inline)) {
    const int j0 = (tb.x + it) * BN;
    return wave_active && j0 <= w_hi_max && j0 + BN - 1 >= w_lo_min;
  };
  // S^T[key][query] = K Q^T; accumulator element r of block kb holds key
  // j0 + 32kb + 8(r/4) + 4half + r%4 for this lane's query row.
  // k-step outer, key block inner: consecutive MFMAs are independent, and the
  // fragments of step ks+1 are read before the MFMAs of step ks are issued.
  auto qk = [&](int stage, f32x16 (*sacc)[NKB]) __attribute__((always_inline)) {
    uint32_t kbase = k_lane + (uint32_t)(stage * 2 * TILE_ELEMS * 2);
    // d = 256 keeps the per-read XORs in the loop (hoisting them spills there)
    if constexpr (D == 256) asm volatile("" : "+v"(kbase));
    auto kfrag = [&](int kb, int ks) __attribute__((always_inline)) {
      const uint32_t addr = (kbase + (uint32_t)(kb * 32 * D * 2)) ^ (uint32_t)(32 * ks);
      return *(const lds_u32x4*)(uintptr_t)addr;
    };
    // Fragment i = (k-step i / NKB, key block i % NKB).  Reads run QK_DEPTH
    // fragments ahead of the MFMA that consumes them, so LDS latency overlaps
    // the matrix pipe; the scheduling barriers keep the compiler from sinking
    // the reads next to their uses.
    constexpr int NF = KSTEPS * NKB;
    constexpr int PD = QK_DEPTH < NF ? QK_DEPTH : NF;
    u32x4 fr[PD];
#pragma unroll
    for (int i = 0; i < PD; ++i) fr[i] = kfrag(i % NKB, i / NKB);
    __builtin_amdgcn_sched_group_barrier(0x100, PD, 0);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const u32x4 a = fr[i % PD];
      if (i + PD < NF) fr[i % PD] = kfrag((i + PD) % NKB, (i + PD) / NKB);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        sacc[rb][i % NKB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, a), qf[rb][i / NKB],
            i < NKB ? f32x16{} : sacc[rb][i % NKB], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, RB, 0);
      if (i + PD < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  // Element mask (boundary tiles only), row max, lazy rescale of O and l.
  auto mask_rowmax = [&](int it, f32x16 (*sacc)[NKB]) __attribute__((always_inline)) {
    const int j0 = (tb.x + it) * BN;
    const bool interior = j0 >= w_lo_max && j0 + BN - 1 <= w_hi_min;
    if (!interior) {
      asm volatile("");  // keep this a branch: interior tiles skip the mask
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        // element (kb, r) holds key j0 + 4half + o with o = 32kb + 8(r/4) + r%4;
        // it is allowed iff (unsigned)(o - lo) <= (unsigned)(hi - lo), relative
        // to this lane's keys.
        const int lo = lo_a[rb] - j0 - 4 * half;
        const uint32_t width = (uint32_t)(hi_a[rb] - lo_a[rb]);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int o = kb * 32 + 8 * (r >> 2) + (r & 3);
            float v = sacc[rb][kb][r];
            v = (uint32_t)(o - lo) <= width ? v : -INFINITY;
            asm volatile("" : "+v"(v));
            sacc[rb][kb][r] = v;
          }
      }
    }
    float mx[RB];
    bool adj[RB];
    bool any_adj = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float m = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, sacc[rb][kb][r]);
      // the tile's row max in log2 units, relative to the reference (c > 0, so
      // the max commutes with the scaling; a fully masked row stays -inf)
      mx[rb] = fmaf(pair_max(m), c_log2, mi[rb]);
      // (d = 256 has no register to spare for thr and tests m_run instead)
      adj[rb] = D <= 128 ? mx[rb] > thr[rb]
                         : (m_run[rb] == -INFINITY ? mx[rb] > -INFINITY : mx[rb] > kLazy);
      any_adj |= adj[rb];
    }
    if (__builtin_amdgcn_ballot_w64(any_adj) != 0) {  // wave-uniform branch
      asm volatile("");  // keep this a branch: it is taken rarely
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const bool unset = m_run[rb] == -INFINITY;
        const float d = adj[rb] ? mx[rb] : 0.f;
        const float alpha = unset ? 1.f : __builtin_amdgcn_exp2f(-d);
        l_run[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[rb][db][r] *= alpha;
        m_run[rb] = unset ? (adj[rb] ? mx[rb] : m_run[rb]) : m_run[rb] + d;
        mi[rb] = m_run[rb] == -INFINITY ? 0.f : -m_run[rb];
        thr[rb] = m_run[rb] == -INFINITY ? -INFINITY : kLazy;
      }
    }
  };
  // p = exp2(s * scale * log2(e) - m_run) (one FMA into exp2), row sum, and
  // P^T as bf16 B operands (PV step ks2 covers keys 16ks2..16ks2+15).
  auto expsum = [&](f32x16 (*sacc)[NKB], bf16x8 (*pf)[PSTEPS]) __attribute__((always_inline)) {
    // The row sum adds the bf16-rounded p that the PV product uses.
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sacc[rb][kb][r] = __builtin_amdgcn_exp2f(fmaf(sacc[rb][kb][r], c_log2, mi[rb]));
#pragma unroll
      for (int ks2 = 0; ks2 < PSTEPS; ++ks2) {
        const f32x16& sv = sacc[rb][ks2 >> 1];
        const int o = 8 * (ks2 & 1);
        const f32x8 v = {sv[o + 0], sv[o + 1], sv[o + 2], sv[o + 3],
                         sv[o + 4], sv[o + 5], sv[o + 6], sv[o + 7]};
        const bf16x8 b = __builtin_convertvector(v, bf16x8);
        pf[rb][ks2] = b;
        float l = l_run[rb];
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(b, b, 0, 1), ones, l, false);
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(b, b, 2, 3), ones, l, false);
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(b, b, 4, 5), ones, l, false);
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(b, b, 6, 7), ones, l, false);
        l_run[rb] = l;
      }
    }
  };
  // O^T[dim][query] += V^T P^T.  A element e holds key 16ks2 + 8(e/4) + 4half + e%4 at
  // dim 32db + col: two transpose reads of 4 keys x 16 dims per 16-lane group.
  // Key step outer, dim block inner: consecutive MFMAs are independent; the
  // fragments of the next (ks2, db) pair are read one MFMA ahead.
  auto pv = [&](int stage, const bf16x8 (*pf)[PSTEPS]) __attribute__((always_inline)) {
    uint32_t vbase = v_lane + (uint32_t)((stage * 2 + 1) * TILE_ELEMS * 2);
    asm volatile("" : "+v"(vbase));
    auto vfrag = [&](int ks2, int db) __attribute__((always_inline)) {
      const uint32_t a0 = (vbase ^ (uint32_t)(64 * db)) + (uint32_t)(16 * ks2 * 2 * D);
      const uint32_t a1 = a0 + (uint32_t)(8 * 2 * D);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a0);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a1);
      const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
      const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
      return u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
    };
    // Fragment i = (key step i / NDB, dim block i % NDB), PV_DEPTH ahead.
    constexpr int NV = PSTEPS * NDB;
    constexpr int PD = PV_DEPTH < NV ? PV_DEPTH : NV;
    u32x4 fr[PD];
#pragma unroll
    for (int i = 0; i < PD; ++i) fr[i] = vfrag(i / NDB, i % NDB);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * PD, 0);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const u32x4 a = fr[i % PD];
      if (i + PD < NV) fr[i % PD] = vfrag((i + PD) / NDB, (i + PD) % NDB);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        oacc[rb][i % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, a), pf[rb][i / NDB], oacc[rb][i % NDB], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, RB, 0);
      if (i + PD < NV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  // Step i covers tiles 2i and 2i + 1: both for every wavefront, or in
  // KV-pair mode tile 2i + khalf for half khalf.  The copies of step i + 1
  // go into the stages of step i - 1, so they are issued after the barrier
  // of step i, once every wavefront has left step i - 1.
  for (int i = 0; 2 * i < ntile; ++i) {
    vm_wait<0>();
    block_barrier();
    // d <= 128: the copy of tile 2i + 2 + h goes behind the QK^T MFMAs of
    // tile 2i + h, so the workgroup's copies do not all queue for the address
    // unit right after the barrier.  (d = 256 issues both here: the live
    // scores would spill.)
    constexpr bool kCopyAfterQk = D <= 128;
    if constexpr (!kCopyAfterQk) {
      if (2 * i + 2 < ntile) issue_tile(tb.x + 2 * i + 2, (2 * i + 2) % NSTAGE);
      if (2 * i + 3 < ntile) issue_tile(tb.x + 2 * i + 3, (2 * i + 3) % NSTAGE);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int it = 2 * i + h;
      const bool run = !((pair && h != khalf) || it >= ntile || !tile_active(it));
      if constexpr (!kCopyAfterQk) {
        if (!run) continue;
      }
      f32x16 sacc[RB][NKB];
      bf16x8 pf[RB][PSTEPS];
      // Wave priority: 2 while the tile's QK^T MFMAs issue, 1 for the rest of
      // the tile, 0 after it.  The arbiter then favours a wavefront that is
      // starting a tile over its SIMD partner, whose softmax fills the matrix
      // pipe's shadow, and a wavefront in its tile over one between tiles.
      if constexpr (kCopyAfterQk) {
        if (run) {
          __builtin_amdgcn_s_setprio(2);
          qk(it % NSTAGE, sacc);
          __builtin_amdgcn_s_setprio(1);
        }
        if (2 * i + 2 + h < ntile) issue_tile(tb.x + 2 * i + 2 + h, (2 * i + 2 + h) % NSTAGE);
        if (!run) continue;
      } else {
        __builtin_amdgcn_s_setprio(2);
        qk(it % NSTAGE, sacc);
        __builtin_amdgcn_s_setprio(1);
      }
      mask_rowmax(it, sacc);
      expsum(sacc, pf);
      pv(it % NSTAGE, pf);
      __builtin_amdgcn_s_setprio(0);
    }
  }
  if (pair) {
    if constexpr (C::PAIR) {
      // Merge: the second half leaves (O, m, l) in the ring, laid out
      // [row block][register][lane]; the first half combines them with its own,
      // both rescaled to the larger reference max (log2 units).
      block_barrier();  // every wavefront is done reading tiles
      lds_f32* xb = (lds_f32*)(lds_u16*)&smem[0][0][0] + (wrow * C::XREGS) * 64 + lane;
      if (khalf == 1) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          lds_f32* xr = xb + rb * (NDB * 16 + 2) * 64;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) xr[(db * 16 + r) * 64] = oacc[rb][db][r];
          xr[NDB * 16 * 64] = m_run[rb];
          xr[(NDB * 16 + 1) * 64] = l_run[rb];
        }
      }
      block_barrier();
      if (khalf == 1) return;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const lds_f32* xr = xb + rb * (NDB * 16 + 2) * 64;
        const float m1 = xr[NDB * 16 * 64];
        const float l1 = xr[(NDB * 16 + 1) * 64];
        const float m0 = m_run[rb];
        const float mn = fmaxf(m0, m1);
        const float a0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m0 - mn);
        const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mn);
        l_run[rb] = l_run[rb] * a0 + l1 * a1;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            oacc[rb][db][r] = oacc[rb][db][r] * a0 + xr[(db * 16 + r) * 64] * a1;
        m_run[rb] = mn;
      }
    }
  }

  // ---- split-KV epilogue: the segment's unnormalised O with its reference max
  // m and sum l (log2 units), merged by merge_splits_kernel.
  if (!whole) {
    const int64_t rows = (int64_t)p.total_q_tokens * p.num_heads;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float l_tot = pair_sum(l_run[rb]);
      if (!valid[rb]) continue;
      const int64_t ri = (int64_t)split * rows + (int64_t)(q0 + tok[rb]) * p.num_heads + head[rb];
      if (half == 0) p.part_ml[ri] = make_float2(m_run[rb], l_tot);
      if (l_tot > 0.f) {
        float* orow = p.part_o + ri * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int b4 = 0; b4 < 4; ++b4) {
            const f32x16& o = oacc[rb][db];
            *(f32x4*)(orow + db * 32 + 8 * b4 + 4 * half) =
                f32x4{o[4 * b4], o[4 * b4 + 1], o[4 * b4 + 2], o[4 * b4 + 3]};
          }
      }
    }
    return;
  }
  // ---- epilogue, usual case: O / l -> bf16 staged through the (now idle)
  // ring, one row-major block of 32 * RB rows per wavefront, so that each
  // store writes whole rows (16 bytes per lane, D / 8 lanes per row).  A lane
  // holds dims 32db + 8b + 4half + 0..3 of its row; 16-byte chunk c of row r
  // sits at chunk c ^ (r % (D / 8)) of the row (conflict-free reads).
  if constexpr (C::STAGE_OUT) {
    if (!pair) {
      constexpr int CH = D / 8;               // 16-byte chunks per row
      constexpr int RPI = 64 / CH;            // rows per store instruction
      block_barrier();                        // every wavefront is done with the ring
      const uint32_t wbase = smem_base + (uint32_t)(wave * RB * 32 * D * 2);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float l_tot = pair_sum(l_run[rb]);
        if (p.kv_splits > 1 && valid[rb] && half == 0)
          p.part_ml[(int64_t)(q0 + tok[rb]) * p.num_heads + head[rb]] = make_float2(0.f, -1.f);
        const float inv = 1.f / l_tot;
        const int r = rb * 32 + col;
        const uint32_t rbase = wbase + (uint32_t)(r * D * 2 + 8 * half);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int b4 = 0; b4 < 4; ++b4) {
            const f32x16& o = oacc[rb][db];
            const f32x4 v = {o[4 * b4] * inv, o[4 * b4 + 1] * inv, o[4 * b4 + 2] * inv,
                             o[4 * b4 + 3] * inv};
            const uint32_t a = rbase + (uint32_t)((((4 * db + b4) ^ (r % CH)) * 16));
            *(lds_u32x2*)(uintptr_t)a =
                __builtin_bit_cast(u32x2, __builtin_convertvector(v, bf16x4));
          }
      }
      // Read back row-major: instruction i covers rows RPI*i + lane / CH.
      const int ch = lane % CH;
#pragma unroll
      for (int i = 0; i < RB * 32 / RPI; ++i) {
        const int r = RPI * i + lane / CH;
        const u32x4 v = *(const lds_u32x4*)(uintptr_t)(wbase + (uint32_t)(r * D * 2 +
                                                                     16 * (ch ^ (r % CH))));
        const int row = wrow * RB * 32 + r;  // tile row
        const int hb = row / p.block_q;
        const int tk = t * p.block_q + (row - hb * p.block_q);
        if (tk < n) {
          const int hd = g * p.group + hblk * p.heads_per_tile + hb;
          *(u32x4*)(p.out + ((int64_t)(q0 + tk) * p.num_heads + hd) * D + 8 * ch) = v;
        }
      }
      return;
    }
  }
  // ---- epilogue otherwise: O / l -> bf16.  A lane holds dims 32db + 8b + 4half + 0..3
  // (b = 0..3) of its row.  One v_permlane32_swap per dword gives lane half 0
  // dims 32db + 16e + 0..7 and half 1 dims 32db + 16e + 8..15 (e = 0, 1), so
  // every store writes 16 contiguous bytes per lane and 32 per row.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_tot = pair_sum(l_run[rb]);
    if (p.kv_splits > 1 && valid[rb] && half == 0) {
      // a whole item under split-KV: tell the merge that this row is final
      p.part_ml[(int64_t)(q0 + tok[rb]) * p.num_heads + head[rb]] = make_float2(0.f, -1.f);
    }
    const float inv = 1.f / l_tot;
    uint16_t* orow = p.out + ((int64_t)(q0 + tok[rb]) * p.num_heads + head[rb]) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const f32x16& o = oacc[rb][db];
        u32x2 w[2];  // bf16 of b = 2e and b = 2e + 1
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const int b4 = 2 * e + bb;
          const f32x4 v = {o[4 * b4] * inv, o[4 * b4 + 1] * inv, o[4 * b4 + 2] * inv,
                           o[4 * b4 + 3] * inv};
          w[bb] = __builtin_bit_cast(u32x2, __builtin_convertvector(v, bf16x4));
        }
        // the first half sends b = 2e + 1 and receives its partner's b = 2e;
        // the second half sends b = 2e and receives its partner's b = 2e + 1
        u32x4 st;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const auto r = __builtin_amdgcn_permlane32_swap(w[0][k], w[1][k], false, false);
          st[k] = half ? (uint32_t)r[0] : w[0][k];
          st[2 + k] = half ? w[1][k] : (uint32_t)r[1];
        }
        if (valid[rb]) *(u32x4*)(orow + db * 32 + 16 * e + 8 * half) = st;
      }
  }
}

// One lane per (sequence, Q tile): the loop range the attention kernel uses.
__global__ void tile_bounds_kernel(const int32_t* qsl, const int32_t* ctx_lens,
                                   const int32_t* mm_ranges, const int32_t* causal_per_seq,
                                   int num_seqs, int num_q_tiles, int block_q, int block_n,
                                   MaskSpec m, int num_ranges, int32_t* out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)num_seqs * num_q_tiles) return;
  const int s = (int)(idx / num_q_tiles);
  const int t = (int)(idx - (int64_t)s * num_q_tiles);
  const int n = qsl[s + 1] - qsl[s];
  const int32_t* ranges = num_ranges > 0 ? mm_ranges + (int64_t)s * num_ranges * 2 : nullptr;
  if (causal_per_seq != nullptr) m.causal = causal_per_seq[s];
  const int2 r = kv_tile_range(ctx_lens[s], n, t, block_q, block_n, m, ranges, num_ranges);
  out[2 * idx] = r.x;
  out[2 * idx + 1] = r.y;
}

// Device-side precondition check (one workgroup): every bit of the result
// names a precondition of prefill_attention that some sequence breaks.  The
// block-table entries are visited as a flat (sequence, page) index space so
// that long tables are shared by all lanes; only the entries the attention
// kernel would read are examined.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void check_metadata_kernel(const int32_t* block_table, const int32_t* qsl,
                           const int32_t* ctx_lens, int cache_only, int page_size,
                           int num_seqs, int total_q_tokens, int max_q_len, int num_pages,
                           int max_pages_per_seq, int32_t* flags_out) {
  __shared__ int flags;
  if (threadIdx.x == 0) flags = 0;
  __syncthreads();
  int f = 0;
  if (threadIdx.x == 0 && (qsl[0] != 0 || qsl[num_seqs] != total_q_tokens))
    f |= PAGED_PREFILL_BAD_QSL;
  for (int s = threadIdx.x; s < num_seqs; s += blockDim.x) {
    const int n = qsl[s + 1] - qsl[s];
    const int c = ctx_lens[s];
    if (n < 0) f |= PAGED_PREFILL_BAD_QSL;
    if (n > max_q_len) f |= PAGED_PREFILL_BAD_QLEN;
    if (c < 0) f |= PAGED_PREFILL_BAD_CTX;
    const int64_t L = (int64_t)max(c, 0) + max(n, 0);
    if (L > kMaxTokens) f |= PAGED_PREFILL_BAD_LENGTH;
    const int64_t cached = cache_only ? L : max(c, 0);
    if ((cached + page_size - 1) / page_size > max_pages_per_seq) f |= PAGED_PREFILL_BAD_PAGES;
  }
  const int64_t entries = (int64_t)num_seqs * max_pages_per_seq;
  for (int64_t i = threadIdx.x; i < entries; i += blockDim.x) {
    const int s = (int)(i / max_pages_per_seq);
    const int pg = (int)(i - (int64_t)s * max_pages_per_seq);
    const int64_t L = (int64_t)max(ctx_lens[s], 0) + max(qsl[s + 1] - qsl[s], 0);
    const int64_t cached = cache_only ? L : max(ctx_lens[s], 0);
    if ((int64_t)pg * page_size >= cached) continue;  // never read
    const int id = block_table[i];
    if (id < 0 || id >= num_pages) f |= PAGED_PREFILL_BAD_PAGE_ID;
  }
  if (f != 0) atomicOr(&flags, f);
  __syncthreads();
  if (threadIdx.x == 0) *flags_out = flags;
}

// Split-KV merge (log-sum-exp rule): for each (token, head) row,
//   out = sum_k 2^(m_k - M) O_k / sum_k 2^(m_k - M) l_k,  M = max over segments
// with l_k > 0.  Rows that segment 0 marked with l = -1 belong to an item that
// was not split; the attention kernel wrote them.  One thread per 8 output dims.
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void merge_splits_kernel(const float* part_o, const float2* part_ml, uint16_t* out,
                         int64_t rows, int splits) {
  constexpr int TPR = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / TPR;
  const int sub = (int)(gid - row * TPR);
  if (row >= rows) return;
  // segment 0 marks rows whose item was not split (l = -1): already final
  if (part_ml[row].y < 0.f) return;
  float M = -INFINITY;
  for (int k = 0; k < splits; ++k) {
    const float2 ml = part_ml[k * rows + row];
    if (ml.y > 0.f) M = fmaxf(M, ml.x);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int k = 0; k < splits; ++k) {
    const float2 ml = part_ml[k * rows + row];
    if (!(ml.y > 0.f)) continue;
    const float w = exp2f(ml.x - M);
    den += w * ml.y;
    const f32x4* src = (const f32x4*)(part_o + (k * rows + row) * D + sub * 8);
    const f32x4 a = src[0], b = src[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += w * a[e];
      acc[4 + e] += w * b[e];
    }
  }
  const float inv = 1.f / den;
  const f32x8 v = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv,
                   acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
  *(u32x4*)(out + row * D + sub * 8) = __builtin_bit_cast(u32x4, __builtin_convertvector(v, bf16x8));
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
struct TileChoice {
  int block_n;
  int heads_per_tile;
  int block_q;
  int wg_per_cu;  // workgroups resident per CU
  int many;       // d = 64 only: 1 = the shape for batches of many work items
};

int gcd_int(int a, int b) {
  while (b) {
    const int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

// Query rows and keys per KV tile of the shape compiled for a head size.
template <int D> void shape_of(int* rows, int* bn, int* wgs) {
  *rows = ShapeFor<D>::T::ROWS;
  *bn = ShapeFor<D>::T::BN;
  *wgs = ShapeFor<D>::T::WG_PER_CU;
}

int cu_count();

// Keys one query row sees at most when the window alone bounds it (the causal
// flag closes the right side), else -1.  Multimodal ranges, per-sequence causal
// flags and chunked masks are not counted: the geometry and split choices that
// use it are performance rules, and every entry point that needs them has these
// arguments in common.
int64_t window_span(int window_left, int window_right, int causal) {
  if (window_left < 0) return -1;
  if (causal) return (int64_t)window_left + 1;
  if (window_right < 0) return -1;
  return (int64_t)window_left + 1 + window_right;
}

// A window of at most this many keys per row makes every KV loop short.
constexpr int64_t kShortSpan = 2048;
bool short_loops(int window_left, int window_right, int causal) {
  const int64_t span = window_span(window_left, window_right, causal);
  return span >= 0 && span <= kShortSpan;
}

// The tile geometry for a head configuration and, at d = 64, the batch.  Both
// d = 64 shapes tile the queries alike; the many-items shape (32-key tiles,
// four workgroups per CU) overlaps each workgroup's prologue, epilogue and
// memory round trips with three others, while the default shape (64-key tiles,
// two per CU) halves the per-tile overhead of long KV loops and backfills a
// second round dynamically.  Measured on gfx950, the many-items shape wins when
// a short window bounds every loop and the Q-tile items (at most num_seqs *
// cdiv(max_q_len, block_q) per (KV head, head block) column) fill one round of
// its slots, or, for loops of any length, from four rounds of items up (at
// three rounds of long loops it still loses); the default shape wins below
// that.  num_seqs = max_q_len = 0: the default shape.
int choose_tiles(int head_size, int num_heads, int num_kv_heads, TileChoice* tc,
                 int num_seqs = 0, int max_q_len = 0, int window_left = -1,
                 int window_right = -1, int causal = 1) {
  if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0)
    return PAGED_PREFILL_ERR_INVALID_ARG;
  if (head_size != 64 && head_size != 128 && head_size != 256)
    return PAGED_PREFILL_ERR_UNSUPPORTED;
  int rows, bn, wgs;
  if (head_size == 64) shape_of<64>(&rows, &bn, &wgs);
  else if (head_size == 128) shape_of<128>(&rows, &bn, &wgs);
  else shape_of<256>(&rows, &bn, &wgs);
  const int group = num_heads / num_kv_heads;
  const int hpt = gcd_int(group, rows);  // heads of one group that share a tile
  tc->block_n = bn;
  tc->heads_per_tile = hpt;
  tc->block_q = rows / hpt;
  tc->wg_per_cu = wgs;
  tc->many = 0;
  if (head_size == 64 && num_seqs > 0 && max_q_len > 0) {
    using M = ShapeD64Many::T;
    static_assert(M::ROWS == ShapeFor<64>::T::ROWS, "both d = 64 shapes tile the queries alike");
    const int64_t items = (int64_t)num_seqs * ((max_q_len + tc->block_q - 1) / tc->block_q) *
                          num_kv_heads * (group / hpt);
    const int64_t slots = (int64_t)cu_count() * M::WG_PER_CU;
    if ((short_loops(window_left, window_right, causal) && items >= slots) ||
        items >= 4 * slots) {
      tc->block_n = M::BN;
      tc->wg_per_cu = M::WG_PER_CU;
      tc->many = 1;
    }
  }
  return PAGED_PREFILL_OK;
}

struct Options {
  const int32_t* causal_per_seq = nullptr;
  int32_t mm_clamp = 1;
  int32_t chunk_size = 0;
  int32_t chunk_lookback = -1;
  int32_t kv_splits = 1;
  void* workspace = nullptr;
  uint64_t workspace_bytes = 0;
  // The workspace is the library's static scratch: an automatic split count
  // whose partials do not fit falls back to no split, an explicit one fails
  // with PAGED_PREFILL_ERR_SCRATCH.
  bool static_scratch = false;
};

// Device address of `scratch` on the current device, looked up once per device
// with that device current and kept for every later call.
constexpr int kMaxDevices = 64;
std::once_flag g_cu_once[kMaxDevices];
int g_cu_count[kMaxDevices];

// CUs of the current device, asked once per device (256 on MI355X, and
// assumed when there is no device to ask).
int cu_count() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  std::call_once(g_cu_once[dev], [dev] {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    g_cu_count[dev] = cus;
  });
  return g_cu_count[dev];
}

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

int scratch_for_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PAGED_PREFILL_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PAGED_PREFILL_ERR_UNSUPPORTED;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr)
    return PAGED_PREFILL_ERR_HIP;
  *ptr = g_scratch_ptr[dev];
  return PAGED_PREFILL_OK;
}

constexpr int kMaxSplits = 64;

int validate(const void* q, const void* k_new, const void* v_new, const void* k_cache,
             const void* v_cache, const int32_t* block_table, const int32_t* qsl,
             const int32_t* ctx_lens, int32_t num_heads, int32_t num_kv_heads,
             int32_t head_size, int32_t page_size, int32_t window_left, int32_t window_right,
             int32_t causal, const int32_t* mm_ranges, float scale, const void* out,
             int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len, int32_t num_pages,
             int32_t max_pages_per_seq, int32_t max_mm_ranges) {
  if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0)
    return PAGED_PREFILL_ERR_INVALID_ARG;
  if (page_size <= 0 || num_seqs < 0 || total_q_tokens < 0 || max_q_len < 0 ||
      num_pages < 0 || max_pages_per_seq < 0)
    return PAGED_PREFILL_ERR_INVALID_ARG;
  if (window_left < -1 || window_right < -1 || (causal != 0 && causal != 1))
    return PAGED_PREFILL_ERR_INVALID_ARG;
  if (!(scale > 0.f) || scale != scale || scale > 3.0e38f) return PAGED_PREFILL_ERR_INVALID_ARG;
  if (max_mm_ranges < 0 || max_mm_ranges > kMaxMmRanges) return PAGED_PREFILL_ERR_INVALID_ARG;
  if (max_mm_ranges > 0 && mm_ranges == nullptr) return PAGED_PREFILL_ERR_INVALID_ARG;
  if ((k_new == nullptr) != (v_new == nullptr)) return PAGED_PREFILL_ERR_INVALID_ARG;
  if (head_size != 64 && head_size != 128 && head_size != 256)
    return PAGED_PREFILL_ERR_UNSUPPORTED;
  if (page_size > 65536) return PAGED_PREFILL_ERR_UNSUPPORTED;
  if ((int64_t)max_pages_per_seq * page_size > kMaxTokens || max_q_len > kMaxTokens)
    return PAGED_PREFILL_ERR_INVALID_ARG;
  if (num_seqs == 0 || total_q_tokens == 0 || max_q_len == 0) return PAGED_PREFILL_OK;
  if (q == nullptr || out == nullptr || block_table == nullptr || qsl == nullptr ||
      ctx_lens == nullptr || k_cache == nullptr || v_cache == nullptr)
    return PAGED_PREFILL_ERR_INVALID_ARG;
  return PAGED_PREFILL_OK;
}

int validate_mask_options(const Options& o) {
  if (o.mm_clamp != 0 && o.mm_clamp != 1) return PAGED_PREFILL_ERR_INVALID_ARG;
  if (o.chunk_size < 0 || o.chunk_lookback < -1) return PAGED_PREFILL_ERR_INVALID_ARG;
  if (o.chunk_size > kMaxTokens) return PAGED_PREFILL_ERR_INVALID_ARG;
  return PAGED_PREFILL_OK;
}

void page_magic(int page_size, uint32_t* magic, int* shift) {
  int l = 0;
  while ((1 << l) < page_size) ++l;  // l = ceil(log2(page_size))
  const uint64_t num = (uint64_t)1 << (24 + l);
  *magic = (uint32_t)((num + page_size - 1) / page_size);
  *shift = 24 + l;
}

// Workgroups per split before the split factor: 8 XCDs x slots per XCD.
int64_t item_slots(int num_seqs, int num_kv_heads, int64_t num_q_tiles, int head_blocks,
                   int total_q_tokens, int block_q) {
  if (num_seqs <= kSortMaxSeqs) {
    // items dealt round-robin over the XCDs: at most one per (sequence, KV
    // head, Q tile, head block), rounded up to whole rounds.  The Q tiles are
    // at most S * cdiv(max_q_len, block_q) and at most (T + S (block_q - 1)) /
    // block_q; slots past the batch's items exit at once.
    const int64_t tiles = std::min<int64_t>(
        (int64_t)num_seqs * num_q_tiles,
        ((int64_t)total_q_tokens + (int64_t)num_seqs * (block_q - 1)) / block_q);
    const int64_t items = tiles * num_kv_heads * head_blocks;
    return (items + kNumXcd - 1) / kNumXcd * kNumXcd;
  }
  // large batches: per XCD a contiguous range of (sequence, KV head) groups,
  // each with up to num_q_tiles tiles
  const int64_t groups_per_xcd = ((int64_t)num_seqs * num_kv_heads + kNumXcd - 1) / kNumXcd;
  return kNumXcd * groups_per_xcd * num_q_tiles * head_blocks;
}

// Split count for kv_splits (0 = automatic).  The Q tiles of the batch number
// at most num_seqs * cdiv(max_q_len, block_q) and at most sum over s of
// cdiv(n_s, block_q) <= (T + S (block_q - 1)) / block_q; times the KV heads and
// head blocks, that bounds the work items.  Automatic choice:
//  - a whole number of rounds (at least one): no split, there is no partial
//    round to even out;
//  - at most half of round_slots items: split every long item (the segment-cap
//    rule) into k segments, k * items filling one round (see below), at most
//    16;
//  - more than half but fewer than twice round_slots items: split every long
//    item to about 2 * round_slots workgroups, at most 16 segments; in both
//    cases no
//    split when a short window bounds the loops: the cap (a share of the
//    longest sequence's tiles) then exceeds every item, so nothing would be cut
//    and the extra slots and the merge would only cost time;
//  - two to four rounds of items whose bound leaves a last round at most a
//    quarter full, for batches whose items the kernel ranks (num_seqs <=
//    kSortMaxSeqs): tail splitting with kTailSplits segments, which cuts only
//    the items of that short last round (the kernel counts them exactly);
//  - otherwise no split.
constexpr int kTailSplits = 4;
struct SplitChoice {
  int splits;
  int tail;  // 1: tail splitting
};
SplitChoice choose_splits(int kv_splits, int num_seqs, int num_kv_heads, int head_blocks,
                          int64_t num_q_tiles, int total_q_tokens, int block_q,
                          int round_slots, bool short_window) {
  if (kv_splits > 0 || round_slots <= 0) return {kv_splits > 0 ? kv_splits : 1, 0};
  const int64_t tiles = std::min<int64_t>(
      (int64_t)num_seqs * num_q_tiles,
      ((int64_t)total_q_tokens + (int64_t)num_seqs * (block_q - 1)) / block_q);
  const int64_t items = tiles * num_kv_heads * head_blocks;
  if (items <= 0) return {1, 0};
  if (items >= round_slots && items % round_slots == 0) return {1, 0};
  if (items < 2 * (int64_t)round_slots) {
    if (short_window) return {1, 0};
    if (2 * items <= round_slots) {
      // At most half a round of items: one round of segments.  Equal items
      // cut k ways take one segment's time per round, so a partial second
      // round costs as much as a full one; the largest k that keeps to one
      // round is taken if it fills at least 3/4 of the slots, else one more.
      int64_t k = round_slots / items;
      if (4 * items * k < 3 * (int64_t)round_slots) ++k;
      return {(int)std::min<int64_t>(16, k), 0};
    }
    return {(int)std::min<int64_t>(16, (2 * (int64_t)round_slots + items - 1) / items), 0};
  }
  const int64_t tail = items % round_slots;
  if (num_seqs <= kSortMaxSeqs && items <= 4 * (int64_t)round_slots && tail > 0 &&
      tail <= round_slots / 4)
    return {kTailSplits, 1};
  return {1, 0};
}

// Workgroups that run at once: CUs of the current device times the workgroups
// one CU holds.
int round_slots_for(const TileChoice& tc) { return cu_count() * tc.wg_per_cu; }

uint64_t workspace_bytes_for(int num_heads, int head_size, int total_q_tokens, int splits) {
  if (splits <= 1) return 0;
  const uint64_t rows = (uint64_t)splits * (uint64_t)total_q_tokens * (uint64_t)num_heads;
  const uint64_t o_bytes = (rows * head_size * sizeof(float) + 255) & ~(uint64_t)255;
  return o_bytes + rows * 2 * sizeof(float);
}

template <typename C>
hipError_t launch(const KernelArgs& a, uint32_t grid, hipStream_t stream) {
  constexpr int D = C::D;
  void* args[] = {(void*)&a};
  hipError_t err = hipLaunchKernel((const void*)&prefill_attention_kernel<C>, dim3(grid),
                                   dim3(C::THREADS), args, 0, stream);
  if (err != hipSuccess || a.kv_splits <= 1) return err;
  const int64_t rows = (int64_t)a.total_q_tokens * a.num_heads;
  const int64_t threads = rows * (D / 8);
  const float* po = a.part_o;
  const float2* pml = a.part_ml;
  uint16_t* out = a.out;
  int64_t r = rows;
  int k = a.kv_splits;
  void* margs[] = {(void*)&po, (void*)&pml, (void*)&out, (void*)&r, (void*)&k};
  return hipLaunchKernel((const void*)&merge_splits_kernel<D>,
                         dim3((uint32_t)((threads + 255) / 256)), dim3(256), margs, 0, stream);
}

int run(const void* q, const void* k_new, const void* v_new, const void* k_cache,
        const void* v_cache, const int32_t* block_table, const int32_t* query_start_loc,
        const int32_t* ctx_lens, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
        int32_t page_size, int32_t window_left, int32_t window_right, int32_t causal,
        const int32_t* mm_ranges, float scale, void* out, int32_t num_seqs,
        int32_t total_q_tokens, int32_t max_q_len, int32_t num_pages,
        int32_t max_pages_per_seq, int32_t max_mm_ranges, const Options& o,
        hipStream_t stream) {
  int rc = validate(q, k_new, v_new, k_cache, v_cache, block_table, query_start_loc, ctx_lens,
                    num_heads, num_kv_heads, head_size, page_size, window_left, window_right,
                    causal, mm_ranges, scale, out, num_seqs, total_q_tokens, max_q_len,
                    num_pages, max_pages_per_seq, max_mm_ranges);
  if (rc != PAGED_PREFILL_OK) return rc;
  rc = validate_mask_options(o);
  if (rc != PAGED_PREFILL_OK) return rc;
  if (o.kv_splits < 0 || o.kv_splits > kMaxSplits) return PAGED_PREFILL_ERR_INVALID_ARG;
  if (num_seqs == 0 || total_q_tokens == 0 || max_q_len == 0) return PAGED_PREFILL_OK;
  TileChoice tc;
  rc = choose_tiles(head_size, num_heads, num_kv_heads, &tc, num_seqs, max_q_len, window_left,
                    window_right, causal);
  if (rc != PAGED_PREFILL_OK) return rc;

  KernelArgs a;
  a.q = (const uint16_t*)q;
  a.k_new = (const uint16_t*)k_new;
  a.v_new = (const uint16_t*)v_new;
  a.k_cache = (const uint16_t*)k_cache;
  a.v_cache = (const uint16_t*)v_cache;
  a.block_table = block_table;
  a.qsl = query_start_loc;
  a.ctx_lens = ctx_lens;
  a.mm_ranges = max_mm_ranges > 0 ? mm_ranges : nullptr;
  a.out = (uint16_t*)out;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_heads / num_kv_heads;
  a.heads_per_tile = tc.heads_per_tile;
  a.head_blocks = a.group / tc.heads_per_tile;
  a.block_q = tc.block_q;
  a.page_size = page_size;
  page_magic(page_size, &a.page_magic, &a.page_shift);
  a.window_left = window_left;
  a.window_right = window_right;
  a.causal = causal;
  a.scale_log2 = scale * 1.4426950408889634f;  // log2(e)
  a.num_seqs = num_seqs;
  a.max_pages_per_seq = max_pages_per_seq;
  a.max_mm_ranges = max_mm_ranges;
  a.cache_only = k_new == nullptr ? 1 : 0;
  a.causal_per_seq = o.causal_per_seq;
  a.mm_clamp = o.mm_clamp;
  a.chunk_size = o.chunk_size;
  a.chunk_lookback = o.chunk_lookback;
  a.total_q_tokens = total_q_tokens;

  const int64_t num_q_tiles = ((int64_t)max_q_len + tc.block_q - 1) / tc.block_q;
  a.num_q_tiles = (int32_t)num_q_tiles;
  // the automatic split count needs the device's CU count (one runtime query)
  const int round_slots = o.kv_splits == 0 ? round_slots_for(tc) : 0;
  SplitChoice sc = choose_splits(o.kv_splits, num_seqs, num_kv_heads, a.head_blocks,
                                 num_q_tiles, total_q_tokens, tc.block_q, round_slots,
                                 short_loops(window_left, window_right, causal));
  if (o.static_scratch && sc.splits > 1 &&
      workspace_bytes_for(num_heads, head_size, total_q_tokens, sc.splits) > o.workspace_bytes) {
    if (o.kv_splits != 0) return PAGED_PREFILL_ERR_SCRATCH;
    sc = {1, 0};  // automatic: the partials would not fit the scratch, so no split
  }
  const int splits = sc.splits;
  a.kv_splits = splits;
  a.tail_mode = sc.tail;
  a.round_slots = round_slots;
  a.part_o = nullptr;
  a.part_ml = nullptr;
  if (splits > 1) {
    const uint64_t need = workspace_bytes_for(num_heads, head_size, total_q_tokens, splits);
    if (o.workspace == nullptr || o.workspace_bytes < need) return PAGED_PREFILL_ERR_INVALID_ARG;
    const uint64_t rows = (uint64_t)splits * total_q_tokens * num_heads;
    const uint64_t o_bytes = (rows * head_size * sizeof(float) + 255) & ~(uint64_t)255;
    a.part_o = (float*)o.workspace;
    a.part_ml = (float2*)((char*)o.workspace + o_bytes);
  }
  const int64_t main_slots = item_slots(num_seqs, num_kv_heads, num_q_tiles, a.head_blocks,
                                        total_q_tokens, tc.block_q);
  // tail splitting: one slot per item, then one round of helper slots
  const int64_t grid = sc.tail ? main_slots + round_slots : main_slots * splits;
  if (grid > 0x7fffffff) return PAGED_PREFILL_ERR_UNSUPPORTED;
  a.main_slots = (int32_t)main_slots;
  hipError_t err;
  switch (head_size) {
    case 64:
      err = tc.many ? launch<ShapeD64Many::T>(a, (uint32_t)grid, stream)
                    : launch<ShapeFor<64>::T>(a, (uint32_t)grid, stream);
      break;
    case 128: err = launch<ShapeFor<128>::T>(a, (uint32_t)grid, stream); break;
    default: err = launch<ShapeFor<256>::T>(a, (uint32_t)grid, stream); break;
  }
  return err == hipSuccess ? PAGED_PREFILL_OK : PAGED_PREFILL_ERR_HIP;
}

int run_tile_bounds(const int32_t* query_start_loc, const int32_t* ctx_lens, int32_t num_heads,
                    int32_t num_kv_heads, int32_t head_size, int32_t window_left,
                    int32_t window_right, int32_t causal, const int32_t* mm_ranges,
                    int32_t num_seqs, int32_t max_q_len, int32_t max_mm_ranges,
                    const Options& o, int32_t* bounds_out, hipStream_t stream) {
  TileChoice tc;
  int rc = choose_tiles(head_size, num_heads, num_kv_heads, &tc, num_seqs, max_q_len,
                        window_left, window_right, causal);
  if (rc != PAGED_PREFILL_OK) return rc;
  if (num_seqs < 0 || max_q_len < 0 || max_q_len > kMaxTokens || window_left < -1 ||
      window_right < -1 || (causal != 0 && causal != 1) || max_mm_ranges < 0 ||
      max_mm_ranges > kMaxMmRanges || (max_mm_ranges > 0 && mm_ranges == nullptr))
    return PAGED_PREFILL_ERR_INVALID_ARG;
  rc = validate_mask_options(o);
  if (rc != PAGED_PREFILL_OK) return rc;
  const int64_t num_q_tiles = ((int64_t)max_q_len + tc.block_q - 1) / tc.block_q;
  const int64_t total = num_q_tiles * num_seqs;
  if (total == 0) return PAGED_PREFILL_OK;
  if (query_start_loc == nullptr || ctx_lens == nullptr || bounds_out == nullptr)
    return PAGED_PREFILL_ERR_INVALID_ARG;
  if (total > 0x7fffffffLL) return PAGED_PREFILL_ERR_UNSUPPORTED;
  const int threads = 256;
  const uint32_t blocks = (uint32_t)((total + threads - 1) / threads);
  const int32_t* mm = max_mm_ranges > 0 ? mm_ranges : nullptr;
  const int32_t* cps = o.causal_per_seq;
  int ns = num_seqs, nt = (int)num_q_tiles, bq = tc.block_q, bn = tc.block_n;
  MaskSpec m{causal, window_left, window_right, o.chunk_size, o.chunk_lookback, o.mm_clamp};
  int nr = max_mm_ranges;
  void* args[] = {(void*)&query_start_loc, (void*)&ctx_lens, (void*)&mm, (void*)&cps,
                  (void*)&ns, (void*)&nt, (void*)&bq, (void*)&bn, (void*)&m, (void*)&nr,
                  (void*)&bounds_out};
  const hipError_t err = hipLaunchKernel((const void*)&tile_bounds_kernel, dim3(blocks),
                                         dim3(threads), args, 0, stream);
  return err == hipSuccess ? PAGED_PREFILL_OK : PAGED_PREFILL_ERR_HIP;
}

int run_check_metadata(const int32_t* block_table, const int32_t* query_start_loc,
                       const int32_t* ctx_lens, int32_t cache_only, int32_t page_size,
                       int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len,
                       int32_t num_pages, int32_t max_pages_per_seq, int32_t* flags_out,
                       hipStream_t stream) {
  if (query_start_loc == nullptr || flags_out == nullptr || (cache_only != 0 && cache_only != 1))
    return PAGED_PREFILL_ERR_INVALID_ARG;
  if (page_size <= 0 || num_seqs < 0 || total_q_tokens < 0 || max_q_len < 0 || num_pages < 0 ||
      max_pages_per_seq < 0)
    return PAGED_PREFILL_ERR_INVALID_ARG;
  if (num_seqs > 0 && ctx_lens == nullptr) return PAGED_PREFILL_ERR_INVALID_ARG;
  if ((int64_t)num_seqs * max_pages_per_seq > 0 && block_table == nullptr)
    return PAGED_PREFILL_ERR_INVALID_ARG;
  int cm = cache_only, ps = page_size, ns = num_seqs, tq = total_q_tokens, mq = max_q_len,
      np = num_pages, mp = max_pages_per_seq;
  void* args[] = {(void*)&block_table, (void*)&query_start_loc, (void*)&ctx_lens, (void*)&cm,
                  (void*)&ps, (void*)&ns, (void*)&tq, (void*)&mq, (void*)&np, (void*)&mp,
                  (void*)&flags_out};
  const hipError_t err = hipLaunchKernel((const void*)&check_metadata_kernel, dim3(1),
                                         dim3(256), args, 0, stream);
  return err == hipSuccess ? PAGED_PREFILL_OK : PAGED_PREFILL_ERR_HIP;
}

Options make_options(const int32_t* causal_per_seq, int32_t mm_clamp, int32_t chunk_size,
                     int32_t chunk_lookback, int32_t kv_splits, void* workspace,
                     uint64_t workspace_bytes) {
  Options o;
  o.causal_per_seq = causal_per_seq;
  o.mm_clamp = mm_clamp;
  o.chunk_size = chunk_size;
  o.chunk_lookback = chunk_lookback;
  o.kv_splits = kv_splits;
  o.workspace = workspace;
  o.workspace_bytes = workspace_bytes;
  return o;
}

}  // namespace

extern "C" {

const char* prefill_attention_strerror(int code) {
  switch (code) {
    case PAGED_PREFILL_OK: return "ok";
    case PAGED_PREFILL_ERR_INVALID_ARG: return "invalid argument";
    case PAGED_PREFILL_ERR_UNSUPPORTED: return "unsupported configuration";
    case PAGED_PREFILL_ERR_HIP: return "HIP runtime error at launch";
    case PAGED_PREFILL_ERR_SCRATCH:
      return "split-KV partials exceed the static scratch of prefill_attention_ex_noalloc";
    default: return "unknown error code";
  }
}

int prefill_attention_validate(const void* q, const void* k_new, const void* v_new,
                               const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* query_start_loc,
                               const int32_t* ctx_lens, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_size, int32_t page_size,
                               int32_t window_left, int32_t window_right, int32_t causal,
                               const int32_t* mm_ranges, float scale, const void* out,
                               int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len,
                               int32_t num_pages, int32_t max_pages_per_seq,
                               int32_t max_mm_ranges) {
  return validate(q, k_new, v_new, k_cache, v_cache, block_table, query_start_loc, ctx_lens,
                  num_heads, num_kv_heads, head_size, page_size, window_left, window_right,
                  causal, mm_ranges, scale, out, num_seqs, total_q_tokens, max_q_len,
                  num_pages, max_pages_per_seq, max_mm_ranges);
}

int prefill_attention_tile_config(int32_t head_size, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t* block_q, int32_t* block_n) {
  return prefill_attention_tile_config_ex(head_size, num_heads, num_kv_heads, 0, 0, -1, -1, 1,
                                          block_q, block_n);
}

int prefill_attention_tile_config_ex(int32_t head_size, int32_t num_heads, int32_t num_kv_heads,
                                     int32_t num_seqs, int32_t max_q_len, int32_t window_left,
                                     int32_t window_right, int32_t causal, int32_t* block_q,
                                     int32_t* block_n) {
  if (block_q == nullptr || block_n == nullptr || num_seqs < 0 || max_q_len < 0 ||
      window_left < -1 || window_right < -1 || (causal != 0 && causal != 1))
    return PAGED_PREFILL_ERR_INVALID_ARG;
  TileChoice tc;
  const int rc = choose_tiles(head_size, num_heads, num_kv_heads, &tc, num_seqs, max_q_len,
                              window_left, window_right, causal);
  if (rc != PAGED_PREFILL_OK) return rc;
  *block_q = tc.block_q;
  *block_n = tc.block_n;
  return PAGED_PREFILL_OK;
}

int prefill_attention(const void* q, const void* k_new, const void* v_new,
                      const void* k_cache, const void* v_cache, const int32_t* block_table,
                      const int32_t* query_start_loc, const int32_t* ctx_lens,
                      int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                      int32_t page_size, int32_t window_left, int32_t window_right,
                      int32_t causal, const int32_t* mm_ranges, float scale, void* out,
                      int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len,
                      int32_t num_pages, int32_t max_pages_per_seq, int32_t max_mm_ranges,
                      hipStream_t stream) {
  return run(q, k_new, v_new, k_cache, v_cache, block_table, query_start_loc, ctx_lens,
             num_heads, num_kv_heads, head_size, page_size, window_left, window_right, causal,
             mm_ranges, scale, out, num_seqs, total_q_tokens, max_q_len, num_pages,
             max_pages_per_seq, max_mm_ranges, Options(), stream);
}

int prefill_attention_ex(const void* q, const void* k_new, const void* v_new,
                         const void* k_cache, const void* v_cache, const int32_t* block_table,
                         const int32_t* query_start_loc, const int32_t* ctx_lens,
                         int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                         int32_t page_size, int32_t window_left, int32_t window_right,
                         int32_t causal, const int32_t* mm_ranges, float scale, void* out,
                         int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len,
                         int32_t num_pages, int32_t max_pages_per_seq, int32_t max_mm_ranges,
                         const int32_t* causal_per_seq, int32_t mm_clamp, int32_t chunk_size,
                         int32_t chunk_lookback, int32_t kv_splits, void* workspace,
                         uint64_t workspace_bytes, hipStream_t stream) {
  return run(q, k_new, v_new, k_cache, v_cache, block_table, query_start_loc, ctx_lens,
             num_heads, num_kv_heads, head_size, page_size, window_left, window_right, causal,
             mm_ranges, scale, out, num_seqs, total_q_tokens, max_q_len, num_pages,
             max_pages_per_seq, max_mm_ranges,
             make_options(causal_per_seq, mm_clamp, chunk_size, chunk_lookback, kv_splits,
                          workspace, workspace_bytes),
             stream);
}

int prefill_attention_ex_noalloc(const void* q, const void* k_new, const void* v_new,
                                 const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* query_start_loc,
                                 const int32_t* ctx_lens, int32_t num_heads,
                                 int32_t num_kv_heads, int32_t head_size, int32_t page_size,
                                 int32_t window_left, int32_t window_right, int32_t causal,
                                 const int32_t* mm_ranges, float scale, void* out,
                                 int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len,
                                 int32_t num_pages, int32_t max_pages_per_seq,
                                 int32_t max_mm_ranges, const int32_t* causal_per_seq,
                                 int32_t mm_clamp, int32_t chunk_size, int32_t chunk_lookback,
                                 int32_t kv_splits, hipStream_t stream) {
  // the host-side argument checks first, so that a bad call needs no device
  int rc = validate(q, k_new, v_new, k_cache, v_cache, block_table, query_start_loc, ctx_lens,
                    num_heads, num_kv_heads, head_size, page_size, window_left, window_right,
                    causal, mm_ranges, scale, out, num_seqs, total_q_tokens, max_q_len,
                    num_pages, max_pages_per_seq, max_mm_ranges);
  if (rc != PAGED_PREFILL_OK) return rc;
  Options o = make_options(causal_per_seq, mm_clamp, chunk_size, chunk_lookback, kv_splits,
                           nullptr, PAGED_PREFILL_NOALLOC_SCRATCH_BYTES);
  o.static_scratch = true;
  rc = validate_mask_options(o);
  if (rc != PAGED_PREFILL_OK) return rc;
  if (kv_splits < 0 || kv_splits > kMaxSplits) return PAGED_PREFILL_ERR_INVALID_ARG;
  if (num_seqs == 0 || total_q_tokens == 0 || max_q_len == 0) return PAGED_PREFILL_OK;
  rc = scratch_for_current_device(&o.workspace);
  if (rc != PAGED_PREFILL_OK) return rc;
  return run(q, k_new, v_new, k_cache, v_cache, block_table, query_start_loc, ctx_lens,
             num_heads, num_kv_heads, head_size, page_size, window_left, window_right, causal,
             mm_ranges, scale, out, num_seqs, total_q_tokens, max_q_len, num_pages,
             max_pages_per_seq, max_mm_ranges, o, stream);
}

int prefill_attention_kv_splits(int32_t head_size, int32_t num_heads, int32_t num_kv_heads,
                                int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len,
                                int32_t window_left, int32_t window_right, int32_t causal,
                                int32_t kv_splits) {
  if (kv_splits < 0 || kv_splits > kMaxSplits || num_seqs < 0 || total_q_tokens < 0 ||
      max_q_len < 0 || window_left < -1 || window_right < -1 || (causal != 0 && causal != 1))
    return PAGED_PREFILL_ERR_INVALID_ARG;
  TileChoice tc;
  const int rc = choose_tiles(head_size, num_heads, num_kv_heads, &tc, num_seqs, max_q_len,
                              window_left, window_right, causal);
  if (rc != PAGED_PREFILL_OK) return rc;
  const int64_t num_q_tiles = ((int64_t)max_q_len + tc.block_q - 1) / tc.block_q;
  return choose_splits(kv_splits, num_seqs, num_kv_heads,
                       num_heads / num_kv_heads / tc.heads_per_tile, num_q_tiles,
                       total_q_tokens, tc.block_q, kv_splits == 0 ? round_slots_for(tc) : 0,
                       short_loops(window_left, window_right, causal)).splits;
}

uint64_t prefill_attention_workspace_size(int32_t num_heads, int32_t head_size,
                                          int32_t total_q_tokens, int32_t splits) {
  if (num_heads <= 0 || head_size <= 0 || total_q_tokens < 0 || splits < 0) return 0;
  return workspace_bytes_for(num_heads, head_size, total_q_tokens, splits);
}

int prefill_attention_tile_bounds(const int32_t* query_start_loc, const int32_t* ctx_lens,
                                  int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                  int32_t window_left, int32_t window_right, int32_t causal,
                                  const int32_t* mm_ranges, int32_t num_seqs,
                                  int32_t max_q_len, int32_t max_mm_ranges,
                                  int32_t* bounds_out, hipStream_t stream) {
  return run_tile_bounds(query_start_loc, ctx_lens, num_heads, num_kv_heads, head_size,
                         window_left, window_right, causal, mm_ranges, num_seqs, max_q_len,
                         max_mm_ranges, Options(), bounds_out, stream);
}

int prefill_attention_tile_bounds_ex(const int32_t* query_start_loc, const int32_t* ctx_lens,
                                     int32_t num_heads, int32_t num_kv_heads,
                                     int32_t head_size, int32_t window_left,
                                     int32_t window_right, int32_t causal,
                                     const int32_t* mm_ranges, int32_t num_seqs,
                                     int32_t max_q_len, int32_t max_mm_ranges,
                                     const int32_t* causal_per_seq, int32_t mm_clamp,
                                     int32_t chunk_size, int32_t chunk_lookback,
                                     int32_t* bounds_out, hipStream_t stream) {
  return run_tile_bounds(query_start_loc, ctx_lens, num_heads, num_kv_heads, head_size,
                         window_left, window_right, causal, mm_ranges, num_seqs, max_q_len,
                         max_mm_ranges,
                         make_options(causal_per_seq, mm_clamp, chunk_size, chunk_lookback, 1,
                                      nullptr, 0),
                         bounds_out, stream);
}

int prefill_attention_check_metadata(const int32_t* block_table,
                                     const int32_t* query_start_loc, const int32_t* ctx_lens,
                                     int32_t cache_only, int32_t page_size, int32_t num_seqs,
                                     int32_t total_q_tokens, int32_t max_q_len,
                                     int32_t num_pages, int32_t max_pages_per_seq,
                                     int32_t* flags_out, hipStream_t stream) {
  return run_check_metadata(block_table, query_start_loc, ctx_lens, cache_only, page_size,
                            num_seqs, total_q_tokens, max_q_len, num_pages, max_pages_per_seq,
                            flags_out, stream);
}

}  // extern "C"
