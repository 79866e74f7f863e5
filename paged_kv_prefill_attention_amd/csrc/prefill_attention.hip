// Paged-KV prefill attention for MI355X (gfx950, CDNA4).
//
// One workgroup (4 wavefronts, 256 lanes) owns one Q tile: `block_q` query
// tokens of one sequence times the `heads_per_tile` query heads of one GQA
// group that it packs into 128 MFMA rows, so one K/V gather serves every head
// of the group.  The workgroup walks the KV tiles [lo, hi) given by the tile
// bound calculator (the window unioned with every multimodal range that
// overlaps the tile's queries; vLLM PR #50776 report, "Key source snippets";
// vLLM PR #53147 report, "Implementation breakdown" item 2).  Per KV tile:
//
//   1. page-offset resolver: key position j < ctx_len is slot j % P of page
//      block_table[j / P] (division by an invariant integer with a
//      Granlund-Montgomery multiply-shift, PLDI 1994), j >= ctx_len is a row of
//      the chunk's new K/V; tiles never depend on pages, so any page size works
//      (vLLM PR #54194 report, "Features and motivation");
//   2. coalesced 16-byte gather of K and V rows into LDS (K row-major, V
//      transposed so the PV contraction reads keys contiguously);
//   3. S^T = K Q^T on v_mfma_f32_32x32x16_bf16: every lane ends up holding
//      one query row's scores, so softmax row reductions are in-lane plus one
//      exchange with the lane 32 away;
//   4. the element mask, only on tiles that are not provably all-allowed;
//   5. online softmax in the exp2 domain (Milakov & Gimelshein 2018, with the
//      scale folded into exp2 as in FlashAttention-2, Dao 2023);
//   6. O^T += V^T P^T on the same MFMA, P rounded to bf16 (round-to-nearest-
//      even, v_cvt_pk_bf16_f32).
// The epilogue divides by the row sum and stores bf16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "paged_prefill.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;  // MFMA rows (query token x head pairs) per workgroup
constexpr int kMaxTokens = 1 << 24; // positions per sequence the resolver handles exactly
constexpr int kMaxMmRanges = 4096;

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
  int32_t block_q;         // query tokens per Q tile = kRows / heads_per_tile
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
};

// ---------------------------------------------------------------------------
// Tile bound calculator.  Query rows of tile t are [t*block_q, min(..., n)-1];
// the base window runs from a_lo - window_left (key 0 without a left window)
// to a_hi (causal), a_hi + window_right, or the last key; every valid range
// [st, en] (st < en) overlapping [a_lo, a_hi] may lower the left edge to
// max(st, a_lo - window_left) and raise the right edge to en; the result is
// clamped to [0, L-1] and converted to KV tiles of `block_n` keys.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int2 kv_tile_range(int c, int n, int t, int block_q, int block_n,
                                              int causal, int wl, int wr,
                                              const int32_t* ranges, int num_ranges) {
  const int i_lo = t * block_q;
  if (i_lo >= n) return make_int2(0, 0);
  const int i_hi = min(i_lo + block_q - 1, n - 1);
  const int L = c + n;
  const int a_lo = c + i_lo;
  const int a_hi = c + i_hi;
  int first = wl >= 0 ? a_lo - wl : 0;
  int last = causal ? a_hi : (wr >= 0 ? a_hi + min(wr, L) : L - 1);
  for (int r = 0; r < num_ranges; ++r) {
    const int st = ranges[2 * r];
    const int en = ranges[2 * r + 1];
    if (st < en && st <= a_hi && en >= a_lo) {
      first = min(first, wl >= 0 ? max(st, a_lo - wl) : st);
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
__device__ __forceinline__ void row_interval(int a, int L, int causal, int wl, int wr,
                                             const int32_t* ranges, int num_ranges,
                                             int& lo, int& hi) {
  lo = wl >= 0 ? a - wl : 0;
  hi = causal ? a : (wr >= 0 ? a + min(wr, L) : L - 1);
  for (int r = 0; r < num_ranges; ++r) {
    const int st = ranges[2 * r];
    const int en = ranges[2 * r + 1];
    if (st < en && st <= a && a <= en) {
      lo = min(lo, wl >= 0 ? max(st, a - wl) : st);
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

__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

// Element offset of key position j (KV head g) in the cache or the new rows;
// -1 when j is past the sequence (the row is zero-filled, never read).
__device__ __forceinline__ int64_t key_offset(const KernelArgs& p, int s, int g, int j, int c,
                                              int L, int q0, int D, bool& from_cache) {
  from_cache = false;
  if (j >= L) return -1;
  const int cache_end = p.cache_only ? L : c;
  if (j < cache_end) {
    from_cache = true;
    const uint32_t pg = (uint32_t)(((uint64_t)(uint32_t)j * p.page_magic) >> p.page_shift);
    const int slot = j - (int)pg * p.page_size;
    const int page = p.block_table[(int64_t)s * p.max_pages_per_seq + pg];
    return (((int64_t)page * p.page_size + slot) * p.num_kv_heads + g) * D;
  }
  return ((int64_t)(q0 + j - c) * p.num_kv_heads + g) * D;
}

template <int D, int BN>
struct Tile {
  static constexpr int KLD = D + 8;    // K row stride in LDS (elements): 16 B pad
  static constexpr int VLD = BN + 4;   // V^T row stride in LDS (elements): 8 B pad
  static constexpr int CHUNKS = D / 8; // 16-byte chunks per key row
  static constexpr int QUADS = (BN / 4) * CHUNKS;  // (4 keys x 8 dims) loader units
  static constexpr int QPT = QUADS / kThreads;     // units per lane
  static_assert(QUADS % kThreads == 0, "tile must split evenly over the workgroup");
  static_assert(BN % 32 == 0 && D % 32 == 0, "MFMA blocking");
};

template <int D, int BN, int WAVES_PER_EU>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(WAVES_PER_EU, WAVES_PER_EU)))
void prefill_attention_kernel(const KernelArgs p) {
  using T = Tile<D, BN>;
  constexpr int KSTEPS = D / 16;   // QK^T contraction steps of 16 dims
  constexpr int NKB = BN / 32;     // 32-key blocks per KV tile
  constexpr int PSTEPS = BN / 16;  // PV contraction steps of 16 keys
  constexpr int NDB = D / 32;      // 32-dim blocks of the output
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[BN * T::KLD];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[D * T::VLD];

  // ---- work decode: blockIdx -> (Q tile from the end, sequence, head block)
  const int HB = p.num_kv_heads * p.head_blocks;
  int b = blockIdx.x;
  const int hb_all = b % HB;
  b /= HB;
  const int s = b % p.num_seqs;
  const int z = b / p.num_seqs;
  const int q0 = p.qsl[s];
  const int n = p.qsl[s + 1] - q0;
  const int ntiles = (n + p.block_q - 1) / p.block_q;
  if (z >= ntiles) return;  // padding tile of a shorter sequence
  const int t = ntiles - 1 - z;  // heaviest (last) tiles are dispatched first
  const int c = p.ctx_lens[s];
  const int L = c + n;
  const int g = hb_all / p.head_blocks;
  const int hblk = hb_all % p.head_blocks;
  const int R = p.max_mm_ranges;
  const int32_t* ranges = R > 0 ? p.mm_ranges + (int64_t)s * R * 2 : nullptr;

  const int2 tb = kv_tile_range(c, n, t, p.block_q, BN, p.causal, p.window_left,
                                p.window_right, ranges, R);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;

  // ---- this lane's query row (both lane halves hold the same row)
  const int row = wave * 32 + col;
  const int hb = row / p.block_q;
  const int tok = t * p.block_q + (row - hb * p.block_q);
  const bool valid = tok < n;
  const int head = g * p.group + hblk * p.heads_per_tile + hb;
  int lo_a = 1, hi_a = 0;
  if (valid)
    row_interval(c + tok, L, p.causal, p.window_left, p.window_right, ranges, R, lo_a, hi_a);
  const int w_lo_max = wave_max(valid ? lo_a : INT_MIN);
  const int w_hi_min = wave_min(valid ? hi_a : INT_MAX);
  const int w_lo_min = wave_min(valid ? lo_a : INT_MAX);
  const int w_hi_max = wave_max(valid ? hi_a : INT_MIN);
  const bool wave_active = w_hi_max != INT_MIN;

  // ---- Q fragments: B operand of S^T = K Q^T (lane: row `col`, dims 16ks + 8half..+8)
  bf16x8 qf[KSTEPS];
  {
    const uint16_t* qrow = p.q + ((int64_t)(q0 + (valid ? tok : 0)) * p.num_heads + head) * D;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4 v = valid ? *(const u32x4*)(qrow + 16 * ks + 8 * half) : u32x4{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;  // running row max of scale*log2(e)*score
  float l_run = 0.f;        // running row sum (this lane half's keys)

  // ---- loader: each lane moves T::QPT units of 4 consecutive keys x 8 dims
  u32x4 kreg[T::QPT][4];
  u32x4 vreg[T::QPT][4];
  auto load_tile = [&](int tile) {
    const int j0 = tile * BN;
#pragma unroll
    for (int u = 0; u < T::QPT; ++u) {
      const int unit = tid + u * kThreads;
      const int kq = unit / T::CHUNKS;
      const int kc = unit - kq * T::CHUNKS;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bool from_cache;
        const int64_t off = key_offset(p, s, g, j0 + 4 * kq + i, c, L, q0, D, from_cache);
        if (off < 0) {
          kreg[u][i] = u32x4{0, 0, 0, 0};
          vreg[u][i] = u32x4{0, 0, 0, 0};
        } else {
          const uint16_t* kb = from_cache ? p.k_cache : p.k_new;
          const uint16_t* vb = from_cache ? p.v_cache : p.v_new;
          kreg[u][i] = *(const u32x4*)(kb + off + 8 * kc);
          vreg[u][i] = *(const u32x4*)(vb + off + 8 * kc);
        }
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < T::QPT; ++u) {
      const int unit = tid + u * kThreads;
      const int kq = unit / T::CHUNKS;
      const int kc = unit - kq * T::CHUNKS;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(u32x4*)(k_lds + (4 * kq + i) * T::KLD + 8 * kc) = kreg[u][i];
      // 4 keys x 8 dims -> 8 rows of V^T, 4 consecutive keys each
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const u32x2 even = {pack_lo16(vreg[u][0][e2], vreg[u][1][e2]),
                            pack_lo16(vreg[u][2][e2], vreg[u][3][e2])};
        const u32x2 odd = {pack_hi16(vreg[u][0][e2], vreg[u][1][e2]),
                           pack_hi16(vreg[u][2][e2], vreg[u][3][e2])};
        *(u32x2*)(v_lds + (8 * kc + 2 * e2) * T::VLD + 4 * kq) = even;
        *(u32x2*)(v_lds + (8 * kc + 2 * e2 + 1) * T::VLD + 4 * kq) = odd;
      }
    }
  };

  if (tb.x < tb.y) load_tile(tb.x);
  for (int tile = tb.x; tile < tb.y; ++tile) {
    __syncthreads();  // every wave is done reading the previous tile
    store_tile();
    __syncthreads();
    if (tile + 1 < tb.y) load_tile(tile + 1);  // in flight during this tile's math
    const int j0 = tile * BN;
    if (!wave_active || j0 > w_hi_max || j0 + BN - 1 < w_lo_min) continue;
    const bool interior = j0 >= w_lo_max && j0 + BN - 1 <= w_hi_min;

    // S^T[key][query] = K Q^T
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const u32x4 a = *(const u32x4*)(k_lds + (kb * 32 + col) * T::KLD + 16 * ks + 8 * half);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                          qf[ks], sacc[kb], 0, 0, 0);
      }
    }
    // accumulator element r of block kb holds key j0 + 32kb + 8(r/4) + 4half + r%4
    if (!interior) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key < lo_a || key > hi_a) sacc[kb][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * p.scale_log2);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], p.scale_log2, -m_use));
        sacc[kb][r] = e;
        rs += e;
      }
    l_run = l_run * alpha + rs;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    // P^T as B operands: PV step ks2 covers keys 16ks2..16ks2+15
    bf16x8 pf[PSTEPS];
#pragma unroll
    for (int ks2 = 0; ks2 < PSTEPS; ++ks2) {
      const f32x8 v = {sacc[ks2 >> 1][8 * (ks2 & 1) + 0], sacc[ks2 >> 1][8 * (ks2 & 1) + 1],
                       sacc[ks2 >> 1][8 * (ks2 & 1) + 2], sacc[ks2 >> 1][8 * (ks2 & 1) + 3],
                       sacc[ks2 >> 1][8 * (ks2 & 1) + 4], sacc[ks2 >> 1][8 * (ks2 & 1) + 5],
                       sacc[ks2 >> 1][8 * (ks2 & 1) + 6], sacc[ks2 >> 1][8 * (ks2 & 1) + 7]};
      pf[ks2] = __builtin_convertvector(v, bf16x8);
    }
    // O^T[dim][query] += V^T P^T; A element e holds key 16ks2 + 8(e/4) + 4half + e%4
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ks2 = 0; ks2 < PSTEPS; ++ks2) {
        const uint16_t* vp = v_lds + (db * 32 + col) * T::VLD + 16 * ks2 + 4 * half;
        const u32x2 lo = *(const u32x2*)vp;
        const u32x2 hi = *(const u32x2*)(vp + 8);
        const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                          pf[ks2], oacc[db], 0, 0, 0);
      }
  }

  // ---- epilogue: O / l -> bf16; lane holds dims 32db + 8(r/4) + 4half + r%4
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (valid) {
    const float inv = 1.f / l_tot;
    uint16_t* orow = p.out + ((int64_t)(q0 + tok) * p.num_heads + head) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        const f32x4 v = {oacc[db][4 * b4] * inv, oacc[db][4 * b4 + 1] * inv,
                         oacc[db][4 * b4 + 2] * inv, oacc[db][4 * b4 + 3] * inv};
        const bf16x4 h = __builtin_convertvector(v, bf16x4);
        *(u32x2*)(orow + db * 32 + 8 * b4 + 4 * half) = __builtin_bit_cast(u32x2, h);
      }
  }
}

// One lane per (sequence, Q tile): the loop range the attention kernel uses.
__global__ void tile_bounds_kernel(const int32_t* qsl, const int32_t* ctx_lens,
                                   const int32_t* mm_ranges, int num_seqs, int num_q_tiles,
                                   int block_q, int block_n, int causal, int wl, int wr,
                                   int num_ranges, int32_t* out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)num_seqs * num_q_tiles) return;
  const int s = (int)(idx / num_q_tiles);
  const int t = (int)(idx - (int64_t)s * num_q_tiles);
  const int n = qsl[s + 1] - qsl[s];
  const int32_t* ranges = num_ranges > 0 ? mm_ranges + (int64_t)s * num_ranges * 2 : nullptr;
  const int2 r = kv_tile_range(ctx_lens[s], n, t, block_q, block_n, causal, wl, wr, ranges,
                               num_ranges);
  out[2 * idx] = r.x;
  out[2 * idx + 1] = r.y;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
struct TileChoice {
  int block_n;
  int heads_per_tile;
  int block_q;
};

int gcd_int(int a, int b) {
  while (b) {
    const int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

int choose_tiles(int head_size, int num_heads, int num_kv_heads, TileChoice* tc) {
  if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0)
    return PAGED_PREFILL_ERR_INVALID_ARG;
  int bn;
  switch (head_size) {
    case 64: bn = 128; break;
    case 128: bn = 64; break;
    case 256: bn = 32; break;
    default: return PAGED_PREFILL_ERR_UNSUPPORTED;
  }
  const int group = num_heads / num_kv_heads;
  const int hpt = gcd_int(group, kRows);  // heads of one group that share a tile
  tc->block_n = bn;
  tc->heads_per_tile = hpt;
  tc->block_q = kRows / hpt;
  return PAGED_PREFILL_OK;
}

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

void page_magic(int page_size, uint32_t* magic, int* shift) {
  int l = 0;
  while ((1 << l) < page_size) ++l;  // l = ceil(log2(page_size))
  const uint64_t num = (uint64_t)1 << (24 + l);
  *magic = (uint32_t)((num + page_size - 1) / page_size);
  *shift = 24 + l;
}

template <int D, int BN, int W>
hipError_t launch(const KernelArgs& a, uint32_t grid, hipStream_t stream) {
  void* args[] = {(void*)&a};
  return hipLaunchKernel((const void*)&prefill_attention_kernel<D, BN, W>, dim3(grid),
                         dim3(kThreads), args, 0, stream);
}

}  // namespace

extern "C" {

const char* prefill_attention_strerror(int code) {
  switch (code) {
    case PAGED_PREFILL_OK: return "ok";
    case PAGED_PREFILL_ERR_INVALID_ARG: return "invalid argument";
    case PAGED_PREFILL_ERR_UNSUPPORTED: return "unsupported configuration";
    case PAGED_PREFILL_ERR_HIP: return "HIP runtime error at launch";
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
  if (block_q == nullptr || block_n == nullptr) return PAGED_PREFILL_ERR_INVALID_ARG;
  TileChoice tc;
  const int rc = choose_tiles(head_size, num_heads, num_kv_heads, &tc);
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
  int rc = validate(q, k_new, v_new, k_cache, v_cache, block_table, query_start_loc, ctx_lens,
                    num_heads, num_kv_heads, head_size, page_size, window_left, window_right,
                    causal, mm_ranges, scale, out, num_seqs, total_q_tokens, max_q_len,
                    num_pages, max_pages_per_seq, max_mm_ranges);
  if (rc != PAGED_PREFILL_OK) return rc;
  if (num_seqs == 0 || total_q_tokens == 0 || max_q_len == 0) return PAGED_PREFILL_OK;
  TileChoice tc;
  rc = choose_tiles(head_size, num_heads, num_kv_heads, &tc);
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

  const int64_t num_q_tiles = ((int64_t)max_q_len + tc.block_q - 1) / tc.block_q;
  const int64_t grid = num_q_tiles * num_seqs * num_kv_heads * a.head_blocks;
  if (grid > 0x7fffffff) return PAGED_PREFILL_ERR_UNSUPPORTED;
  hipError_t err;
  switch (head_size) {
    case 64: err = launch<64, 128, 2>(a, (uint32_t)grid, stream); break;
    case 128: err = launch<128, 64, 2>(a, (uint32_t)grid, stream); break;
    default: err = launch<256, 32, 1>(a, (uint32_t)grid, stream); break;
  }
  return err == hipSuccess ? PAGED_PREFILL_OK : PAGED_PREFILL_ERR_HIP;
}

int prefill_attention_tile_bounds(const int32_t* query_start_loc, const int32_t* ctx_lens,
                                  int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                  int32_t window_left, int32_t window_right, int32_t causal,
                                  const int32_t* mm_ranges, int32_t num_seqs,
                                  int32_t max_q_len, int32_t max_mm_ranges,
                                  int32_t* bounds_out, hipStream_t stream) {
  TileChoice tc;
  int rc = choose_tiles(head_size, num_heads, num_kv_heads, &tc);
  if (rc != PAGED_PREFILL_OK) return rc;
  if (num_seqs < 0 || max_q_len < 0 || max_q_len > kMaxTokens || window_left < -1 ||
      window_right < -1 || (causal != 0 && causal != 1) || max_mm_ranges < 0 ||
      max_mm_ranges > kMaxMmRanges || (max_mm_ranges > 0 && mm_ranges == nullptr))
    return PAGED_PREFILL_ERR_INVALID_ARG;
  const int64_t num_q_tiles = ((int64_t)max_q_len + tc.block_q - 1) / tc.block_q;
  const int64_t total = num_q_tiles * num_seqs;
  if (total == 0) return PAGED_PREFILL_OK;
  if (query_start_loc == nullptr || ctx_lens == nullptr || bounds_out == nullptr)
    return PAGED_PREFILL_ERR_INVALID_ARG;
  if (total > 0x7fffffffLL) return PAGED_PREFILL_ERR_UNSUPPORTED;
  const int threads = 256;
  const uint32_t blocks = (uint32_t)((total + threads - 1) / threads);
  const int32_t* mm = max_mm_ranges > 0 ? mm_ranges : nullptr;
  int ns = num_seqs, nt = (int)num_q_tiles, bq = tc.block_q, bn = tc.block_n;
  int cz = causal, wl = window_left, wr = window_right, nr = max_mm_ranges;
  void* args[] = {(void*)&query_start_loc, (void*)&ctx_lens, (void*)&mm, (void*)&ns,
                  (void*)&nt, (void*)&bq, (void*)&bn, (void*)&cz, (void*)&wl, (void*)&wr,
                  (void*)&nr, (void*)&bounds_out};
  const hipError_t err = hipLaunchKernel((const void*)&tile_bounds_kernel, dim3(blocks),
                                         dim3(threads), args, 0, stream);
  return err == hipSuccess ? PAGED_PREFILL_OK : PAGED_PREFILL_ERR_HIP;
}

}  // extern "C"
