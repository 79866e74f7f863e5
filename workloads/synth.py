"""Seeded synthetic workloads (input creation only, no attention arithmetic).

Recipe (shared by tests, ``smoke()`` and ``bench.py``):

* ``numpy.random.default_rng(seed)`` draws, in this order: context lengths,
  new-token lengths (inclusive uniform ranges), multimodal-prefix ranges, then
  for every sequence ``q`` [n, H, d], logical ``K`` [L, Hkv, d] and logical
  ``V`` [L, Hkv, d], all N(0, 1) in fp32 and rounded to bf16
  (round-to-nearest-even).  Precision tests widen Q and K to N(0, sigma^2)
  (``qk_sigma``), which reaches realistic logit magnitudes.
* The page layout comes from a *separate* stream ``default_rng(table_seed)``:
  a random permutation of the physical pool hands each sequence its pages in
  order.  The pool holds the pages that are needed plus ``spare_frac`` spare
  pages.  Logical K/V are drawn before the layout, so two page sizes with the
  same ``seed`` hold identical logical tensors.
* Every slot that holds no token of any sequence is poisoned with bf16 NaN;
  block-table entries that name no page are -1.  With ``new_in_cache=False``
  (the default) the new-token slots of the last context page are poison too,
  so a kernel that reads the cache where it should read ``k_new`` shows NaN.

Arrays are returned as raw bf16 bit patterns (``uint16``); ``bf16_bits_to_f32``
widens them exactly.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, IEEE-754 round-to-nearest-even; NaN -> 0x7FC0."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[np.isnan(x)] = BF16_NAN
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the exact fp32 values they encode."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


@dataclasses.dataclass
class Workload:
    """One batch of paged-prefill inputs, in the layout the C ABI takes."""

    name: str
    num_heads: int
    num_kv_heads: int
    head_size: int
    page_size: int
    causal: bool
    window_left: int
    window_right: int
    scale: float
    ctx_lens: np.ndarray          # int32 [S]
    q_lens: np.ndarray            # int32 [S]
    query_start_loc: np.ndarray   # int32 [S+1]
    block_table: np.ndarray       # int32 [S][max_pages_per_seq], -1 = no page
    mm_ranges: Optional[np.ndarray]  # int32 [S][R][2] inclusive [start, end], or None
    q: np.ndarray                 # uint16 bf16 bits [T][H][d]
    k_new: np.ndarray             # uint16 bf16 bits [T][Hkv][d]
    v_new: np.ndarray             # uint16 bf16 bits [T][Hkv][d]
    k_cache: np.ndarray           # uint16 bf16 bits [num_pages][P][Hkv][d]
    v_cache: np.ndarray           # uint16 bf16 bits [num_pages][P][Hkv][d]
    new_in_cache: bool = False
    seed: int = 0
    table_seed: int = 0
    causal_per_seq: Optional[np.ndarray] = None  # int32 [S] 0/1; overrides ``causal``
    mm_clamp: bool = True         # multimodal ranges clamped by window_left
    chunk_size: int = 0           # chunked local attention when > 0 ...
    chunk_lookback: int = -1      # ... and >= 0

    @property
    def causal_arg(self):
        """The causal setting as the oracle takes it: one flag, or one per sequence."""
        return self.causal if self.causal_per_seq is None else self.causal_per_seq

    def mask_kwargs(self) -> dict:
        return dict(chunk_size=self.chunk_size, chunk_lookback=self.chunk_lookback,
                    mm_clamp=self.mm_clamp)

    @property
    def num_seqs(self) -> int:
        return int(self.ctx_lens.shape[0])

    @property
    def total_q_tokens(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.q_lens.size else 0

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_mm_ranges(self) -> int:
        return 0 if self.mm_ranges is None else int(self.mm_ranges.shape[1])

    def seq_lens(self) -> np.ndarray:
        return (self.ctx_lens.astype(np.int64) + self.q_lens).astype(np.int64)

    def f32(self, field: str) -> np.ndarray:
        return bf16_bits_to_f32(getattr(self, field))

    def mm_list(self, s: int) -> list:
        """Ranges of sequence ``s`` as a list of (start, end) python ints."""
        if self.mm_ranges is None:
            return []
        return [(int(a), int(b)) for a, b in self.mm_ranges[s]]


def make_workload(*, seed: int, table_seed: Optional[int] = None, ctx_lens, q_lens,
                  num_heads: int, num_kv_heads: int, head_size: int, page_size: int,
                  causal: bool, window_left: int = -1, window_right: int = -1,
                  mm_ranges=None, scale: Optional[float] = None,
                  spare_frac: float = 0.1, new_in_cache: bool = False,
                  block_table_override=None, name: str = "custom",
                  rng: Optional[np.random.Generator] = None, causal_per_seq=None,
                  mm_clamp: bool = True, chunk_size: int = 0,
                  chunk_lookback: int = -1, qk_sigma: float = 1.0) -> Workload:
    """Build a workload from explicit lengths; tensors are drawn from ``rng``
    (or ``default_rng(seed)``), the page layout from ``default_rng(table_seed)``.

    ``qk_sigma`` widens Q and K to N(0, qk_sigma^2) before the bf16 rounding
    (V stays N(0, 1)); with 1.0 the bits are those of the plain draw."""
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32).reshape(-1)
    q_lens = np.asarray(q_lens, dtype=np.int32).reshape(-1)
    assert ctx_lens.shape == q_lens.shape
    S = ctx_lens.shape[0]
    H, Hkv, d, P = num_heads, num_kv_heads, head_size, page_size
    if rng is None:
        rng = np.random.default_rng(seed)
    if table_seed is None:
        table_seed = seed + 1
    qsl = np.zeros(S + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(q_lens)
    T = int(qsl[-1])
    L = ctx_lens.astype(np.int64) + q_lens

    q_bits = np.empty((T, H, d), dtype=np.uint16)
    k_new = np.empty((T, Hkv, d), dtype=np.uint16)
    v_new = np.empty((T, Hkv, d), dtype=np.uint16)
    logical_k, logical_v = [], []
    for s in range(S):
        n, c, Ls = int(q_lens[s]), int(ctx_lens[s]), int(L[s])
        qf = rng.standard_normal((n, H, d), dtype=np.float32)
        kf = rng.standard_normal((Ls, Hkv, d), dtype=np.float32)
        if qk_sigma != 1.0:
            qf *= np.float32(qk_sigma)
            kf *= np.float32(qk_sigma)
        qs = f32_to_bf16_bits(qf)
        ks = f32_to_bf16_bits(kf)
        vs = f32_to_bf16_bits(rng.standard_normal((Ls, Hkv, d), dtype=np.float32))
        q_bits[qsl[s]:qsl[s + 1]] = qs
        k_new[qsl[s]:qsl[s + 1]] = ks[c:]
        v_new[qsl[s]:qsl[s + 1]] = vs[c:]
        logical_k.append(ks)
        logical_v.append(vs)

    # Paged layout (separate stream).
    in_cache = [int(L[s]) if new_in_cache else int(ctx_lens[s]) for s in range(S)]
    pages_needed = [_cdiv(x, P) for x in in_cache]
    trng = np.random.default_rng(table_seed)
    if block_table_override is not None:
        bt = np.asarray(block_table_override, dtype=np.int32).reshape(S, -1).copy()
        num_pages = int(bt.max()) + 1
        for s in range(S):
            assert bt.shape[1] >= pages_needed[s]
    else:
        total = sum(pages_needed)
        num_pages = max(1, total + int(math.ceil(spare_frac * total)))
        perm = trng.permutation(num_pages).astype(np.int32)
        width = max(1, max(pages_needed) if S else 1)
        bt = np.full((S, width), -1, dtype=np.int32)
        off = 0
        for s in range(S):
            bt[s, :pages_needed[s]] = perm[off:off + pages_needed[s]]
            off += pages_needed[s]
    k_cache = np.full((num_pages, P, Hkv, d), BF16_NAN, dtype=np.uint16)
    v_cache = np.full((num_pages, P, Hkv, d), BF16_NAN, dtype=np.uint16)
    for s in range(S):
        for p in range(pages_needed[s]):
            t0, t1 = p * P, min((p + 1) * P, in_cache[s])
            k_cache[bt[s, p], :t1 - t0] = logical_k[s][t0:t1]
            v_cache[bt[s, p], :t1 - t0] = logical_v[s][t0:t1]

    mm = None
    if mm_ranges is not None:
        mm = np.asarray(mm_ranges, dtype=np.int32).reshape(S, -1, 2)
        if mm.shape[1] == 0:
            mm = None
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return Workload(name=name, num_heads=H, num_kv_heads=Hkv, head_size=d, page_size=P,
                    causal=bool(causal), window_left=int(window_left),
                    window_right=int(window_right), scale=float(scale),
                    ctx_lens=ctx_lens, q_lens=q_lens, query_start_loc=qsl,
                    block_table=bt, mm_ranges=mm, q=q_bits, k_new=k_new, v_new=v_new,
                    k_cache=k_cache, v_cache=v_cache, new_in_cache=new_in_cache,
                    seed=seed, table_seed=table_seed,
                    causal_per_seq=(None if causal_per_seq is None else
                                    np.asarray(causal_per_seq, dtype=np.int32).reshape(S)),
                    mm_clamp=bool(mm_clamp), chunk_size=int(chunk_size),
                    chunk_lookback=int(chunk_lookback))


# The five benchmark workloads.  Shapes follow the pages' own test shapes and
# benchmark runs; the values are synthetic.
CONFIGS = {
    1: dict(name="tiny_paged_prefill", S=1, ctx=(32, 32), new=(48, 48), H=4, Hkv=2, d=64,
            P=16, causal=True, wl=-1, wr=-1),
    2: dict(name="ragged_batch_page544", S=8, ctx=(0, 4096), new=(1, 1024), H=64, Hkv=64,
            d=128, P=544, causal=True, wl=-1, wr=-1),
    3: dict(name="gqa_d256_page1040", S=8, ctx=(0, 8192), new=(256, 2048), H=8, Hkv=2,
            d=256, P=1040, causal=True, wl=-1, wr=-1),
    4: dict(name="sliding_window_16k", S=1, ctx=(0, 0), new=(16384, 16384), H=8, Hkv=8,
            d=64, P=16, causal=False, wl=64, wr=64),
    5: dict(name="window_clamped_mm_prefix", S=1, ctx=(4096, 4096), new=(12454, 12454),
            H=16, Hkv=8, d=256, P=16, causal=True, wl=1023, wr=-1, mm=(60, 256, 1190)),
}


def make_config(cid: int, *, page_size: Optional[int] = None, new_tokens: Optional[int] = None,
                new_in_cache: bool = False, heads: Optional[tuple] = None,
                seed: Optional[int] = None) -> Workload:
    """Build benchmark workload ``cid`` (1..5) with seed ``1000 + cid``.

    ``page_size`` overrides P (config 3 is also run at 1056), ``new_tokens``
    overrides the new-token count of the single-sequence configs (the linear
    scaling sweep of config 4), ``heads=(H, Hkv)`` shrinks the head count.
    """
    spec = CONFIGS[cid]
    if seed is None:
        seed = 1000 + cid
    rng = np.random.default_rng(seed)
    S = spec["S"]
    ctx = rng.integers(spec["ctx"][0], spec["ctx"][1] + 1, size=S).astype(np.int32)
    new = rng.integers(spec["new"][0], spec["new"][1] + 1, size=S).astype(np.int32)
    if new_tokens is not None:
        new = np.full(S, new_tokens, dtype=np.int32)
    mm = None
    if "mm" in spec:
        count, width, slack = spec["mm"]
        offs = np.sort(rng.integers(0, slack + 1, size=count))
        st = offs + width * np.arange(count)
        mm = np.stack([st, st + width - 1], axis=-1).astype(np.int32)[None]
    H, Hkv = spec["H"], spec["Hkv"]
    if heads is not None:
        H, Hkv = heads
    P = page_size if page_size is not None else spec["P"]
    override = None
    if cid == 1 and not new_in_cache:
        # The tiny config's block table is a seeded permutation of all 8 pages.
        override = np.random.default_rng(seed + 1).permutation(8).astype(np.int32)[None]
    name = spec["name"] if page_size is None else f"{spec['name']}_P{P}"
    if cid == 3 and page_size is not None:
        name = f"gqa_d256_page{P}"
    return make_workload(seed=seed, table_seed=seed + 1, ctx_lens=ctx, q_lens=new,
                         num_heads=H, num_kv_heads=Hkv, head_size=spec["d"], page_size=P,
                         causal=spec["causal"], window_left=spec["wl"], window_right=spec["wr"],
                         mm_ranges=mm, new_in_cache=new_in_cache,
                         block_table_override=override, name=name, rng=rng)


# Workloads of the extended rows (mask variants and split-KV), seeded like the
# benchmark configurations.  Shapes: a short chunk after a long cached context
# (few Q tiles, the split-KV case); a long sequence under chunked local
# attention with one chunk of lookback; the multimodal workload with its
# ranges unclamped; the ragged batch with a causal flag per sequence.
def make_named(name: str) -> Workload:
    if name == "long_context_short_chunk":
        return make_workload(seed=2001, ctx_lens=[32768, 30000], q_lens=[256, 200],
                             num_heads=32, num_kv_heads=8, head_size=128, page_size=16,
                             causal=True, name=name)
    if name == "chunked_local_16k":
        return make_workload(seed=2002, ctx_lens=[0], q_lens=[16384], num_heads=16,
                             num_kv_heads=4, head_size=128, page_size=16, causal=True,
                             chunk_size=4096, chunk_lookback=1, name=name)
    if name == "window_mm_prefix_unclamped":
        w = make_config(5)
        w.name = name
        w.mm_clamp = False
        return w
    if name == "ragged_batch_per_seq_causal":
        w = make_config(2)
        w.name = name
        w.causal_per_seq = np.array([1, 0, 1, 1, 0, 1, 0, 1], dtype=np.int32)
        return w
    if name == "ragged_batch_page544_d64":
        c2 = make_config(2)
        return make_workload(seed=2003, ctx_lens=c2.ctx_lens, q_lens=c2.q_lens, num_heads=64,
                             num_kv_heads=64, head_size=64, page_size=544, causal=True,
                             name=name)
    if name == "sliding_window_16k_full":
        # config 4 without its window: every key for every query, the work the
        # window's tile bounds save (measured once for contrast)
        w = make_config(4)
        w.name = name
        w.window_left = -1
        w.window_right = -1
        return w
    if name == "dense_noncausal_d128":
        return make_workload(seed=2004, ctx_lens=[0, 0], q_lens=[8192, 8192], num_heads=32,
                             num_kv_heads=8, head_size=128, page_size=64, causal=False,
                             name=name)
    raise KeyError(name)


# Workloads a tile-shape sweep times: the benchmark shapes of each head size,
# the ragged batch at head size 64, and a dense non-causal batch (no masking,
# no ragged tails) that isolates the tile loop.
# The page-size rows (1056 and the power of two 512 or 1024 beside 544 and 1040)
# show whether the best shape depends on the page size as well as the head size.
TILE_SWEEP = ["ragged_batch_page544", "gqa_d256_page1040", "sliding_window_16k",
              "window_clamped_mm_prefix", "ragged_batch_page544_d64", "dense_noncausal_d128",
              "ragged_batch_page1056", "ragged_batch_page512", "gqa_d256_page1056",
              "gqa_d256_page1024"]


def make_sweep(name: str) -> Workload:
    configs = {"ragged_batch_page544": (2, None), "gqa_d256_page1040": (3, 1040),
               "sliding_window_16k": (4, None), "window_clamped_mm_prefix": (5, None),
               "ragged_batch_page1056": (2, 1056), "ragged_batch_page512": (2, 512),
               "gqa_d256_page1056": (3, 1056), "gqa_d256_page1024": (3, 1024)}
    if name in configs:
        cid, P = configs[name]
        return make_config(cid, page_size=P)
    return make_named(name)


NAMED = ["long_context_short_chunk", "chunked_local_16k", "window_mm_prefix_unclamped",
         "ragged_batch_per_seq_causal"]
