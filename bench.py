"""Benchmark: paged-KV prefill attention on one MI355X.

One step = one launch of the whole hot path (work decode, tile bounds, page
resolution, K/V gather, QK^T, mask, online softmax, PV, epilogue) over the
ragged batch "ragged_batch_page544": 8 sequences with U[0,4096] cached tokens
in 544-token pages (randomly permuted block tables) and U[1,1024] new tokens,
64 query / 64 KV heads, head size 128, causal, bf16 inputs ~ N(0,1).

Prints ONE JSON line.  ``value`` is useful TFLOP/s: 4 * head_size FLOP per
allowed (query, key) pair per query head, divided by the mean time per step
(one launch per step, each bracketed by HIP events on the launch stream,
inputs resident in HBM).  ``pct_bf16_peak`` and ``roofline`` use that same
mean; the median, extremes and the first-to-last event span per step are
reported beside it.  ``cpu_baseline`` times the CPU oracle on a bounded sample
of the same workload, ``cpu_baseline_pruned`` the same oracle restricted to each
Q tile's KV-tile bounds.

Before the warm-up steps the GPU runs the same launch back to back for
``--prewarm-ms`` (default 200 ms, untimed, reported as ``prewarm_ms``): coming
out of idle, or after light work, its clock ramps up over the first tens of
milliseconds of load, and launches in that window run up to 40% slower than at
steady state, which a handful of warm-up steps does not cover.  The suite and
the tile sweep do the same before every workload.

``--suite FILE`` additionally times every configuration and the sliding-window
length sweep and writes them to FILE (one JSON object per line).

``--tile-sweep FILE`` instead times only the tile-shape sweep workloads (one
JSON object per workload, eager launches) with the library given by ``--lib``,
e.g. a build with another tile shape:

    python -m paged_kv_prefill_attention_amd._build \
        --define PREFILL_TILE_D128=4,32,4,2,1 --out /tmp/lib_d128_4_32.so
    python bench.py --lib /tmp/lib_d128_4_32.so --tile-sweep /tmp/d128_4_32.jsonl
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "prefill attention useful TFLOP/s + ms/batch; % of MI355X bf16 MFMA peak"
KERNEL_SRC = os.path.join(ROOT, "paged_kv_prefill_attention_amd", "csrc",
                          "prefill_attention.hip")


def kernel_source_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def algorithmic_bytes(w) -> int:
    """Q read + O write once per query row and head; K and V read once per key
    position and KV head (cached + new)."""
    d = w.head_size
    qo = 2 * 2 * d * w.num_heads * w.total_q_tokens
    kv = 2 * 2 * d * w.num_kv_heads * int(w.seq_lens().sum())
    return qo + kv


def traffic_from_profiles(workload: str):
    """HBM bytes per launch measured by rocprofv3 counters, if the committed
    summary was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_prefill_attention_%s.md" % workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_val.group(1))


def prewarm(fn, ms: float):
    """Launch ``fn`` back to back, untimed, for about ``ms`` milliseconds of
    wall time, so that the timed steps run at the GPU's loaded clock."""
    import torch
    t_end = time.perf_counter() + ms / 1e3
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def time_launches(fn, steps: int, warmup: int):
    """Run ``fn`` warmup times, then time ``steps`` launches with events on the
    current stream.  Returns (mean ms per launch, per-launch ms list, wall s)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    span = starts[0].elapsed_time(ends[-1])
    return span / steps, per, wall


def time_graph(fn, steps: int, warmup: int, reps: int = 10):
    """Device time per launch: ``reps`` launches captured in one HIP graph, the
    graph replayed ``steps`` times between events (no host gaps between
    launches, which dominate small workloads when launched eagerly)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for _ in range(reps):
                fn()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / (steps * reps)
    del g
    return ms


def to_device(w, cache_only=False):
    """Upload a seeded workload (bf16 bit patterns, int32 metadata) to cuda:0."""
    import numpy as np
    import torch

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(
            torch.bfloat16)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()

    return dict(q=bf(w.q), k_new=None if cache_only else bf(w.k_new),
                v_new=None if cache_only else bf(w.v_new), k_cache=bf(w.k_cache),
                v_cache=bf(w.v_cache), block_table=i32(w.block_table),
                query_start_loc=i32(w.query_start_loc), ctx_lens=i32(w.ctx_lens),
                mm_ranges=None if w.mm_ranges is None else i32(w.mm_ranges),
                causal_per_seq=None if w.causal_per_seq is None else i32(w.causal_per_seq))


def make_launcher(w, cache_only=False, kv_splits=1):
    """A closure launching the library on the resident workload.  Split-KV gets its
    workspace once, outside the timed launches."""
    import torch
    import paged_kv_prefill_attention_amd as ppa
    dev = to_device(w, cache_only=cache_only)
    out = torch.empty_like(dev["q"])
    k = ppa.split_count(w.head_size, w.num_heads, w.num_kv_heads, w.num_seqs,
                        w.total_q_tokens, w.max_q_len, kv_splits,
                        window_left=w.window_left, window_right=w.window_right, causal=w.causal)
    need = ppa.workspace_size(w.num_heads, w.head_size, w.total_q_tokens, k)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
    dev["workspace"] = ws
    extra = dict(causal_per_seq=dev["causal_per_seq"], mm_clamp=w.mm_clamp,
                 chunk_size=w.chunk_size, chunk_lookback=w.chunk_lookback,
                 kv_splits=kv_splits, workspace=ws)

    def fn():
        ppa.prefill_attention(dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"],
                              dev["v_cache"], dev["block_table"], dev["query_start_loc"],
                              dev["ctx_lens"], w.num_heads, w.num_kv_heads, w.head_size,
                              w.page_size, w.window_left, w.window_right, w.causal,
                              dev["mm_ranges"], w.scale, out=out, max_q_len=w.max_q_len,
                              **extra)
    return fn, dev, out


def count_useful_pairs(w) -> int:
    """Allowed (query row, key) pairs for one query head.  Each query's allowed
    keys form one interval holding its own position: the base window
    [left edge, a | a + window_right | L-1] (left edge: a - window_left, or the
    chunk start with lookback under chunked local attention), widened by every
    valid multimodal range [st, en] (st < en) that holds the query, whose left
    edge is clamped to the window unless the clamp is off; then clamped to
    [0, L-1].  The causal flag may be per sequence."""
    import numpy as np
    total = 0
    chunked = w.chunk_size > 0 and w.chunk_lookback >= 0
    for s in range(w.num_seqs):
        c, n = int(w.ctx_lens[s]), int(w.q_lens[s])
        L = c + n
        a = c + np.arange(n, dtype=np.int64)
        causal = w.causal if w.causal_per_seq is None else bool(w.causal_per_seq[s])
        if chunked:
            lo = (a // w.chunk_size - w.chunk_lookback) * w.chunk_size
        else:
            lo = a - w.window_left if w.window_left >= 0 else np.zeros_like(a)
        if causal:
            hi = a.copy()
        elif w.window_right >= 0:
            hi = a + w.window_right
        else:
            hi = np.full_like(a, L - 1)
        for st, en in w.mm_list(s):
            if st < en:
                hold = (a >= st) & (a <= en)
                clamp = w.mm_clamp and w.window_left >= 0
                left = np.maximum(st, a - w.window_left) if clamp else st
                lo = np.where(hold, np.minimum(lo, left), lo)
                hi = np.where(hold, np.maximum(hi, en), hi)
        lo, hi = np.maximum(lo, 0), np.minimum(hi, L - 1)
        total += int(np.maximum(hi - lo + 1, 0).sum())
    return total


def useful_flop(w) -> int:
    """4 * head_size FLOP (QK^T and PV) per allowed pair per query head."""
    return 4 * w.head_size * w.num_heads * count_useful_pairs(w)


def cpu_baseline(w, heads: int, min_seconds: float = 10.0, max_passes: int = 8):
    """Time the CPU oracle (as it stands) on heads [0, heads) of every sequence,
    repeating whole passes until at least ``min_seconds`` have elapsed."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = 1
    args = (w.f32("q"), w.f32("k_new"), w.f32("v_new"), w.f32("k_cache"), w.f32("v_cache"),
            w.block_table, w.query_start_loc, w.ctx_lens, w.num_heads, w.num_kv_heads,
            w.head_size, w.page_size, w.window_left, w.window_right, w.causal, w.mm_ranges,
            w.scale)
    t0 = time.perf_counter()
    passes = 0
    while passes < max_passes:
        for s in range(w.num_seqs):
            n = int(w.q_lens[s])
            if n:
                oracle.reference_rows(*args, s, np.arange(n), heads=range(heads))
        passes += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    el = time.perf_counter() - t0
    flop = useful_flop(w) * heads // w.num_heads * passes
    return {"value": flop / el / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": "fp32 numpy oracle, query heads 0..%d of all %d sequences (all rows), "
                      "%d pass(es), %.1f s, %.3g useful FLOP; host %s, os.cpu_count()=%s, "
                      "affinity=%d, BLAS threads %d" % (
                          heads - 1, w.num_seqs, passes, el, flop,
                          platform.processor() or "cpu", os.cpu_count(),
                          len(os.sched_getaffinity(0)), threads)}


def cpu_baseline_pruned(w, heads: int, block_q: int, block_n: int, min_seconds: float = 5.0,
                        max_passes: int = 8):
    """The same oracle restricted, per Q tile of the kernel's geometry, to the keys
    of that tile's bounds (``key_range`` from ``oracle.tile_bounds_ref``): the
    CPU counterpart of the kernel's tile pruning, timed like ``cpu_baseline``."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = 1
    args = (w.f32("q"), w.f32("k_new"), w.f32("v_new"), w.f32("k_cache"), w.f32("v_cache"),
            w.block_table, w.query_start_loc, w.ctx_lens, w.num_heads, w.num_kv_heads,
            w.head_size, w.page_size, w.window_left, w.window_right, w.causal, w.mm_ranges,
            w.scale)
    t0 = time.perf_counter()
    passes = 0
    while passes < max_passes:
        for s in range(w.num_seqs):
            n, c = int(w.q_lens[s]), int(w.ctx_lens[s])
            for t in range(-(-n // block_q)):
                lo, hi = oracle.tile_bounds_ref(c, n, t, block_q, block_n, w.causal,
                                                w.window_left, w.window_right, w.mm_list(s))
                rows = np.arange(t * block_q, min(n, (t + 1) * block_q))
                oracle.reference_rows(*args, s, rows, heads=range(heads),
                                      key_range=(lo * block_n, min(hi * block_n, c + n)))
        passes += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    el = time.perf_counter() - t0
    flop = useful_flop(w) * heads // w.num_heads * passes
    return {"value": flop / el / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle, keys pruned to the tile bounds",
            "sample": "fp32 numpy oracle per Q tile of %d tokens over its %d-key tile range, "
                      "query heads 0..%d of all %d sequences, %d pass(es), %.1f s" % (
                          block_q, block_n, heads - 1, w.num_seqs, passes, el)}


def run_suite(path, steps, warmup, prewarm_ms=0.0):
    """Every configuration plus the sliding-window length sweep."""
    import torch
    from workloads import NAMED, make_config, make_named
    rows = []
    cases = [(1, None, None), (2, None, None), (3, 1040, None), (3, 1056, None),
             (4, None, None), (5, None, None)]
    cases += [(4, None, n) for n in (2048, 4096, 8192, 16384, 32768, 65536)]
    cases = [(cid, P, n, 1) for cid, P, n in cases]
    # split-KV: explicit and automatic counts, beside the unsplit launch
    cases += [(3, 1040, None, 2), (3, 1040, None, 4), (3, 1040, None, 0), (5, None, None, 0)]
    cases += [(name, None, None, k) for name in NAMED for k in
              ((1, 0) if name == "long_context_short_chunk" else (1,))]
    # the window's pruning, for contrast: config 4 attending to every key
    cases += [("sliding_window_16k_full", None, None, 1)]
    for cid, P, n, splits in cases:
        w = make_named(cid) if isinstance(cid, str) else make_config(cid, page_size=P,
                                                                      new_tokens=n)
        fn, dev, out = make_launcher(w, kv_splits=splits)
        prewarm(fn, prewarm_ms)
        ms, per, _ = time_launches(fn, steps, warmup)
        per.sort()
        ms_dev = time_graph(fn, max(3, steps // 5), 2)
        flop = useful_flop(w)
        import paged_kv_prefill_attention_amd as ppa
        k = ppa.split_count(w.head_size, w.num_heads, w.num_kv_heads, w.num_seqs,
                            w.total_q_tokens, w.max_q_len, splits,
                            window_left=w.window_left, window_right=w.window_right, causal=w.causal)
        rec = {"config": cid, "workload": w.name, "new_tokens": int(w.q_lens.sum()),
               "kv_splits": k, "requested_splits": splits, "ms_mean": ms,
               "ms_median": per[len(per) // 2],
               "ms_device": ms_dev, "device_tflops": flop / (ms_dev / 1e3) / 1e12,
               "useful_tflops": flop / (ms / 1e3) / 1e12,
               "frac_mfma_peak": flop / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
               "alg_gbs": algorithmic_bytes(w) / (ms / 1e3) / 1e9, "useful_flop": flop}
        rows.append(rec)
        print(json.dumps(rec), file=sys.stderr, flush=True)
        del dev, out, fn
        torch.cuda.empty_cache()
    with open(path, "w") as f:
        for r in rows:
            f.write(json.dumps(r) + "\n")


def run_tile_sweep(path, steps, warmup, prewarm_ms=0.0):
    """Eager timing of the tile-sweep workloads, in the order of TILE_SWEEP
    (under a counter profiler each workload is warmup + steps dispatches)."""
    import torch
    from workloads import TILE_SWEEP, make_sweep
    import paged_kv_prefill_attention_amd as ppa
    rows = []
    for name in TILE_SWEEP:
        w = make_sweep(name)
        fn, dev, out = make_launcher(w)
        prewarm(fn, prewarm_ms)
        ms, per, _ = time_launches(fn, steps, warmup)
        per.sort()
        bq, bn = ppa.tile_config(w.head_size, w.num_heads, w.num_kv_heads, w.num_seqs, w.max_q_len,
                                 window_left=w.window_left, window_right=w.window_right,
                                 causal=w.causal)
        flop = useful_flop(w)
        rec = {"workload": name, "head_size": w.head_size, "block_q": bq, "block_n": bn,
               "ms_median": per[len(per) // 2], "ms_mean": ms,
               "useful_tflops": flop / (per[len(per) // 2] / 1e3) / 1e12}
        rows.append(rec)
        print(json.dumps(rec), flush=True)
        del dev, out, fn
        torch.cuda.empty_cache()
    with open(path, "w") as f:
        for r in rows:
            f.write(json.dumps(r) + "\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prewarm-ms", type=float, default=200.0,
                    help="untimed back-to-back launches before the warm-up steps (ms)")
    ap.add_argument("--cpu-heads", type=int, default=64,
                    help="query heads in the bounded CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--suite", default=None, help="also time every config; write JSON lines")
    ap.add_argument("--lib", default=None,
                    help="load this build of the library instead of the in-tree one")
    ap.add_argument("--tile-sweep", default=None,
                    help="only time the tile-sweep workloads; write JSON lines")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead: time a plain device copy of this many bytes (the "
                         "reference kernel for scaling the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_prefill_attention_amd as ppa
    from workloads import make_config

    if args.lib:
        ppa.use_library(args.lib)
    else:
        if not os.path.exists(ppa.library_path()):
            ppa.build()
        ppa.load_library()
    torch.cuda.set_device(0)

    if args.tile_sweep:
        run_tile_sweep(args.tile_sweep, args.steps, args.warmup, args.prewarm_ms)
        return

    if args.copy_bytes:
        src = torch.ones(args.copy_bytes // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        ms, _, _ = time_launches(lambda: dst.copy_(src), args.steps, args.warmup)
        print(json.dumps({"copy_bytes": args.copy_bytes, "ms": ms,
                          "gbs_read_plus_write": 2 * args.copy_bytes / (ms / 1e3) / 1e9}))
        return

    w = make_config(2)
    fn, dev, out = make_launcher(w)
    flop = useful_flop(w)
    torch.cuda.synchronize()
    prewarm(fn, args.prewarm_ms)
    span_ms, per, wall = time_launches(fn, args.steps, args.warmup)
    # One timing for every figure: a step is one launch, timed by HIP events on
    # the launch stream; value, pct_bf16_peak and the roofline all use their mean.
    ms = sum(per) / len(per)
    per_sorted = sorted(per)
    value = flop / (ms / 1e3) / 1e12
    achieved = value
    traffic = traffic_from_profiles(w.name)
    bq, bn = ppa.tile_config(w.head_size, w.num_heads, w.num_kv_heads, w.num_seqs, w.max_q_len,
                             window_left=w.window_left, window_right=w.window_right,
                             causal=w.causal)
    rec = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "prewarm_ms": args.prewarm_ms,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "num_heads": w.num_heads,
                   "num_kv_heads": w.num_kv_heads, "head_size": w.head_size,
                   "page_size": w.page_size, "causal": w.causal,
                   "ctx_lens": w.ctx_lens.tolist(), "q_lens": w.q_lens.tolist(),
                   "total_q_tokens": w.total_q_tokens, "useful_flop": flop,
                   "block_q": bq, "block_n": bn, "seed": w.seed},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "alg_hbm_gbs": round(algorithmic_bytes(w) / (ms / 1e3) / 1e9, 1),
        "ms_launch_mean": round(ms, 5),
        "ms_launch_median": round(per_sorted[len(per) // 2], 5),
        "ms_launch_min_max": [round(per_sorted[0], 5), round(per_sorted[-1], 5)],
        "ms_span_per_step": round(span_ms, 5),
        "wall_s_timed": round(wall, 4),
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    del dev, out, fn
    torch.cuda.empty_cache()
    if args.suite:
        run_suite(args.suite, args.steps, args.warmup, args.prewarm_ms)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, min(args.cpu_heads, w.num_heads))
        rec["cpu_baseline_pruned"] = cpu_baseline_pruned(w, min(args.cpu_heads, w.num_heads),
                                                         bq, bn)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
