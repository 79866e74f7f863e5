"""Host-side checks of bench.py: its useful-work counter agrees with the
oracle's, and it refuses more than one GPU."""

import subprocess
import sys
import os

import numpy as np

import bench
import oracle
from workloads import NAMED, TILE_SWEEP, make_config, make_named, make_sweep, make_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_useful_pairs_counter_matches_oracle():
    ws = [make_config(1), make_config(4, new_tokens=4096),
          make_config(5, heads=(2, 1), new_tokens=12454)]
    rng = np.random.default_rng(12)
    for i in range(30):
        S = int(rng.integers(1, 4))
        mm = None
        if i % 2:
            mm = rng.integers(0, 300, size=(S, 3, 2)).astype(np.int32)
            mm[..., 1] += rng.integers(0, 80, size=(S, 3))
        ws.append(make_workload(seed=i, ctx_lens=rng.integers(0, 200, S),
                                q_lens=rng.integers(1, 150, S), num_heads=2, num_kv_heads=1,
                                head_size=8, page_size=16, causal=bool(i % 3),
                                window_left=int(rng.choice([-1, 0, 9, 70])),
                                window_right=int(rng.choice([-1, 0, 5, 90])), mm_ranges=mm,
                                causal_per_seq=rng.integers(0, 2, S) if i % 4 == 1 else None,
                                mm_clamp=bool(i % 5), chunk_size=int(rng.choice([0, 16, 50])),
                                chunk_lookback=int(rng.choice([-1, 0, 2]))))
    ws += [make_named(n) for n in NAMED]
    ws += [make_sweep(n) for n in TILE_SWEEP]
    for w in ws:
        assert bench.count_useful_pairs(w) == oracle.useful_pairs(
            w.ctx_lens, w.q_lens, w.causal_arg, w.window_left, w.window_right, w.mm_ranges,
            **w.mask_kwargs()), w.name


def test_bench_refuses_multi_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_variant_build_command_line(tmp_path):
    """The build step takes preprocessor defines and an output path (tile-shape
    variants for sweeps) and leaves the in-tree library alone; a static check of
    the kernel rejects a shape whose copies do not split over its wavefronts."""
    from paged_kv_prefill_attention_amd import _build
    lib = _build.library_path()
    before = os.path.getmtime(lib) if os.path.exists(lib) else None
    out = str(tmp_path / "lib_variant.so")
    r = subprocess.run([sys.executable, "-m", "paged_kv_prefill_attention_amd._build",
                        "--define", "PREFILL_TILE_D64=8,32,4,2,1", "--out", out],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode != 0 and "copies must split evenly" in (r.stdout + r.stderr)
    assert not os.path.exists(out)
    after = os.path.getmtime(lib) if os.path.exists(lib) else None
    assert before == after
