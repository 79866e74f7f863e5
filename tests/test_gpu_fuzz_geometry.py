"""GPU fuzz of the per-call geometry: random batches large enough for the 32-key d=64
tile shape, and long-context batches of few Q-tile items under the automatic split
count.  Every head of each sequence's Q-tile edge rows and of random rows against the
oracle (bar as in test_gpu_parity)."""

import numpy as np
import pytest

from tests.harness import compare, edge_rows, oracle_rows, out_to_f32, run_gpu, to_device
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    import paged_kv_prefill_attention_amd as ppa
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    ppa.load_library()


def check_rows(w, outs, bq, seed):
    rng = np.random.default_rng(seed)
    for s in range(w.num_seqs):
        rows = edge_rows(w, s, bq, rng)
        q0 = int(w.query_start_loc[s])
        ref = oracle_rows(w, s, rows)
        for what, out in outs.items():
            compare(out[q0 + rows], ref, "%s seq %d %s" % (w.name, s, what))


def many_items_case(i):
    """A d=64 batch with enough Q-tile items for the 32-key shape: at least one round
    of its slots (1024 on 256 CUs) under a window of at most 2048 keys per row, else
    four rounds; random heads, page sizes, masks, multimodal ranges and magnitudes."""
    rng = np.random.default_rng(777000 + i)
    H, Hkv = [(8, 8), (16, 8), (16, 16), (32, 8), (8, 1)][int(rng.integers(0, 5))]
    P = int(rng.choice([1, 16, 64, 544, 1056]))
    causal = bool(rng.integers(0, 2))
    windowed = rng.random() < 0.7
    wl = int(rng.integers(0, 1500)) if windowed else -1
    wr = -1 if causal else (int(rng.integers(0, 500)) if windowed else -1)
    S = int(rng.integers(1, 6))
    g = H // Hkv
    hpt = int(np.gcd(g, 128))
    bq = 128 // hpt
    short = windowed and (causal or wr >= 0)
    need = 1024 if short else 4096
    qmax = int(np.ceil(need / (S * Hkv * (g // hpt)))) * bq
    q = rng.integers(max(1, qmax // 2), qmax + 1, size=S)
    q[0] = qmax
    ctx = rng.integers(0, 3000, size=S)
    mm = None
    if rng.random() < 0.3:
        R = int(rng.integers(1, 4))
        mm = np.zeros((S, R, 2), dtype=np.int32)
        for s in range(S):
            L = int(ctx[s] + q[s])
            for r in range(R):
                st = int(rng.integers(0, L))
                mm[s, r] = (st, st + int(rng.choice([3, 40, 300])))
    return make_workload(seed=880000 + i, ctx_lens=ctx, q_lens=q, num_heads=H, num_kv_heads=Hkv,
                         head_size=64, page_size=P, causal=causal, window_left=wl,
                         window_right=wr, mm_ranges=mm, name="many%d" % i,
                         qk_sigma=float(rng.choice([1.0, 3.0])))


def few_items_case(i):
    """A long-context batch of few Q-tile items (cached 2k-40k tokens, 1-700 new), any
    head size, optionally windowed or with multimodal ranges: the automatic split count
    cuts its long items into up to 16 segments."""
    rng = np.random.default_rng(990000 + i)
    d = int(rng.choice([64, 128, 256]))
    H, Hkv = [(8, 8), (16, 8), (32, 8), (8, 2), (64, 64), (16, 1)][int(rng.integers(0, 6))]
    S = int(rng.integers(1, 5))
    ctx = rng.integers(2000, 40000, size=S)
    q = rng.integers(1, 700, size=S)
    causal = bool(rng.integers(0, 2))
    wl = int(rng.choice([-1, -1, -1, 3000, 9000]))
    wr = -1 if causal else int(rng.choice([-1, 100]))
    mm = None
    if rng.random() < 0.3:
        mm = np.zeros((S, 2, 2), dtype=np.int32)
        for s in range(S):
            L = int(ctx[s] + q[s])
            for r in range(2):
                st = int(rng.integers(0, L))
                mm[s, r] = (st, st + int(rng.choice([40, 600])))
    P = int(rng.choice([16, 544, 1040]))
    return make_workload(seed=991000 + i, ctx_lens=ctx, q_lens=q, num_heads=H, num_kv_heads=Hkv,
                         head_size=d, page_size=P, causal=causal, window_left=wl,
                         window_right=wr, mm_ranges=mm, name="split%d" % i)


def geometry(w):
    import paged_kv_prefill_attention_amd as ppa
    return ppa.tile_config(w.head_size, w.num_heads, w.num_kv_heads, w.num_seqs, w.max_q_len,
                           window_left=w.window_left, window_right=w.window_right,
                           causal=w.causal)


@pytest.mark.parametrize("chunk", range(4))
def test_fuzz_32key_d64_shape(chunk):
    """Three random batches per chunk on the 32-key d=64 shape, plain and under the
    automatic split count."""
    for i in range(chunk * 3, chunk * 3 + 3):
        w = many_items_case(i)
        bq, bn = geometry(w)
        print(w.name, "S", w.num_seqs, "heads", w.num_heads, w.num_kv_heads, "page", w.page_size,
              "causal", w.causal, "window", w.window_left, w.window_right, "block_n", bn,
              flush=True)
        assert bn == 32
        dev = to_device(w)
        outs = {"plain": out_to_f32(run_gpu(w, dev=dev)),
                "automatic split": out_to_f32(run_gpu(w, dev=dev, kv_splits=0))}
        check_rows(w, outs, bq, seed=i)


@pytest.mark.parametrize("chunk", range(4))
def test_fuzz_automatic_split_few_items(chunk):
    """Three random long-context batches of few items per chunk under the automatic
    split count (which picks 2-16 segments for them, or none under a short window)."""
    import paged_kv_prefill_attention_amd as ppa
    for i in range(chunk * 3, chunk * 3 + 3):
        w = few_items_case(i)
        bq, _ = geometry(w)
        k = ppa.split_count(w.head_size, w.num_heads, w.num_kv_heads, w.num_seqs,
                            w.total_q_tokens, w.max_q_len, 0, window_left=w.window_left,
                            window_right=w.window_right, causal=w.causal)
        print(w.name, "d", w.head_size, "S", w.num_seqs, "heads", w.num_heads, w.num_kv_heads,
              "window", w.window_left, w.window_right, "automatic splits", k, flush=True)
        dev = to_device(w)
        check_rows(w, {"automatic split": out_to_f32(run_gpu(w, dev=dev, kv_splits=0))}, bq,
                   seed=i)
