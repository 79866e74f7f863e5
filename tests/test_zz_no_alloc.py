"""The allocation-free entry point (prefill_attention_ex_noalloc) against the
workspace entry point (prefill_attention_ex) it varies: the split-KV partials
live in the library's static scratch instead of a caller workspace.  Two calls
in a row, the second with a smaller input, so the second reads a scratch that
still holds the first call's partials.  Outputs must equal the workspace entry
point's bit for bit and the oracle within 2e-2 + 2e-2 |ref|."""

import math

import numpy as np
import pytest

from tests.harness import compare, oracle_full, out_to_f32, run_gpu, to_device
from workloads import make_config, make_workload

pytestmark = pytest.mark.gpu

SCRATCH = 64 << 20


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    import paged_kv_prefill_attention_amd as ppa
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    ppa.load_library()


def run_noalloc(w, dev, kv_splits, out):
    import paged_kv_prefill_attention_amd as ppa
    return ppa.prefill_attention_ex_noalloc(
        dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
        dev["block_table"], dev["query_start_loc"], dev["ctx_lens"], w.num_heads,
        w.num_kv_heads, w.head_size, w.page_size, w.window_left, w.window_right, w.causal,
        dev["mm_ranges"], w.scale, out, max_q_len=w.max_q_len,
        causal_per_seq=dev["causal_per_seq"], mm_clamp=w.mm_clamp, chunk_size=w.chunk_size,
        chunk_lookback=w.chunk_lookback, kv_splits=kv_splits)


def test_noalloc_matches_workspace_entry_two_calls():
    import torch
    import paged_kv_prefill_attention_amd as ppa
    # 1: long cached contexts, 8 explicit segments: 8 x 456 x 32 x 128 x 4 B of partials
    #    (60 MB of the 64 MiB scratch); 2: a smaller GQA batch, 3 segments, d = 64
    big = make_workload(seed=8101, ctx_lens=[32768, 30000], q_lens=[256, 200], num_heads=32,
                        num_kv_heads=8, head_size=128, page_size=16, causal=True,
                        name="noalloc_big")
    small = make_workload(seed=8102, ctx_lens=[3000, 0, 700], q_lens=[90, 130, 5], num_heads=8,
                          num_kv_heads=2, head_size=64, page_size=544, causal=False,
                          window_left=500, window_right=40, qk_sigma=3.0, name="noalloc_small")
    for w, k in ((big, 8), (small, 3)):
        need = ppa.workspace_size(w.num_heads, w.head_size, w.total_q_tokens, k)
        assert 0 < need <= SCRATCH, need
        print("noalloc case", w.name, "splits", k, "partials", need, flush=True)
        dev = to_device(w)
        ref = run_gpu(w, dev=dev, kv_splits=k)             # caller workspace
        out = torch.full_like(dev["q"], float("nan"))
        got = run_noalloc(w, dev, k, out)                  # static scratch
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), w.name
        compare(out_to_f32(got), oracle_full(w), w.name + " noalloc")


def test_noalloc_automatic_splits_and_scratch_limit():
    import torch
    import paged_kv_prefill_attention_amd as ppa
    # automatic count on a batch whose automatic partials fit: same bits as the
    # workspace entry point with the automatic count
    w = make_workload(seed=8103, ctx_lens=[20000], q_lens=[300], num_heads=16, num_kv_heads=4,
                      head_size=128, page_size=1056, causal=True, name="noalloc_auto")
    k = ppa.split_count(w.head_size, w.num_heads, w.num_kv_heads, w.num_seqs, w.total_q_tokens,
                        w.max_q_len, 0,
                        window_left=w.window_left, window_right=w.window_right, causal=w.causal)
    assert k > 1 and ppa.workspace_size(w.num_heads, w.head_size, w.total_q_tokens, k) <= SCRATCH
    dev = to_device(w)
    ref = run_gpu(w, dev=dev, kv_splits=0)
    got = run_noalloc(w, dev, 0, torch.empty_like(dev["q"]))
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    # the multimodal workload's automatic count (tail splitting, 4 segments) needs more
    # than the scratch: the automatic mode falls back to no split, an explicit count fails
    w5 = make_config(5)
    k5 = ppa.split_count(w5.head_size, w5.num_heads, w5.num_kv_heads, w5.num_seqs,
                         w5.total_q_tokens, w5.max_q_len, 0,
                         window_left=w5.window_left, window_right=w5.window_right, causal=w5.causal)
    assert ppa.workspace_size(w5.num_heads, w5.head_size, w5.total_q_tokens, k5) > SCRATCH
    dev5 = to_device(w5)
    plain = run_gpu(w5, dev=dev5)
    got5 = run_noalloc(w5, dev5, 0, torch.empty_like(dev5["q"]))
    torch.cuda.synchronize()
    assert torch.equal(got5.view(torch.int16), plain.view(torch.int16))
    with pytest.raises(ppa.PrefillError) as e:
        run_noalloc(w5, dev5, 4, torch.empty_like(dev5["q"]))
    assert e.value.code == ppa.ERR_SCRATCH
