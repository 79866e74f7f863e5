"""GPU tests: the library's launches captured in a HIP graph (as the benchmark's
device-time measurement does) give the same bits as eager launches, on every
replay.  The library allocates nothing and records no memset, so a capture
holds only its kernels; each replay is checked after eager work on the same
stream has overwritten the output."""

import numpy as np
import pytest

from tests.harness import to_device, variant_kwargs
from workloads import make_config, make_named

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    import paged_kv_prefill_attention_amd as ppa
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    ppa.load_library()


def launcher(w, dev, out, kv_splits, workspace):
    import paged_kv_prefill_attention_amd as ppa

    def fn():
        ppa.prefill_attention(
            dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
            dev["block_table"], dev["query_start_loc"], dev["ctx_lens"], w.num_heads,
            w.num_kv_heads, w.head_size, w.page_size, w.window_left, w.window_right,
            w.causal, dev["mm_ranges"], w.scale, out=out, max_q_len=w.max_q_len,
            workspace=workspace, **variant_kwargs(w, dev, kv_splits))
    return fn


@pytest.mark.parametrize("case,kv_splits", [(2, 1), (5, 1), (5, 0), (3, 2), (3, 0),
                                            ("long_context_short_chunk", 0),
                                            ("window_mm_prefix_unclamped", 1),
                                            (4, 0), ("sliding_window_16k_full", 0)])
def test_graph_replays_match_eager_bitwise(case, kv_splits):
    import torch
    import paged_kv_prefill_attention_amd as ppa
    w = make_config(case, page_size=1040 if case == 3 else None) if isinstance(case, int) \
        else make_named(case)
    print(w.name, "kv_splits", kv_splits, flush=True)
    dev = to_device(w)
    k = ppa.split_count(w.head_size, w.num_heads, w.num_kv_heads, w.num_seqs,
                        w.total_q_tokens, w.max_q_len, kv_splits,
                        window_left=w.window_left, window_right=w.window_right, causal=w.causal)
    need = ppa.workspace_size(w.num_heads, w.head_size, w.total_q_tokens, k)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
    out = torch.empty_like(dev["q"])
    fn = launcher(w, dev, out, kv_splits, ws)
    fn()
    torch.cuda.synchronize()
    eager = out.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        fn()
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(out.view(torch.int16), eager.view(torch.int16))
        assert same, "replay %d differs from the eager launch" % rep
    assert torch.isfinite(out.float()).all()
    del g
