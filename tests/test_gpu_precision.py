"""GPU parity at realistic logit magnitudes and non-default scales.

With Q and K drawn N(0, sigma^2) the scores s * scale reach tens to hundreds,
where any rounding applied to the scaled scores before exp2 shows in the
output.  The kernel keeps Q as the exact bf16 input and applies
scale * log2(e) in fp32 (one FMA per score before exp2), so the bar stays
|gpu - oracle| <= 2e-2 + 2e-2 * |oracle| elementwise (vLLM PR #53147 report,
"Implementation breakdown" item 4), on whole outputs.  The retiled kernel of
the vLLM PR #54194 report ("Risks and impact" item 1) is held to the stock
kernel's error against the fp32 reference; the max-abs errors printed here
are that figure for this kernel.
"""

import math

import pytest

from tests.harness import compare, oracle_full, out_to_f32, run_gpu
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    import paged_kv_prefill_attention_amd as ppa
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    ppa.load_library()


def magnitude_workload(d, sigma, scale_mult, seed, cache_only=False):
    """Two sequences with long cached contexts (2048 and 900 keys) in 544-token
    pages, GQA 4/2 heads, causal."""
    return make_workload(seed=seed, ctx_lens=[1748, 700], q_lens=[300, 200], num_heads=4,
                         num_kv_heads=2, head_size=d, page_size=544, causal=True,
                         scale=scale_mult / math.sqrt(d), qk_sigma=sigma,
                         new_in_cache=cache_only,
                         name="mag_d%d_s%g_x%g" % (d, sigma, scale_mult))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("sigma", [2.0, 3.0, 4.0])
def test_input_magnitude_and_scale(d, sigma):
    """sigma in {2, 3, 4} x scale in {0.5, 1, 2}/sqrt(d) and 1.0, whole outputs."""
    worst = 0.0
    for k, mult in enumerate([0.5, 1.0, 2.0, math.sqrt(d)]):
        w = magnitude_workload(d, sigma, mult, seed=7000 + 100 * d + 10 * int(sigma) + k)
        got = out_to_f32(run_gpu(w))
        err = compare(got, oracle_full(w), w.name)
        worst = max(worst, err[0])
        print("%s scale=%.4g max_abs=%.3g max_rel=%.3g" % (w.name, w.scale, err[0], err[1]),
              flush=True)
    print("d=%d sigma=%g worst max_abs=%.3g" % (d, sigma, worst), flush=True)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_magnitude_split_kv_and_cache_sourced(d):
    """sigma = 4 at scale 1/sqrt(d) through the split-KV merge (3 segments) and
    the cache-sourced mode."""
    w = magnitude_workload(d, 4.0, 1.0, seed=7500 + d)
    ref = oracle_full(w)
    compare(out_to_f32(run_gpu(w, kv_splits=3)), ref, w.name + " splits=3")
    wc = magnitude_workload(d, 4.0, 1.0, seed=7500 + d, cache_only=True)
    compare(out_to_f32(run_gpu(wc, cache_only=True)), oracle_full(wc, cache_only=True),
            w.name + " cache-only")
