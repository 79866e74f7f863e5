"""CPU oracle for paged-KV prefill attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never calls it and never falls back to it.

It is a plain, slow, obviously correct implementation of what the method
computes, written from the pages' definitions:

* ``attention.reference_prefill`` — the dense definition: gather K/V from the
  paged cache through the block table (plus the chunk's new K/V), build the
  explicit boolean mask, softmax over allowed keys, weighted sum of V.
  Sources: vLLM PR #54194 report ("Implementation breakdown", item 4: the fp32
  reference built by gathering K/V from the paged cache); vLLM PR #53147
  report ("Implementation breakdown", items 2 and 4: the window-clamped
  multimodal-prefix mask ORed onto the base mask, and its dense reference).
* ``bounds.tile_bounds_ref`` — the per-Q-tile KV-tile loop range: window
  union intersecting multimodal ranges, clamped.  Sources: vLLM PR #50776
  report ("Key source snippets", _fwd_kernel loop limits) and vLLM PR #53147
  report ("Key source snippets", compute_tile_loop_bounds).
* ``bounds.useful_pairs`` — the number of allowed (query, key) pairs, which
  prices useful work at 4 * head_size FLOP per pair per query head.
* mask variants (chunked local attention, a causal flag per sequence,
  unclamped multimodal ranges) and ``attention.merge_partials``, the
  log-sum-exp merge of split-KV segments.  Source: vLLM PR #53147 report
  ("Key source snippets", compute_tile_loop_bounds; "Review highlights").

Precision: fp32, as the pages' reference is fp32.  The oracle never rounds
intermediates to bf16.  It shares no code with the HIP path and imports only
numpy.

Every function is pinned by ``tests/test_oracle_*.py`` against things other
than itself: a pure-Python brute force with a differently structured mask,
torch's CPU scaled_dot_product_attention on the special cases it covers,
closed forms, invariants, and the integer tile bounds printed on the vLLM
PR #53147 report.
"""

from .attention import (  # noqa: F401
    allowed_mask,
    gather_kv,
    merge_partials,
    reference_prefill,
    reference_rows,
)
from .bounds import (  # noqa: F401
    row_intervals,
    tile_bounds_all,
    tile_bounds_ref,
    useful_flops,
    useful_pairs,
)
