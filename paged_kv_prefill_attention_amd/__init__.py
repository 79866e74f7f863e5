"""Paged-KV prefill attention for MI355X (gfx950): Python binding of the C ABI.

The computation lives in ``libpagedprefill.so`` (hand-written HIP, built
in-tree by ``_build.build()``); this package only marshals torch tensors into
device pointers and streams.
"""

from ._binding import (  # noqa: F401
    BAD_CTX,
    BAD_LENGTH,
    BAD_PAGE_ID,
    BAD_PAGES,
    BAD_QLEN,
    BAD_QSL,
    ERR_HIP,
    ERR_SCRATCH,
    ERR_INVALID_ARG,
    ERR_UNSUPPORTED,
    OK,
    PrefillError,
    check_metadata,
    load_library,
    prefill_attention,
    prefill_attention_ex_noalloc,
    split_count,
    strerror,
    tile_bounds,
    tile_config,
    use_library,
    validate,
    workspace_size,
)
from ._build import build, library_path  # noqa: F401
