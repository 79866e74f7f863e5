"""Thin ctypes binding over the C ABI in ``include/paged_prefill.h``.

Argument marshalling only: torch tensors are checked for device, dtype, shape
and contiguity, and passed as raw device pointers with torch's current HIP
stream.  Every step of the computation runs in the HIP library; if the
library is missing the calls raise, there is no other path.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

from ._build import library_path

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_HIP = -3
ERR_SCRATCH = -4

# bits of prefill_attention_check_metadata's result
BAD_QSL = 1
BAD_QLEN = 2
BAD_CTX = 4
BAD_LENGTH = 8
BAD_PAGES = 16
BAD_PAGE_ID = 32

_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_U64 = ctypes.c_uint64

_SIGNATURES = {
    "prefill_attention": ([_P] * 8 + [_I] * 7 + [_P, _F, _P] + [_I] * 6 + [_P], _I),
    "prefill_attention_validate": ([_P] * 8 + [_I] * 7 + [_P, _F, _P] + [_I] * 6, _I),
    "prefill_attention_tile_config": ([_I, _I, _I, _P, _P], _I),
    "prefill_attention_tile_config_ex": ([_I] * 8 + [_P, _P], _I),
    "prefill_attention_tile_bounds": ([_P, _P] + [_I] * 6 + [_P] + [_I] * 3 + [_P, _P], _I),
    "prefill_attention_strerror": ([_I], ctypes.c_char_p),
    "prefill_attention_ex": ([_P] * 8 + [_I] * 7 + [_P, _F, _P] + [_I] * 6
                             + [_P, _I, _I, _I, _I, _P, _U64, _P], _I),
    "prefill_attention_kv_splits": ([_I] * 10, _I),
    "prefill_attention_workspace_size": ([_I] * 4, _U64),
    "prefill_attention_tile_bounds_ex": ([_P, _P] + [_I] * 6 + [_P] + [_I] * 3
                                         + [_P, _I, _I, _I, _P, _P], _I),
    "prefill_attention_check_metadata": ([_P, _P, _P] + [_I] * 7 + [_P, _P], _I),
    "prefill_attention_ex_noalloc": ([_P] * 8 + [_I] * 7 + [_P, _F, _P] + [_I] * 6
                                     + [_P, _I, _I, _I, _I, _P], _I),
}

_lib = None


class PrefillError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s failed: %s (%d)" % (where, strerror(code), code))


_lib_path = None  # another build of the library to load instead (use_library)


def use_library(path: str):
    """Load ``path`` (another build of this library, e.g. a tile-shape variant)
    instead of the in-tree one from now on."""
    global _lib, _lib_path
    _lib, _lib_path = None, path
    return load_library()


def load_library():
    """Load the in-tree HIP library; raise if it has not been built."""
    global _lib
    if _lib is None:
        path = _lib_path or library_path()
        if not os.path.exists(path):
            raise RuntimeError("HIP library %s is not built; run __graft_entry__.build()" % path)
        lib = ctypes.CDLL(path)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def strerror(code: int) -> str:
    return load_library().prefill_attention_strerror(int(code)).decode()


def tile_config(head_size: int, num_heads: int, num_kv_heads: int, num_seqs: int = 0,
                max_q_len: int = 0, window_left: int = -1, window_right: int = -1,
                causal: bool = True):
    """(block_q, block_n): query tokens per Q tile and keys per KV tile, for a batch of
    ``num_seqs`` sequences of at most ``max_q_len`` new tokens under the given window
    (0, 0: a small batch; only head size 64 depends on the batch and window)."""
    bq, bn = ctypes.c_int32(), ctypes.c_int32()
    rc = load_library().prefill_attention_tile_config_ex(
        int(head_size), int(num_heads), int(num_kv_heads), int(num_seqs), int(max_q_len),
        int(window_left), int(window_right), int(bool(causal)), ctypes.byref(bq),
        ctypes.byref(bn))
    if rc != OK:
        raise PrefillError(rc, "prefill_attention_tile_config_ex")
    return bq.value, bn.value


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, dtype, shape=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def split_count(head_size: int, num_heads: int, num_kv_heads: int, num_seqs: int,
                total_q_tokens: int, max_q_len: int, requested: int = 0,
                window_left: int = -1, window_right: int = -1, causal: bool = True) -> int:
    """The split-KV segment count the library uses for ``requested`` (0 = automatic) on a
    batch of these sizes under the given window."""
    rc = load_library().prefill_attention_kv_splits(
        int(head_size), int(num_heads), int(num_kv_heads), int(num_seqs), int(total_q_tokens),
        int(max_q_len), int(window_left), int(window_right), int(bool(causal)), int(requested))
    if rc < 0:
        raise PrefillError(rc, "prefill_attention_kv_splits")
    return rc


def workspace_size(num_heads: int, head_size: int, total_q_tokens: int, splits: int) -> int:
    return int(load_library().prefill_attention_workspace_size(num_heads, head_size,
                                                               total_q_tokens, splits))


def _marshal(q, k_new, v_new, k_cache, v_cache, block_table, query_start_loc, ctx_lens,
             num_heads, num_kv_heads, head_size, page_size, window_left, window_right, causal,
             mm_ranges, scale, out, max_q_len, causal_per_seq):
    """Check the tensors and build the first 24 C arguments; returns (args, out, sizes)."""
    import torch
    H, Hkv, d, P = int(num_heads), int(num_kv_heads), int(head_size), int(page_size)
    T = int(q.shape[0])
    S = int(ctx_lens.shape[0])
    _check(q, "q", torch.bfloat16, (T, H, d))
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new must both be given or both be None")
    if k_new is not None:
        _check(k_new, "k_new", torch.bfloat16, (T, Hkv, d))
        _check(v_new, "v_new", torch.bfloat16, (T, Hkv, d))
    num_pages = int(k_cache.shape[0])
    _check(k_cache, "k_cache", torch.bfloat16, (num_pages, P, Hkv, d))
    _check(v_cache, "v_cache", torch.bfloat16, (num_pages, P, Hkv, d))
    _check(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != S:
        raise ValueError("block_table must be [num_seqs, max_pages_per_seq]")
    _check(query_start_loc, "query_start_loc", torch.int32, (S + 1,))
    _check(ctx_lens, "ctx_lens", torch.int32, (S,))
    R = 0
    if mm_ranges is not None:
        _check(mm_ranges, "mm_ranges", torch.int32)
        if mm_ranges.dim() != 3 or mm_ranges.shape[0] != S or mm_ranges.shape[2] != 2:
            raise ValueError("mm_ranges must be [num_seqs, max_mm_ranges, 2]")
        R = int(mm_ranges.shape[1])
        if R == 0:
            mm_ranges = None
    if causal_per_seq is not None:
        _check(causal_per_seq, "causal_per_seq", torch.int32, (S,))
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", torch.bfloat16, (T, H, d))
    if max_q_len is None:
        max_q_len = int((query_start_loc[1:] - query_start_loc[:-1]).max().item()) if S else 0
    base = (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(query_start_loc), _ptr(ctx_lens), H, Hkv, d, P, int(window_left),
            int(window_right), int(bool(causal)), _ptr(mm_ranges), float(scale), _ptr(out), S,
            T, int(max_q_len), num_pages, int(block_table.shape[1]), R)
    return base, out, (S, T, H, Hkv, d, int(max_q_len))


def prefill_attention(q, k_new, v_new, k_cache, v_cache, block_table, query_start_loc,
                      ctx_lens, num_heads: int, num_kv_heads: int, head_size: int,
                      page_size: int, window_left: int, window_right: int, causal: bool,
                      mm_ranges, scale: float, out=None, *, max_q_len: Optional[int] = None,
                      stream=None, causal_per_seq=None, mm_clamp: bool = True,
                      chunk_size: int = 0, chunk_lookback: int = -1, kv_splits: int = 1,
                      workspace=None):
    """Paged-KV prefill attention; returns ``out`` (bf16 [T, H, d]).

    ``k_new = v_new = None`` selects the cache-sourced mode.  ``max_q_len``
    (the largest new-token count of a sequence) should be passed by callers
    that know it; when omitted it is read back from ``query_start_loc``,
    which synchronises the stream.  The keyword-only mask variants and
    ``kv_splits`` select ``prefill_attention_ex``; with more than one split a
    workspace is taken from ``workspace`` (a uint8 device tensor) or
    allocated through torch.
    """
    import torch
    base, out, (S, T, H, Hkv, d, mq) = _marshal(
        q, k_new, v_new, k_cache, v_cache, block_table, query_start_loc, ctx_lens, num_heads,
        num_kv_heads, head_size, page_size, window_left, window_right, causal, mm_ranges,
        scale, out, max_q_len, causal_per_seq)
    plain = (causal_per_seq is None and mm_clamp and chunk_size == 0 and chunk_lookback == -1
             and kv_splits == 1)
    if plain:
        rc = load_library().prefill_attention(*base, _stream(stream))
        if rc != OK:
            raise PrefillError(rc, "prefill_attention")
        return out
    splits = split_count(d, H, Hkv, S, T, mq, int(kv_splits), window_left, window_right, causal)
    need = workspace_size(H, d, T, splits)
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        _check(workspace, "workspace", torch.uint8)
        if workspace.numel() < need:
            raise ValueError("workspace needs %d bytes" % need)
    ws_bytes = 0 if workspace is None else int(workspace.numel())
    rc = load_library().prefill_attention_ex(
        *base, _ptr(causal_per_seq), int(bool(mm_clamp)), int(chunk_size), int(chunk_lookback),
        int(kv_splits), _ptr(workspace), ws_bytes, _stream(stream))
    if rc != OK:
        raise PrefillError(rc, "prefill_attention_ex")
    return out


def prefill_attention_ex_noalloc(q, k_new, v_new, k_cache, v_cache, block_table,
                                 query_start_loc, ctx_lens, num_heads: int, num_kv_heads: int,
                                 head_size: int, page_size: int, window_left: int,
                                 window_right: int, causal: bool, mm_ranges, scale: float,
                                 out, *, max_q_len: int, stream=None, causal_per_seq=None,
                                 mm_clamp: bool = True, chunk_size: int = 0,
                                 chunk_lookback: int = -1, kv_splits: int = 1):
    """``prefill_attention_ex`` without a workspace: the split-KV partials use the
    library's static scratch, and nothing is allocated (``out`` and ``max_q_len``
    are required, so that no tensor is created and the stream is not synchronised)."""
    if out is None:
        raise ValueError("prefill_attention_ex_noalloc needs a caller-provided out tensor")
    base, out, _ = _marshal(
        q, k_new, v_new, k_cache, v_cache, block_table, query_start_loc, ctx_lens, num_heads,
        num_kv_heads, head_size, page_size, window_left, window_right, causal, mm_ranges,
        scale, out, max_q_len, causal_per_seq)
    rc = load_library().prefill_attention_ex_noalloc(
        *base, _ptr(causal_per_seq), int(bool(mm_clamp)), int(chunk_size), int(chunk_lookback),
        int(kv_splits), _stream(stream))
    if rc != OK:
        raise PrefillError(rc, "prefill_attention_ex_noalloc")
    return out


def tile_bounds(query_start_loc, ctx_lens, num_heads: int, num_kv_heads: int, head_size: int,
                window_left: int, window_right: int, causal: bool, mm_ranges, max_q_len: int,
                stream=None, *, causal_per_seq=None, mm_clamp: bool = True,
                chunk_size: int = 0, chunk_lookback: int = -1):
    """int32 [S, cdiv(max_q_len, block_q), 2] of (lo, hi) KV-tile loop ranges, on device."""
    import torch
    S = int(ctx_lens.shape[0])
    _check(query_start_loc, "query_start_loc", torch.int32, (S + 1,))
    _check(ctx_lens, "ctx_lens", torch.int32, (S,))
    R = 0
    if mm_ranges is not None:
        _check(mm_ranges, "mm_ranges", torch.int32)
        R = int(mm_ranges.shape[1])
        if R == 0:
            mm_ranges = None
    bq, _ = tile_config(head_size, num_heads, num_kv_heads)
    nt = -(-int(max_q_len) // bq)
    out = torch.empty((S, nt, 2), dtype=torch.int32, device=ctx_lens.device)
    if causal_per_seq is not None:
        _check(causal_per_seq, "causal_per_seq", torch.int32, (S,))
    rc = load_library().prefill_attention_tile_bounds_ex(
        _ptr(query_start_loc), _ptr(ctx_lens), int(num_heads), int(num_kv_heads),
        int(head_size), int(window_left), int(window_right), int(bool(causal)), _ptr(mm_ranges),
        S, int(max_q_len), R, _ptr(causal_per_seq), int(bool(mm_clamp)), int(chunk_size),
        int(chunk_lookback), _ptr(out), _stream(stream))
    if rc != OK:
        raise PrefillError(rc, "prefill_attention_tile_bounds_ex")
    return out


def check_metadata(block_table, query_start_loc, ctx_lens, page_size: int, num_pages: int,
                   total_q_tokens: int, max_q_len: int, cache_only: bool = False,
                   stream=None) -> int:
    """Device-side check of the metadata preconditions of ``prefill_attention``
    (``prefill_attention_check_metadata``): 0, or the OR of the ``BAD_*`` bits.
    Synchronises the stream to read the result."""
    import torch
    S = int(ctx_lens.shape[0])
    _check(query_start_loc, "query_start_loc", torch.int32, (S + 1,))
    _check(ctx_lens, "ctx_lens", torch.int32, (S,))
    _check(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or int(block_table.shape[0]) != S:
        raise ValueError("block_table must be [num_seqs, max_pages_per_seq]")
    flags = torch.full((1,), -1, dtype=torch.int32, device=ctx_lens.device)
    rc = load_library().prefill_attention_check_metadata(
        _ptr(block_table), _ptr(query_start_loc), _ptr(ctx_lens), int(bool(cache_only)),
        int(page_size), S, int(total_q_tokens), int(max_q_len), int(num_pages),
        int(block_table.shape[1]), _ptr(flags), _stream(stream))
    if rc != OK:
        raise PrefillError(rc, "prefill_attention_check_metadata")
    (torch.cuda.current_stream() if stream is None else stream).synchronize()
    return int(flags.item())


def validate(**kw) -> int:
    """Host-only argument check (``prefill_attention_validate``); integers stand in for
    pointers, nothing is dereferenced."""
    names = ["q", "k_new", "v_new", "k_cache", "v_cache", "block_table", "query_start_loc",
             "ctx_lens", "num_heads", "num_kv_heads", "head_size", "page_size", "window_left",
             "window_right", "causal", "mm_ranges", "scale", "out", "num_seqs",
             "total_q_tokens", "max_q_len", "num_pages", "max_pages_per_seq", "max_mm_ranges"]
    ptrs = {"q", "k_new", "v_new", "k_cache", "v_cache", "block_table", "query_start_loc",
            "ctx_lens", "mm_ranges", "out"}
    args = []
    for nm in names:
        v = kw[nm]
        if nm in ptrs:
            args.append(None if v is None else ctypes.c_void_p(int(v)))
        elif nm == "scale":
            args.append(float(v))
        else:
            args.append(int(v))
    return int(load_library().prefill_attention_validate(*args))
