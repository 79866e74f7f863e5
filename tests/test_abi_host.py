"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad scalar arguments without touching a GPU."""

import os
import re
import subprocess

import pytest

import paged_kv_prefill_attention_amd as ppa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ppa.library_path()):
        ppa.build()
    return ppa.load_library()


def declared_functions():
    names = []
    inc = os.path.join(ROOT, "include")
    for fn in sorted(os.listdir(inc)):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(inc, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return names


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert "prefill_attention" in names and "prefill_attention_tile_bounds" in names
    out = subprocess.run(["nm", "-D", "--defined-only", ppa.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for nm in names:
        assert nm in exported, nm
        assert hasattr(lib, nm)


GOOD = dict(q=1, k_new=2, v_new=3, k_cache=4, v_cache=5, block_table=6, query_start_loc=7,
            ctx_lens=8, num_heads=8, num_kv_heads=2, head_size=128, page_size=544,
            window_left=-1, window_right=-1, causal=1, mm_ranges=None, scale=0.088, out=9,
            num_seqs=4, total_q_tokens=100, max_q_len=40, num_pages=10, max_pages_per_seq=8,
            max_mm_ranges=0)


@pytest.mark.parametrize("change,code", [
    ({}, ppa.OK),
    ({"num_heads": 6, "num_kv_heads": 4}, ppa.ERR_INVALID_ARG),
    ({"num_kv_heads": 0}, ppa.ERR_INVALID_ARG),
    ({"page_size": 0}, ppa.ERR_INVALID_ARG),
    ({"window_left": -2}, ppa.ERR_INVALID_ARG),
    ({"window_right": -5}, ppa.ERR_INVALID_ARG),
    ({"causal": 2}, ppa.ERR_INVALID_ARG),
    ({"scale": 0.0}, ppa.ERR_INVALID_ARG),
    ({"scale": float("nan")}, ppa.ERR_INVALID_ARG),
    ({"scale": float("inf")}, ppa.ERR_INVALID_ARG),
    ({"max_mm_ranges": 3}, ppa.ERR_INVALID_ARG),          # ranges without a pointer
    ({"max_mm_ranges": 3, "mm_ranges": 10}, ppa.OK),
    ({"max_mm_ranges": -1}, ppa.ERR_INVALID_ARG),
    ({"k_new": None}, ppa.ERR_INVALID_ARG),                # only one of k_new/v_new
    ({"k_new": None, "v_new": None}, ppa.OK),             # cache-sourced mode
    ({"q": None}, ppa.ERR_INVALID_ARG),
    ({"out": None}, ppa.ERR_INVALID_ARG),
    ({"block_table": None}, ppa.ERR_INVALID_ARG),
    ({"head_size": 96}, ppa.ERR_UNSUPPORTED),
    ({"head_size": 64}, ppa.OK),
    ({"head_size": 256}, ppa.OK),
    ({"page_size": 1 << 17}, ppa.ERR_UNSUPPORTED),
    ({"max_pages_per_seq": 1 << 20}, ppa.ERR_INVALID_ARG),  # beyond 2^24 positions
    ({"num_seqs": 0, "q": None}, ppa.OK),                 # empty batch: nothing to do
    ({"max_q_len": 0}, ppa.OK),
    ({"num_seqs": -1}, ppa.ERR_INVALID_ARG),
])
def test_validate_codes(lib, change, code):
    args = dict(GOOD)
    args.update(change)
    assert ppa.validate(**args) == code


def test_invalid_call_returns_before_launch(lib):
    # an unsupported head size is rejected on the host, before any HIP call
    import ctypes
    rc = lib.prefill_attention(*([None] * 8), 8, 2, 96, 16, -1, -1, 1, None, 0.1, None,
                               1, 10, 10, 1, 1, 0, None)
    assert rc == ppa.ERR_UNSUPPORTED
    rc = lib.prefill_attention(*([None] * 8), 8, 3, 128, 16, -1, -1, 1, None, 0.1, None,
                               1, 10, 10, 1, 1, 0, None)
    assert rc == ppa.ERR_INVALID_ARG


def test_tile_config(lib):
    # 8 wavefronts x 32 rows for head sizes 128/256, 4 x 32 rows for 64
    assert ppa.tile_config(128, 64, 64) == (256, 64)
    assert ppa.tile_config(64, 8, 8) == (128, 64)
    # d = 64 takes 32-key tiles (four workgroups per CU: 1024 slots on 256 CUs without a GPU to
    # ask) for four rounds of Q-tile items, or for one round when a window of at most 2048 keys
    # per row bounds every loop
    win = dict(window_left=64, window_right=64, causal=False)          # 129 keys per row
    assert ppa.tile_config(64, 8, 8, 1, 16384) == (128, 64)             # 128 x 8 = 1024 items
    assert ppa.tile_config(64, 8, 8, 1, 16384, **win) == (128, 32)
    assert ppa.tile_config(64, 8, 8, 1, 16256, **win) == (128, 64)     # 127 x 8 = 1016 items
    assert ppa.tile_config(64, 8, 8, 1, 128 * 512) == (128, 32)         # 4096 items
    assert ppa.tile_config(64, 8, 8, 1, 128 * 512 - 128) == (128, 64)   # 4088 items
    assert ppa.tile_config(64, 64, 64, 8, 1024) == (128, 32)            # 8 x 8 x 64 = 4096
    assert ppa.tile_config(64, 16, 8, 4, 512) == (64, 64)               # 4 x 8 x 8 = 256 items
    assert ppa.tile_config(64, 16, 8, 4, 4096) == (64, 64)              # 2048 items
    assert ppa.tile_config(64, 16, 8, 4, 4096, 2047, -1, True) == (64, 32)   # 2048 keys
    assert ppa.tile_config(64, 16, 8, 4, 4096, 2048, -1, True) == (64, 64)   # 2049 keys
    assert ppa.tile_config(64, 16, 8, 4, 4096, 1023, 1024, False) == (64, 32)  # 2048 keys
    assert ppa.tile_config(64, 16, 8, 4, 4096, 1023, 1025, False) == (64, 64)
    assert ppa.tile_config(64, 16, 8, 4, 4096, -1, 10, False) == (64, 64)    # unbounded left
    assert ppa.tile_config(64, 16, 8, 4, 4096, 100, -1, False) == (64, 64)   # unbounded right
    assert ppa.tile_config(128, 64, 64, 8, 1024) == (256, 64)   # other head sizes: one shape
    assert ppa.tile_config(256, 8, 2, 8, 2048, 64, 64, False) == (64, 32)
    assert ppa.tile_config(256, 8, 2) == (64, 32)     # 4 query heads share a tile
    assert ppa.tile_config(256, 16, 8) == (128, 32)
    assert ppa.tile_config(128, 64, 1) == (4, 64)     # MQA: 64 heads x 4 tokens
    assert ppa.tile_config(128, 24, 8) == (256, 64)   # group 3 does not divide the rows
    with pytest.raises(ppa.PrefillError):
        ppa.tile_config(80, 8, 8)
    with pytest.raises(ppa.PrefillError):
        ppa.tile_config(128, 8, 3)


def test_strerror(lib):
    assert ppa.strerror(0) == "ok"
    assert "invalid" in ppa.strerror(-1)
    assert "unsupported" in ppa.strerror(-2)
    assert "unknown" in ppa.strerror(7)
    assert "scratch" in ppa.strerror(ppa.ERR_SCRATCH)


def test_noalloc_rejects_bad_arguments_before_touching_a_device(lib):
    """The allocation-free entry point runs the host checks (arguments, mask options,
    split count) before it looks its scratch up on the device, so these calls need
    no GPU; an empty batch returns OK without a launch."""
    import ctypes
    P = [None] * 8
    common = (8, 2, 128, 16, -1, -1, 1, None, 0.1, None, 0, 0, 0, 1, 1, 0)
    assert lib.prefill_attention_ex_noalloc(*P, *common, None, 1, 0, -1, 1, None) == 0
    F = [ctypes.c_void_p(4096 * (i + 1)) for i in range(8)]
    nonempty = (8, 2, 128, 16, -1, -1, 1, None, 0.1, ctypes.c_void_p(1 << 20), 1, 10, 10, 1,
                1, 0)
    for bad in [(None, 2, 0, -1, 1), (None, 1, -1, -1, 1), (None, 1, 16, -2, 1),
                (None, 1, 0, -1, -1), (None, 1, 0, -1, 65)]:
        assert lib.prefill_attention_ex_noalloc(*F, *nonempty, *bad, None) == ppa.ERR_INVALID_ARG
    bad_heads = (6, 4) + nonempty[2:]
    assert lib.prefill_attention_ex_noalloc(*F, *bad_heads, None, 1, 0, -1, 1, None) == \
        ppa.ERR_INVALID_ARG


def test_invalid_ex_options_return_before_launch(lib):
    # option checks run on the host before any pointer is touched or kernel launched
    P = [None] * 8
    common = (8, 2, 128, 16, -1, -1, 1, None, 0.1, None, 0, 0, 0, 1, 1, 0)
    # empty batch with valid options: OK without a launch
    assert lib.prefill_attention_ex(*P, *common, None, 1, 0, -1, 1, None, 0, None) == 0
    # non-null stand-in pointers (never dereferenced: every case fails a host check)
    import ctypes
    F = [ctypes.c_void_p(4096 * (i + 1)) for i in range(8)]
    nonempty = (8, 2, 128, 16, -1, -1, 1, None, 0.1, ctypes.c_void_p(1 << 20), 1, 10, 10, 1,
                1, 0)
    for bad in [(None, 2, 0, -1, 1), (None, 1, -1, -1, 1), (None, 1, 16, -2, 1),
                (None, 1, 0, -1, -1), (None, 1, 0, -1, 65),
                (None, 1, 0, -1, 4)]:  # four splits without a workspace
        rc = lib.prefill_attention_ex(*F, *nonempty, *bad, None, 0, None)
        assert rc == ppa.ERR_INVALID_ARG, bad


def test_split_count_and_workspace_size(lib):
    # explicit counts pass through; automatic splits only small batches
    assert ppa.split_count(128, 64, 64, 8, 3317, 873, 1) == 1
    assert ppa.split_count(128, 64, 64, 8, 3317, 873, 5) == 5
    assert ppa.split_count(128, 64, 64, 8, 3317, 873, 0) == 1   # <= 20 Q tiles x 64 heads
    # at most half a round of items (W = 256 at d=128 and 256, 512 for the 64-key d=64
    # shape without a GPU to ask): k segments per item fill one round, or k + 1 if k
    # would leave more than a quarter of it idle
    assert ppa.split_count(128, 32, 8, 2, 456, 256, 0) == 4     # 2*4 tiles x 8 = 64 items
    assert ppa.split_count(128, 16, 16, 2, 1350, 700, 0) == 2   # 96 items: 192 of 256
    assert ppa.split_count(256, 8, 2, 4, 2560, 1024, 0) == 3    # 86 items: 172 < 192
    assert ppa.split_count(64, 16, 8, 1, 512, 512, 0) == 8      # 64 items, W = 512
    assert ppa.split_count(64, 8, 8, 1, 64, 64, 0) == 16        # 8 items, capped at 16
    # the 8-sequence d=256 GQA batch: max_q_len alone allows 8*32 tiles x 2 KV heads = 512
    # items, but 10155 tokens allow at most (10155 + 8*63) / 64 = 166 tiles -> 332 items
    assert ppa.split_count(256, 8, 2, 8, 10155, 2048, 0) == 2
    # two to four rounds of items with a last round at most a quarter full: tail splitting
    assert ppa.split_count(256, 16, 8, 1, 12454, 12454, 0) == 4   # 784 items, 16 past 3 rounds
    # d = 64 without a window: 64-key tiles, 512 per round
    assert ppa.split_count(64, 8, 8, 1, 33024, 33024, 0) == 1     # 2064 items: past 4 rounds
    assert ppa.split_count(64, 8, 8, 1, 32768, 32768, 0) == 1     # 2048 items: whole rounds
    assert ppa.split_count(64, 8, 8, 1, 16384, 16384, 0) == 1     # 1024 items: whole rounds
    assert ppa.split_count(64, 8, 8, 1, 16640, 16640, 0) == 4     # 1040 items: 2 rounds + 16
    # d = 64 under a short window: 32-key tiles, 1024 per round
    win = dict(window_left=64, window_right=64, causal=False)
    assert ppa.split_count(64, 8, 8, 1, 33024, 33024, 0, **win) == 4   # 2 rounds + 16
    assert ppa.split_count(64, 8, 8, 1, 32768, 32768, 0, **win) == 1
    assert ppa.split_count(64, 8, 8, 1, 16384, 16384, 0, **win) == 1
    assert ppa.split_count(64, 8, 8, 1, 16640, 16640, 0, **win) == 1   # 1 round + 16: short
    # fewer than two rounds: long items are split, but not under a short window (2048 keys)
    assert ppa.split_count(64, 8, 8, 1, 4096, 4096, 0) == 2                  # 256 items
    assert ppa.split_count(64, 8, 8, 1, 4096, 4096, 0, 2047, -1, True) == 1
    assert ppa.split_count(64, 8, 8, 1, 4096, 4096, 0, 2048, -1, True) == 2
    assert ppa.split_count(128, 32, 8, 2, 456, 256, 0, 100, 100, False) == 1
    assert ppa.split_count(128, 32, 8, 2, 456, 256, 0, -1, 100, False) == 4  # left open
    assert ppa.split_count(256, 8, 2, 8, 1 << 20, 2048, 0) == 1   # 512 items: whole rounds
    assert ppa.split_count(128, 8, 8, 1, 256 * 80, 256 * 80, 0) == 1  # tail of 128: too full
    assert ppa.split_count(128, 64, 64, 8, 1 << 20, 1024, 0) == 1  # 2048 items: no split
    with pytest.raises(ppa.PrefillError):
        ppa.split_count(128, 8, 8, 1, 64, 64, 65)
    with pytest.raises(ppa.PrefillError):
        ppa.split_count(128, 8, 8, 1, -1, 64, 0)
    with pytest.raises(ppa.PrefillError):
        ppa.split_count(64, 8, 8, 1, 64, 64, 0, window_left=-2)
    with pytest.raises(ppa.PrefillError):
        ppa.tile_config(64, 8, 8, 1, 64, window_left=0, window_right=-2)
    assert ppa.workspace_size(8, 128, 100, 1) == 0
    rows = 3 * 100 * 8
    o_bytes = -(-(rows * 128 * 4) // 256) * 256
    assert ppa.workspace_size(8, 128, 100, 3) == o_bytes + rows * 8


def test_check_metadata_rejects_bad_arguments_before_launch(lib):
    # host checks only: stand-in pointers are never dereferenced
    import ctypes
    bt, qsl, ctx, flags = (ctypes.c_void_p(4096 * (i + 1)) for i in range(4))
    # (block_table, qsl, ctx, cache_only, page_size, S, T, max_q_len, num_pages, max_pages, flags)
    good = [bt, qsl, ctx, 0, 16, 2, 10, 8, 4, 3, flags]
    for idx, value in [(1, None), (10, None), (2, None), (0, None), (3, 2), (4, 0), (5, -1),
                       (6, -1), (7, -1), (8, -1), (9, -1)]:
        args = list(good)
        args[idx] = value
        rc = lib.prefill_attention_check_metadata(*args, None)
        assert rc == ppa.ERR_INVALID_ARG, (idx, value)
