"""The C-ABI library loads and exports every entry point include/specverify.h
declares, with the binding's argument counts matching the header.  Host-only
calls (version, status strings, workspace queries, argument validation that
returns before any launch) run without a GPU."""
import ctypes
import re
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "specverify.h"


def declared():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    out = {}
    for m in re.finditer(r"\b(?:int|size_t|const char\s*\*)\s*(spec_\w+)\s*\(([^)]*)\)\s*;", text):
        params = [p for p in m.group(2).split(",") if p.strip() and p.strip() != "void"]
        out[m.group(1)] = len(params)
    return out


@pytest.fixture(scope="module")
def lib():
    from tree_attention_verification_beam_amd import binding
    if not binding.LIB_PATH.exists():
        import __graft_entry__
        __graft_entry__.build()
    return binding


def test_header_lists_the_calls():
    d = declared()
    for name in ("spec_build_tree", "spec_tree_attention", "spec_verify", "spec_kv_compact",
                 "spec_beam_topk", "spec_select_tree", "spec_last_device_status"):
        assert name in d


def test_every_declared_symbol_is_exported_and_bound(lib):
    cdll = lib.load()
    for name, n_args in declared().items():
        assert hasattr(cdll, name), name
        assert name in lib.SIGNATURES, name
        assert len(lib.SIGNATURES[name][1]) == n_args, name


def test_host_only_calls(lib):
    cdll = lib.load()
    assert cdll.spec_version() >= 100
    assert cdll.spec_status_string(-3) == b"SPEC_ERR_CAPACITY"
    # workspace queries are pure host arithmetic
    assert cdll.spec_verify_workspace_size(0, 64, 17, 128000, 0) > 0
    assert cdll.spec_tree_attention_workspace_size(1, 64, 17, 32, 32, 128, 1024) == 0
    assert cdll.spec_tree_attention_workspace_size(1, 4, 49, 32, 8, 128, 32768) > 0
    assert cdll.spec_beam_topk_workspace_size(1, 8, 8, 32000) > 0
    assert cdll.spec_beam_topk_workspace_size(1, 8, 17, 32000) == 0


def test_select_tree_rejects_before_launch(lib):
    cdll = lib.load()
    args = [16] * 7 + [None, 16]
    assert cdll.spec_select_tree(1, 10, 11, *args) == -1      # budget above the candidates
    assert cdll.spec_select_tree(1, 2000, 8, *args) == -3     # too many candidates
    assert cdll.spec_select_tree(1, 300, 128, *args) == -3    # budget beyond a tree
    assert cdll.spec_select_tree(1, 10, 4, None, *args[1:]) == -1
    assert cdll.spec_select_tree(0, 10, 4, *([None] * 9)) == 0


def test_beam_topk_rejects_before_launch(lib):
    cdll = lib.load()
    # K_out beyond the limit or beyond K_in * V, and mismatched history buffers
    assert cdll.spec_beam_topk(1, 8, 17, 32000, 16, None, 16, 16, 16, None, 0, None, 16,
                               1 << 20, None) == -3
    assert cdll.spec_beam_topk(1, 1, 6, 5, 16, None, 16, 16, 16, None, 0, None, 16,
                               1 << 20, None) == -3
    assert cdll.spec_beam_topk(1, 2, 2, 8, 16, None, 16, 16, 16, 16, 3, None, 16,
                               1 << 20, None) == -1
    assert cdll.spec_beam_topk(1, 2, 2, 8, 16, None, 16, 16, 16, None, 0, None, None, 0,
                               None) == -4
    assert cdll.spec_beam_topk(0, 2, 2, 8, None, None, None, None, None, None, 0, None, None,
                               0, None) == 0


def test_validation_rejects_before_launch(lib):
    cdll = lib.load()
    # T_cap above the limit, bad mode, bad head grouping: rejected on the host
    assert cdll.spec_build_tree(0, 1, 4, 4, 129, 1, None, 1, 1, 1, 1, 1, 1, None, None, None) == -3
    assert cdll.spec_build_tree(0, 1, 8, 8, 17, 1, None, 1, 1, 1, 1, 1, 1, None, None, None) == -3
    assert cdll.spec_verify(7, 1, 17, 100, 0, *([1] * 17), 0, None, None) == -1
    assert cdll.spec_tree_attention(1, 1, 17, 6, 4, 128, 100, 64, *([1] * 6), 0.0, 1, None, 0,
                                    None, None) == -1
    assert cdll.spec_kv_compact(1, 1, 8, 128, 10, 200, *([1] * 5), 16, 256, None, None) == -3


def test_empty_batch_is_a_no_op(lib):
    """B = 0 returns SPEC_OK before any launch, whatever the pointers."""
    cdll = lib.load()
    assert cdll.spec_build_tree(0, 0, 4, 4, 17, None, None, None, None, None, None, None, None,
                                None, None, None) == 0
    assert cdll.spec_tree_attention(1, 0, 17, 32, 32, 128, 1100, 1024, *([None] * 6), 0.0, None,
                                    None, 0, None, None) == 0
    assert cdll.spec_verify(0, 0, 17, 1000, 0, *([None] * 17), 0, None, None) == 0
    assert cdll.spec_kv_compact(1, 0, 8, 128, 1100, 17, *([None] * 5), None, 0, None,
                                None) == 0


def test_attention_rejects_a_row_block_beyond_32_bit_ranges(lib):
    """bf16 tile loads address one (b, KV head) cache row block through 32-bit
    buffer ranges: cache_cap * D * 2 >= 2^31 is refused on the host."""
    cdll = lib.load()
    cap = (1 << 23) + 1  # * 128 * 2 bytes > 2^31
    assert cdll.spec_tree_attention(1, 1, 17, 32, 32, 128, cap, 1024, *([16] * 6), 0.0, 16,
                                    None, 0, None, None) == -2


def test_verify_refuses_a_vocabulary_beyond_the_row_merge(lib):
    """The one-pass verify merges a row's chunk partials in LDS batches of 1024
    chunks of at most 16384 entries: a larger vocabulary is refused on the host
    (workspace size 0, SPEC_ERR_UNSUPPORTED) before anything is launched."""
    cdll = lib.load()
    big = 64 * 256 * 1024 + 1
    assert cdll.spec_verify_workspace_size(0, 1, 17, 64 * 256 * 1024, 0) > 0
    for mode in (0, 1, 2):
        assert cdll.spec_verify_workspace_size(mode, 1, 17, big, 4) == 0
        assert cdll.spec_verify(mode, 1, 17, big, 4, *([16] * 17), 1 << 30, None, None) == -2
    # the walk addresses a row through a 32-bit byte range
    assert cdll.spec_verify(3, 1, 17, 1 << 29, 0, *([16] * 17), 1 << 30, None, None) == -2


def test_compact_refuses_a_path_beyond_its_buffer(lib):
    """One path's rows of one KV head go through a 64 KiB LDS buffer:
    (T_cap - 1) rows of D values must fit it.  fp32 rows of 128 values at
    T_cap 128 (63.5 KiB) pass the check, 256 values are refused; a missing or
    small workspace is refused too."""
    cdll = lib.load()
    ptrs = [16] * 5
    assert cdll.spec_kv_compact(0, 1, 8, 256, 10000, 128, *ptrs, 256, 256, None, None) == -2
    assert cdll.spec_kv_compact(0, 1, 8, 128, 10000, 128, *ptrs, None, 0, None, None) == -4
    assert cdll.spec_kv_compact(0, 300, 8, 128, 10000, 128, *ptrs, 256, 256, None, None) == -4
    assert cdll.spec_kv_compact_workspace_size(300) == 1280


def test_verify_noalloc_refuses_beyond_its_array(lib):
    """The no-allocation verify takes at most 4 MiB of workspace from the
    library's own device array; a larger need is refused on the host."""
    cdll = lib.load()
    assert cdll.spec_verify_workspace_size(3, 4096, 17, 1000, 0) > 4 << 20
    assert cdll.spec_verify_noalloc(3, 4096, 17, 1000, 0, *([16] * 16), None, None) == -3
    assert cdll.spec_verify_noalloc(0, 0, 17, 1000, 0, *([None] * 16), None, None) == 0
