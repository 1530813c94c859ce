"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects invalid arguments before touching the GPU."""

import ctypes
import os
import re

import pytest

import fp4_kv_cache_index_amd as csa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:char\s*\*|int|size_t)\s+(\w+)\s*\(", text, flags=re.M)
    return set(names)


def _lib_or_skip():
    if not os.path.exists(csa2.LIB_PATH):
        pytest.skip("libcsa2.so not built (run __graft_entry__.build())")
    return csa2.lib()


def test_header_and_binding_agree():
    assert _header_functions() == set(csa2.EXPORTS)


def test_library_exports_every_header_symbol():
    lib = _lib_or_skip()
    for name in _header_functions():
        assert getattr(lib, name) is not None


def test_status_strings_and_version():
    lib = _lib_or_skip()
    for s in range(6):
        assert lib.csa2_status_string(s)
    assert lib.csa2_status_string(99) == b"unknown status"
    assert re.match(rb"^\d+\.\d+\.\d+$", lib.csa2_version())


def test_invalid_arguments_are_rejected_on_the_host():
    lib = _lib_or_skip()
    fake = ctypes.c_void_p(0x1000)
    # d not a multiple of 16 / 32
    assert lib.kv_fp4_quantize(fake, 4, 15, 15, fake, 8, fake, 1, None) == 1
    assert lib.swa_fp8_quantize(fake, 4, 48, 48, fake, 48, fake, 1, None) == 1
    # zero rows is a no-op even with null pointers
    assert lib.kv_fp4_quantize(None, 0, 16, 16, None, 8, None, 1, None) == 0
    # null required pointer
    assert lib.kv_fp4_quantize(None, 4, 16, 16, fake, 8, fake, 1, None) == 1
    # misaligned code rows
    assert lib.kv_fp4_quantize(fake, 4, 16, 16, fake, 9, fake, 1, None) == 1
    # index_score_topk: k_top <= 0, bad D_I, misaligned ws, short workspace
    args = [fake, fake, fake, 0, 128, fake, None, 1, 1, 8, 128, 4096, 0, fake, None, 0, 0, None, None, fake, 1 << 30,
            None]
    assert lib.csa2_index_score_topk(*args) == 1
    args[12] = 64
    args[10] = 96  # D_I multiple of 32 but not compiled
    assert lib.csa2_index_score_topk(*args) == 2
    args[10] = 128
    args[19] = ctypes.c_void_p(0x1010)  # workspace not 256-aligned
    assert lib.csa2_index_score_topk(*args) == 1
    args[19] = fake
    args[20] = 16  # too small
    assert lib.csa2_index_score_topk(*args) == 3
    # key rows 4 MiB apart or more are beyond the scan's 32-bit row offsets
    args[20] = 1 << 30
    args[4] = 1 << 22
    assert lib.csa2_index_score_topk(*args) == 2
    args[4] = 128
    # pool requested with a bad block size
    args[15], args[16], args[17], args[18] = 3, 16, fake, fake
    assert lib.csa2_index_score_topk(*args) == 1
    # trace attach validation
    assert lib.csa2_trace_attach(None, None, 4) == 1
    assert lib.csa2_trace_attach(None, None, 0) == 0
    n = ctypes.c_int32(-1)
    assert lib.csa2_trace_detach(ctypes.byref(n)) == 0 and n.value == 0
    # the name filter needs an attached trace and a name below 64 characters
    assert lib.csa2_trace_only(b"index_score") == 1
    assert lib.csa2_trace_attach(None, None, 0) == 0
    assert lib.csa2_trace_only(b"x" * 64) == 1
    assert lib.csa2_trace_only(b"index_score") == 0
    assert lib.csa2_trace_only(None) == 0
    assert lib.csa2_trace_detach(ctypes.byref(n)) == 0 and n.value == 0


def test_workspace_sizes_are_monotone():
    lib = _lib_or_skip()
    a = lib.csa2_index_score_topk_workspace_size(1, 1, 4096, 256, 0, 0)
    b = lib.csa2_index_score_topk_workspace_size(2, 1, 4096, 256, 0, 0)
    c = lib.csa2_index_score_topk_workspace_size(2, 1, 4096, 256, 8, 64)
    # more rows need more; either mode holds at least the keys
    assert 0 < a < b and c >= 2 * 4096 * 4 and b >= 2 * 4096 * 4
    # keys dominate: 4 bytes per (row, position)
    big = lib.csa2_index_score_topk_workspace_size(64, 1, 65536, 2048, 0, 0)
    assert big >= 64 * 65536 * 4
    assert lib.csa2_hier_pool_topk_workspace_size(4, 1, 16384, 2048) >= 4 * 16384 * 4


def test_prefill_chunk_workspace_is_bounded():
    """Dense prefill chunks (16 or more query rows per sequence) need no
    [rows][positions] score keys: a 4096-query chunk's default workspace
    stays under 100 MB on contexts from 266,240 to 4M tokens, against the
    4 bytes per (query, position) of the stored-key workspace (4.4 GB of keys
    at 266,240)."""
    lib = _lib_or_skip()
    for n in (266240, 1 << 20, 4 << 20):
        ws = lib.csa2_index_score_topk_workspace_size(1, 4096, n, 2048, 0, 0)
        assert ws < 100 * 10**6, (n, ws)
        assert lib.csa2_index_score_topk_workspace_size_stored(1, 4096, n, 2048, 0, 0) >= 4096 * n * 4
    # the largest chunk the bound is stated for
    assert lib.csa2_index_score_topk_workspace_size(1, 65535, 4 << 20, 8192, 0, 0) < 100 * 10**6
    # more than 8192 selected positions per row, decode rows and pooled calls:
    # the stored keys in either size
    for args in ((1, 64, 266240, 9000, 0, 0), (64, 1, 65536, 2048, 0, 0), (4, 1, 65536, 2048, 8, 2048)):
        assert lib.csa2_index_score_topk_workspace_size(*args) == \
            lib.csa2_index_score_topk_workspace_size_stored(*args)
    # a short chunk keeps the smaller of the two
    assert lib.csa2_index_score_topk_workspace_size(1, 16, 256, 64, 0, 0) <= \
        lib.csa2_index_score_topk_workspace_size_stored(1, 16, 256, 64, 0, 0)
