"""C-ABI checks that need no GPU: the library loads, exports exactly what
include/mla.h declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|mla_status|const char \*)\s*(mla_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    from mla_paged_kv_metadata_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmla.so is not built (python -m mla_paged_kv_metadata_amd.build)")
    return _lib.load()


def test_header_declares_expected_entry_points():
    from mla_paged_kv_metadata_amd import _lib
    assert declared_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    from mla_paged_kv_metadata_amd import _lib
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mla_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    # nothing else of ours leaks out
    assert exported == set(declared_functions())


def test_version(lib):
    assert lib.mla_version() == 2


def test_metadata_size_for_parts(lib):
    md = ctypes.c_size_t()
    ns = ctypes.c_size_t()
    assert lib.mla_metadata_size_for_parts(64, 1, 0, 256, ctypes.byref(md), ctypes.byref(ns)) == 0
    assert md.value == 8 + 8 * 256 + 64 and ns.value == 65
    # sparse: one unit per (sequence, query token)
    assert lib.mla_metadata_size_for_parts(4, 3, 16, 8, ctypes.byref(md), ctypes.byref(ns)) == 0
    assert md.value == 8 + 64 + 12 and ns.value == 13
    assert lib.mla_metadata_size_for_parts(-1, 1, 0, 8, ctypes.byref(md), ctypes.byref(ns)) == -1
    assert lib.mla_metadata_size_for_parts(1, 1, 0, 0, ctypes.byref(md), ctypes.byref(ns)) == -1
    assert b"num_parts" in lib.mla_last_error()
    assert lib.mla_metadata_size_for_parts(1, 1, 0, 2048, ctypes.byref(md), ctypes.byref(ns)) == 0
    assert lib.mla_metadata_size_for_parts(1, 1, 0, 2049, ctypes.byref(md), ctypes.byref(ns)) == -1
    # sparse units are (sequence, token) pairs counted in an int
    assert lib.mla_metadata_size_for_parts(1 << 16, 1 << 15, 8, 8, ctypes.byref(md), ctypes.byref(ns)) == -1
    assert b"2^31" in lib.mla_last_error()
    assert lib.mla_metadata_size_for_parts(1 << 16, 1 << 15, 0, 8, ctypes.byref(md), ctypes.byref(ns)) == 0
    fake = ctypes.c_void_p(16)   # never dereferenced: the count check fails first
    assert lib.mla_get_metadata(fake, fake, 1 << 16, 1 << 15, 1 << 15, 1, 8, 8, fake, fake, None) == -1
    assert b"2^31" in lib.mla_last_error()


def _args(**kw):
    from mla_paged_kv_metadata_amd import _lib
    a = _lib.MlaDecodeArgs()
    a.batch, a.s_q, a.h_q, a.h_kv = 2, 1, 16, 1
    a.d_qk, a.d_v, a.page_size = 576, 512, 64
    a.num_pages, a.max_blocks_per_seq = 4, 3
    a.kv_format = 0
    a.softmax_scale = 576 ** -0.5
    a.num_parts = 8
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_workspace_size_is_host_only(lib):
    n = ctypes.c_size_t()
    a = _args()
    assert lib.mla_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 0
    slots = 2 + 8
    o = -(-slots * 16 * 512 * 2 // 256) * 256   # bf16 partial rows
    l = -(-slots * 16 * 4 // 256) * 256
    assert n.value == o + l


@pytest.mark.parametrize("field,value,code", [
    ("h_kv", 2, -2), ("d_qk", 512, -2), ("d_v", 576, -2), ("page_size", 16, -2),
    ("kv_format", 7, -2), ("s_q", 0, -1), ("h_q", 0, -1), ("num_parts", 0, -1), ("num_parts", 2049, -1),
    ("max_blocks_per_seq", 0, -1), ("topk", 5, -1), ("softmax_scale", float("inf"), -1),
])
def test_decode_rejects_bad_arguments_without_launching(lib, field, value, code):
    a = _args(**{field: value})
    assert lib.mla_decode_kvcache(ctypes.byref(a), None) == code
    assert lib.mla_last_error() != b""
    # the debug audit applies the same checks before it reads any buffer
    assert lib.mla_validate_inputs(ctypes.byref(a), None) == code
    assert lib.mla_last_error() != b""


def test_query_row_and_grid_limits(lib):
    n = ctypes.c_size_t()
    # a 32K-token prefill over 128 heads (4.2M query rows) is in range
    a = _args(batch=1, s_q=32768, h_q=128, causal=1, num_parts=1)
    assert lib.mla_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 0
    assert n.value >= 2 * 32768 * 128 * 512 * 2
    # rows counted in 32 bits: 2^31 rows are refused, also for an empty batch
    for b in (1, 0):
        a = _args(batch=b, s_q=1 << 16, h_q=1 << 15)
        assert lib.mla_decode_kvcache(ctypes.byref(a), None) == -1
        assert b"query rows" in lib.mla_last_error()
    # one workgroup per (part, row tile) in a 1-D grid
    a = _args(batch=1, s_q=1 << 20, h_q=1 << 10, num_parts=2048)
    assert lib.mla_decode_kvcache(ctypes.byref(a), None) == -1
    assert b"grid" in lib.mla_last_error()


def test_decode_rejects_null_pointers_and_small_workspace(lib):
    a = _args()
    assert lib.mla_decode_kvcache(ctypes.byref(a), None) == -1   # q etc. are NULL
    fake = 0x1000   # never dereferenced: the workspace check fails first
    a = _args(q=fake, kcache=fake, block_table=fake, cache_seqlens=fake, tile_metadata=fake,
              num_splits=fake, out=fake, lse=fake, workspace=fake, workspace_bytes=16)
    assert lib.mla_decode_kvcache(ctypes.byref(a), None) == -3
    assert b"workspace" in lib.mla_last_error()


def test_get_metadata_rejects_bad_arguments(lib):
    assert lib.mla_get_metadata(None, None, 2, 1, 16, 2, 0, 8, None, None, None) == -2
    assert lib.mla_get_metadata(None, None, 2, 2, 3, 1, 0, 8, None, None, None) == -1
    assert lib.mla_get_metadata(None, None, 2, 1, 16, 1, 4, 8, None, None, None) == -1
    assert lib.mla_get_metadata(None, None, 2, 1, 16, 1, 0, 8, None, None, None) == -1


def test_empty_batch_decode_is_a_no_op(lib):
    a = _args(batch=0)
    assert lib.mla_decode_kvcache(ctypes.byref(a), None) == 0
    assert lib.mla_validate_inputs(ctypes.byref(a), None) == 0


def test_validate_checks_pointers_and_workspace_before_reading(lib):
    assert lib.mla_validate_inputs(None, None) == -1
    a = _args()
    assert lib.mla_validate_inputs(ctypes.byref(a), None) == -1   # q etc. are NULL
    fake = 0x1000   # never dereferenced: the workspace check fails first
    a = _args(q=fake, kcache=fake, block_table=fake, cache_seqlens=fake, tile_metadata=fake,
              num_splits=fake, out=fake, lse=fake, workspace=fake, workspace_bytes=16)
    assert lib.mla_validate_inputs(ctypes.byref(a), None) == -3
    assert b"workspace" in lib.mla_last_error()


def test_append_rejects_bad_arguments_without_launching(lib):
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: the checks fail first
    assert lib.mla_append_kv(None, None, 0, 0, None, 0, None) == 0      # nothing to write
    assert lib.mla_append_kv(fake, fake, -1, 0, fake, 4, None) == -1
    assert lib.mla_append_kv(fake, fake, 4, 7, fake, 4, None) == -2
    assert lib.mla_append_kv(fake, fake, 4, 1, fake, -1, None) == -1
    assert lib.mla_append_kv(None, fake, 4, 1, fake, 4, None) == -1
    assert lib.mla_append_kv(ctypes.c_void_p(0x1008), fake, 4, 1, fake, 4, None) == -1   # misaligned
    assert b"aligned" in lib.mla_last_error()


def test_status_returning_calls_are_declared_so():
    """Every entry point except the version and the error text returns an
    mla_status."""
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    status = set(re.findall(r"^\s*mla_status\s+(mla_\w+)\s*\(", src, flags=re.M))
    assert status == set(declared_functions()) - {"mla_version", "mla_last_error"}


def test_python_decode_signature_follows_the_boundary():
    """mla_decode_kvcache(q, kcache, block_table, cache_seqlens,
    softmax_scale=None, causal=False, indices=None, metadata=None): the
    schedule is optional (built on the call's stream when omitted)."""
    import inspect
    from mla_paged_kv_metadata_amd import mla_decode_kvcache
    sig = inspect.signature(mla_decode_kvcache)
    names = list(sig.parameters)
    assert names[:8] == ["q", "kcache", "block_table", "cache_seqlens", "softmax_scale", "causal",
                         "indices", "metadata"]
    for n in ("softmax_scale", "indices", "metadata"):
        assert sig.parameters[n].default is None
    assert sig.parameters["causal"].default is False


@pytest.mark.parametrize("kw,code", [
    (dict(qk_fp8=1), -2),                                  # bf16 pool
    (dict(qk_fp8=1, kv_format=1), -2),                     # 16 query rows: the 16-row kernel
    (dict(qk_fp8=1, kv_format=1, h_q=128), 0),             # FP8, 128 rows per unit
    (dict(qk_fp8=1, kv_format=1, h_q=16, s_q=4), 0),       # 64 rows per unit
    (dict(qk_fp8=2, kv_format=1, h_q=128), -1),
])
def test_fp8_query_option_needs_fp8_pool_and_wide_units(lib, kw, code):
    n = ctypes.c_size_t()
    a = _args(**kw)
    assert lib.mla_workspace_size(ctypes.byref(a), ctypes.byref(n)) == code
    if code:
        assert b"qk_fp8" in lib.mla_last_error()


def test_bandwidth_reference_library_rejects_bad_arguments():
    # libmla_bw.so: the benchmark's read-bandwidth reference, apart from the
    # decode ABI.  Bad arguments return -1 before any HIP call.
    path = os.path.join(ROOT, "mla_paged_kv_metadata_amd", "libmla_bw.so")
    if not os.path.exists(path):
        pytest.fail("libmla_bw.so is not built (python -m mla_paged_kv_metadata_amd.build)")
    bw = ctypes.CDLL(path)
    bw.mla_bw_read.restype = ctypes.c_int
    bw.mla_bw_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    fake = ctypes.c_void_p(1 << 20)
    assert bw.mla_bw_read(None, 32768, fake, 1, None) == -1             # no source
    assert bw.mla_bw_read(fake, 32768, None, 1, None) == -1             # no sink
    assert bw.mla_bw_read(fake, 32768, fake, 0, None) == -1             # no workgroups
    assert bw.mla_bw_read(fake, 32768 + 16, fake, 1, None) == -1        # not whole 32 KiB chunks
    assert bw.mla_bw_read(ctypes.c_void_p((1 << 20) + 4), 32768, fake, 1, None) == -1   # misaligned
