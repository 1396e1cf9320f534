"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, its argument structs match the binding, and invalid arguments
return status codes before any device work (no GPU needed)."""
import ctypes
import os
import re

import pytest

from decode_attention_paged_amd import _lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mla_dcp.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from decode_attention_paged_amd import build
        build.build()
    return L.load()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert "mla_decode_partial" in names and "mla_merge_partials" in names
    assert "mla_build_shard_metadata" in names and "mla_append_kv" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(L.EXPORTS) <= set(names)


def test_struct_layouts_and_version(lib):
    assert lib.mla_sizeof_decode_args() == ctypes.sizeof(L.DecodeArgs)
    assert lib.mla_sizeof_merge_args() == ctypes.sizeof(L.MergeArgs)
    assert lib.mla_sizeof_append_args() == ctypes.sizeof(L.AppendArgs)
    assert lib.mla_abi_version() == 8
    assert lib.mla_status_string(L.STATUS_INVALID_ARGUMENT) == b"invalid argument"


def test_workspace_size_is_host_only(lib):
    n = lib.mla_decode_workspace_bytes(128, 128, 1)
    assert n > 128 * 128 * 512 * 4
    assert lib.mla_decode_workspace_bytes(4, 17, 1) == 0       # heads not a multiple of 16
    assert lib.mla_decode_workspace_bytes(4, 16, 5) == 0       # q_len > 4
    assert lib.mla_decode_workspace_bytes(4, L.MAX_HEADS, 4) > 0
    assert lib.mla_decode_workspace_bytes(4, L.MAX_HEADS + 16, 1) == 0    # more than 1024 row blocks at q_len 4
    assert lib.mla_decode_workspace_bytes(2, 16, 4) < lib.mla_decode_workspace_bytes(2, 32, 4)


def _valid_args():
    a = L.DecodeArgs()
    fake = 0x1000
    a.q = a.kv_pages = a.block_table = a.seq_lens = a.out = a.lse = a.workspace = fake
    a.batch, a.num_heads, a.q_len = 2, 16, 1
    a.max_pages, a.num_pages, a.page_size = 4, 8, 64
    a.shard_id, a.num_shards = 0, 4
    a.kv_dtype, a.out_dtype = L.DTYPE_BF16, L.DTYPE_F32
    a.kv_scale, a.softmax_scale = 1.0, 0.07
    a.lse_base = L.LSE_BASE_E
    a.workspace_bytes = 0
    return a


@pytest.mark.parametrize("field,value,status", [
    ("num_heads", 24, L.STATUS_INVALID_ARGUMENT),
    ("num_heads", 0, L.STATUS_INVALID_ARGUMENT),
    ("num_heads", L.MAX_HEADS + 16, L.STATUS_INVALID_ARGUMENT),
    ("q_len", 0, L.STATUS_INVALID_ARGUMENT),
    ("q_len", 5, L.STATUS_INVALID_ARGUMENT),
    ("page_size", 32, L.STATUS_INVALID_ARGUMENT),
    ("shard_id", 4, L.STATUS_INVALID_ARGUMENT),
    ("shard_id", -1, L.STATUS_INVALID_ARGUMENT),
    ("num_shards", 0, L.STATUS_INVALID_ARGUMENT),
    ("num_shards", 17, L.STATUS_INVALID_ARGUMENT),
    ("batch", -1, L.STATUS_INVALID_ARGUMENT),
    ("kv_dtype", L.DTYPE_F32, L.STATUS_INVALID_ARGUMENT),
    ("out_dtype", L.DTYPE_FP8_E4M3, L.STATUS_INVALID_ARGUMENT),
    ("lse", None, L.STATUS_INVALID_ARGUMENT),
    ("softmax_scale", 0.0, L.STATUS_INVALID_ARGUMENT),
    ("num_pages", 0, L.STATUS_INVALID_ARGUMENT),
    ("num_pages", 2 ** 25 + 1, L.STATUS_UNSUPPORTED),           # pool rows past int32
    ("max_pages", 2 ** 25 + 1, L.STATUS_UNSUPPORTED),           # tokens a request can hold past int32
    ("local_seq_lens", 0x2000, L.STATUS_INVALID_ARGUMENT),     # without local_kv_indices
    ("split_target", 100000, L.STATUS_INVALID_ARGUMENT),
    ("workspace_bytes", 0, L.STATUS_WORKSPACE_TOO_SMALL),
])
def test_decode_argument_errors(lib, field, value, status):
    a = _valid_args()
    setattr(a, field, value)
    st = lib.mla_decode_partial(ctypes.byref(a), None, None)
    assert st == status, lib.mla_last_error()
    assert lib.mla_last_error()


def test_schedule_size_bound(lib):
    """The schedule counts tiles in 32-bit integers: sizes whose bound (every
    request as long as its block-table row) reaches 2^31 are refused before
    any device call, and the next smaller batch gets past the check."""
    a = _valid_args()
    a.batch, a.max_pages, a.num_shards, a.shard_id = 2 ** 16, 2 ** 15, 1, 0    # 2^16 x 65536 tiles
    assert lib.mla_decode_partial(ctypes.byref(a), None, None) == L.STATUS_UNSUPPORTED
    assert b"split the batch" in lib.mla_last_error()
    a.batch = 2 ** 10
    assert lib.mla_decode_partial(ctypes.byref(a), None, None) == L.STATUS_WORKSPACE_TOO_SMALL


@pytest.mark.parametrize("fields", [
    dict(q_row_stride=100),                                 # not a multiple of 8
    dict(q_row_stride=512),                                 # below 576 without q_rope
    dict(q_row_stride=-8),
    dict(q=0x1008),                                         # not 16-byte aligned
    dict(q_rope=0x2000, q_row_stride=504),                  # below 512 with q_rope
    dict(q_rope=0x2000, q_rope_row_stride=60),              # below 64
    dict(q_rope=0x2000, q_rope_row_stride=68),              # not a multiple of 8
    dict(q_rope=0x2004),                                    # not 16-byte aligned
])
def test_split_query_argument_errors(lib, fields):
    for fn in (lib.mla_decode_partial, lib.mla_decode_all_shards):
        a = _valid_args()
        a.workspace_bytes = 1 << 40
        for k, v in fields.items():
            setattr(a, k, v)
        assert fn(ctypes.byref(a), None, None) == L.STATUS_INVALID_ARGUMENT, fields
        assert "q" in lib.mla_last_error().decode()


def test_empty_batch_is_ok_without_device(lib):
    a = _valid_args()
    a.batch = 0
    written = ctypes.c_int(-1)
    assert lib.mla_decode_partial(ctypes.byref(a), ctypes.byref(written), None) == L.STATUS_OK
    assert written.value == L.LSE_BASE_E


def test_all_shards_workspace_and_argument_errors(lib):
    # the single launch of every shard schedules B x S segments
    assert lib.mla_decode_all_shards_workspace_bytes(8, 64, 1, 4) == lib.mla_decode_workspace_bytes(32, 64, 1)
    assert lib.mla_decode_all_shards_workspace_bytes(8, 64, 1, 1) == lib.mla_decode_workspace_bytes(8, 64, 1)
    assert lib.mla_decode_all_shards_workspace_bytes(8, 64, 1, 17) == 0
    assert lib.mla_decode_all_shards_workspace_bytes(8, 64, 1, 0) == 0
    assert lib.mla_decode_all_shards_workspace_bytes(8, 17, 1, 2) == 0
    for field, value, status in [("local_seq_lens", 0x2000, L.STATUS_INVALID_ARGUMENT),
                                 ("num_shards", 17, L.STATUS_INVALID_ARGUMENT),
                                 ("q_len", 5, L.STATUS_INVALID_ARGUMENT),
                                 ("workspace_bytes", 0, L.STATUS_WORKSPACE_TOO_SMALL)]:
        a = _valid_args()
        setattr(a, field, value)
        if field == "local_seq_lens":
            a.local_kv_indices, a.local_kv_stride = 0x3000, 8
        assert lib.mla_decode_all_shards(ctypes.byref(a), None, None) == status, field
        assert lib.mla_last_error()
    # the workspace of one shard's decode is too small for all of them
    a = _valid_args()
    a.workspace_bytes = lib.mla_decode_workspace_bytes(a.batch, a.num_heads, a.q_len)
    assert lib.mla_decode_all_shards(ctypes.byref(a), None, None) == L.STATUS_WORKSPACE_TOO_SMALL
    # shard_id is ignored; an empty batch runs nothing
    a = _valid_args()
    a.batch, a.shard_id = 0, 9
    written = ctypes.c_int(-1)
    assert lib.mla_decode_all_shards(ctypes.byref(a), ctypes.byref(written), None) == L.STATUS_OK
    assert written.value == L.LSE_BASE_E


def test_metadata_argument_errors(lib):
    i32 = ctypes.c_int32
    lmax = i32(0)
    f = 0x1000
    assert lib.mla_build_shard_metadata(f, f, 2, 4, 64, 100, 4, 4, f, f, 40, ctypes.byref(lmax), None) \
        == L.STATUS_INVALID_ARGUMENT                       # shard_id == num_shards
    assert lib.mla_build_shard_metadata(f, f, 2, 4, 32, 100, 0, 4, f, f, 40, ctypes.byref(lmax), None) \
        == L.STATUS_INVALID_ARGUMENT                       # page size
    assert lib.mla_build_shard_metadata(f, f, 2, 4, 64, 100, 0, 4, f, f, 24, ctypes.byref(lmax), None) \
        == L.STATUS_INVALID_ARGUMENT                       # stride below local max 25
    assert lib.mla_build_shard_metadata(f, f, 0, 4, 64, 0, 3, 4, None, None, 0, ctypes.byref(lmax), None) \
        == L.STATUS_OK                                     # empty batch: only the host local max
    assert lmax.value == 1


def test_merge_argument_errors(lib):
    a = L.MergeArgs()
    a.num_shards, a.rows, a.num_heads, a.dv = 0, 1, 1, 512
    assert lib.mla_merge_partials(ctypes.byref(a), None) == L.STATUS_INVALID_ARGUMENT
    a.num_shards = 2
    assert lib.mla_merge_partials(ctypes.byref(a), None) == L.STATUS_INVALID_ARGUMENT   # null arrays
    outs = (ctypes.c_void_p * 2)(0x1000, None)
    lses = (ctypes.c_void_p * 2)(0x1000, 0x1000)
    bases = (ctypes.c_int * 2)(0, 1)
    a.outs, a.lses, a.bases = outs, lses, bases
    a.out = 0x1000
    assert lib.mla_merge_partials(ctypes.byref(a), None) == L.STATUS_INVALID_ARGUMENT   # null shard out
    a.dv = 500
    assert lib.mla_merge_partials(ctypes.byref(a), None) == L.STATUS_INVALID_ARGUMENT


def _valid_append():
    a = L.AppendArgs()
    a.k_nope = a.k_rope = a.seq_lens = a.block_table = a.kv_pages = 0x1000
    a.batch, a.n_new, a.max_pages, a.num_pages = 2, 1, 4, 8
    a.shard_id, a.num_shards = 1, 4
    a.kv_dtype, a.kv_scale = L.DTYPE_FP8_E4M3, 0.5
    return a


@pytest.mark.parametrize("field,value", [
    ("batch", -1), ("n_new", 0), ("n_new", 5), ("num_shards", 0), ("num_shards", 17),
    ("shard_id", 4), ("shard_id", -1), ("max_pages", 0), ("num_pages", 0),
    ("kv_dtype", L.DTYPE_F32), ("kv_scale", 0.0), ("kv_scale", -1.0), ("kv_scale", float("inf")),
    ("kv_scale", float("nan")), ("k_rope", None), ("kv_pages", None),
])
def test_append_argument_errors(lib, field, value):
    a = _valid_append()
    setattr(a, field, value)
    assert lib.mla_append_kv(ctypes.byref(a), None) == L.STATUS_INVALID_ARGUMENT
    assert lib.mla_last_error()


def test_append_empty_batch_and_bf16_scale_are_ok_without_device(lib):
    a = _valid_append()
    a.batch = 0
    assert lib.mla_append_kv(ctypes.byref(a), None) == L.STATUS_OK
    a.kv_dtype, a.kv_scale = L.DTYPE_BF16, 0.0          # the scale is not used for a bf16 pool
    assert lib.mla_append_kv(ctypes.byref(a), None) == L.STATUS_OK


@pytest.mark.parametrize("fields", [
    dict(q_scale=-1.0),                                     # negative
    dict(q_scale=float("nan")),
    dict(q_scale=float("inf")),
    dict(q_scale=0.5),                                      # e4m3 query with a bf16 pool
    dict(q_scale=0.5, kv_dtype=L.DTYPE_FP8_E4M3, q_rope=0x2000),       # codes hold all 576 dims
    dict(q_scale=0.5, kv_dtype=L.DTYPE_FP8_E4M3, q_row_stride=584),    # not a multiple of 16
    dict(q_scale=0.5, kv_dtype=L.DTYPE_FP8_E4M3, q_row_stride=560),    # below 576
    dict(q_scale=0.5, kv_dtype=L.DTYPE_FP8_E4M3, q=0x1008),            # not 16-byte aligned
])
def test_e4m3_query_argument_errors(lib, fields):
    for fn in (lib.mla_decode_partial, lib.mla_decode_all_shards):
        a = _valid_args()
        a.workspace_bytes = 1 << 40
        for k, v in fields.items():
            setattr(a, k, v)
        assert fn(ctypes.byref(a), None, None) == L.STATUS_INVALID_ARGUMENT, fields
        assert "q" in lib.mla_last_error().decode()


def test_e4m3_query_empty_batch_is_ok_without_device(lib):
    a = _valid_args()
    a.batch, a.kv_dtype, a.q_scale, a.q_row_stride = 0, L.DTYPE_FP8_E4M3, 0.25, 592
    assert lib.mla_decode_partial(ctypes.byref(a), None, None) == L.STATUS_OK


@pytest.mark.parametrize("args,ok", [
    ((0x1000, None, 0, 0, 0, 1.0, 0x2000), True),           # no rows: nothing to run
    ((0x1000, None, 0, 0, -1, 1.0, 0x2000), False),         # rows < 0
    ((0x1000, None, 0, 0, 4, 0.0, 0x2000), False),          # scale 0
    ((0x1000, None, 0, 0, 4, float("nan"), 0x2000), False),
    ((0x1000, None, 0, 0, 4, float("inf"), 0x2000), False),
    ((None, None, 0, 0, 4, 1.0, 0x2000), False),            # null q
    ((0x1000, None, 0, 0, 4, 1.0, None), False),            # null out
    ((0x1000, None, 572, 0, 4, 1.0, 0x2000), False),        # stride below 576
    ((0x1000, None, 580, 0, 4, 1.0, 0x2000), False),        # stride not a multiple of 8
    ((0x1000, 0x3000, 504, 0, 4, 1.0, 0x2000), False),      # latent stride below 512
    ((0x1000, 0x3000, 512, 60, 4, 1.0, 0x2000), False),     # rope stride below 64
    ((0x1004, None, 0, 0, 4, 1.0, 0x2000), False),          # q not 16-byte aligned
    ((0x1000, None, 0, 0, 4, 1.0, 0x2008), False),          # out not 16-byte aligned
])
def test_quantize_q_argument_errors(lib, args, ok):
    st = lib.mla_quantize_q(*args, None)
    assert (st == L.STATUS_OK) == ok, (args, lib.mla_last_error())
    if not ok:
        assert st == L.STATUS_INVALID_ARGUMENT and lib.mla_last_error()
