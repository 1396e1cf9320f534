"""ctypes binding of libmla_dcp.so (the C ABI in include/mla_dcp.h).

Argument marshalling only: every step of the decode and merge runs in the
library's HIP kernels. PyTorch supplies device memory and the current
stream; functions take torch tensors and pass ``data_ptr()`` values.

The product path never falls back to anything else: if the library is not
built, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla_dcp.so")

# enums (include/mla_dcp.h)
STATUS_OK = 0
STATUS_INVALID_ARGUMENT = 1
STATUS_UNSUPPORTED = 2
STATUS_WORKSPACE_TOO_SMALL = 3
STATUS_DEVICE_ERROR = 4
DTYPE_F32, DTYPE_BF16, DTYPE_FP8_E4M3 = 0, 1, 2
LSE_BASE_E, LSE_BASE_2 = 0, 1
PAGE_SIZE, D_QK, D_V, MAX_SHARDS, MAX_Q_LEN, MAX_HEADS = 64, 576, 512, 16, 4, 16384


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("kv_pages", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("local_seq_lens", ctypes.c_void_p),
        ("local_kv_indices", ctypes.c_void_p),
        ("local_kv_stride", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("shard_id", ctypes.c_int32),
        ("num_shards", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int),
        ("kv_scale", ctypes.c_float),
        ("softmax_scale", ctypes.c_float),
        ("lse_base", ctypes.c_int),
        ("out", ctypes.c_void_p),
        ("out_dtype", ctypes.c_int),
        ("lse", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("split_target", ctypes.c_int32),
        ("event_begin", ctypes.c_void_p),
        ("event_end", ctypes.c_void_p),
        ("reuse_plan", ctypes.c_int32),
        ("q_lens", ctypes.c_void_p),
        ("q_rope", ctypes.c_void_p),
        ("q_row_stride", ctypes.c_int64),
        ("q_rope_row_stride", ctypes.c_int64),
        ("q_scale", ctypes.c_float),
    ]


class MergeArgs(ctypes.Structure):
    _fields_ = [
        ("outs", ctypes.POINTER(ctypes.c_void_p)),
        ("lses", ctypes.POINTER(ctypes.c_void_p)),
        ("bases", ctypes.POINTER(ctypes.c_int)),
        ("num_shards", ctypes.c_int32),
        ("rows", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("dv", ctypes.c_int32),
        ("in_dtype", ctypes.c_int),
        ("out", ctypes.c_void_p),
        ("out_dtype", ctypes.c_int),
        ("lse_out", ctypes.c_void_p),
        ("lse_out_base", ctypes.c_int),
        ("event_begin", ctypes.c_void_p),
        ("event_end", ctypes.c_void_p),
    ]


class AppendArgs(ctypes.Structure):
    _fields_ = [
        ("k_nope", ctypes.c_void_p),
        ("k_rope", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("kv_pages", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("n_new", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("shard_id", ctypes.c_int32),
        ("num_shards", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int),
        ("kv_scale", ctypes.c_float),
    ]


EXPORTS = ("mla_build_shard_metadata", "mla_decode_workspace_bytes", "mla_decode_partial",
           "mla_decode_partial_noalloc", "mla_decode_plan",
           "mla_decode_all_shards", "mla_decode_all_shards_workspace_bytes", "mla_merge_partials", "mla_append_kv",
           "mla_quantize_q", "mla_status_string", "mla_last_error", "mla_abi_version",
           "mla_sizeof_decode_args", "mla_sizeof_merge_args", "mla_sizeof_append_args")

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    # PyTorch ships its own HIP runtime; loading it first makes the library
    # bind to that same runtime (one runtime per process)
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m decode_attention_paged_amd.build`")
    lib = ctypes.CDLL(path)
    i32, vp, sz = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    lib.mla_build_shard_metadata.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, i32,
                                             ctypes.POINTER(i32), vp]
    lib.mla_build_shard_metadata.restype = ctypes.c_int
    lib.mla_decode_workspace_bytes.argtypes = [i32, i32, i32]
    lib.mla_decode_workspace_bytes.restype = sz
    lib.mla_decode_partial.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.POINTER(ctypes.c_int), vp]
    lib.mla_decode_partial.restype = ctypes.c_int
    lib.mla_decode_partial_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.POINTER(ctypes.c_int), vp]
    lib.mla_decode_partial_noalloc.restype = ctypes.c_int
    lib.mla_decode_plan.argtypes = [ctypes.POINTER(DecodeArgs), vp]
    lib.mla_decode_plan.restype = ctypes.c_int
    lib.mla_decode_all_shards.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.POINTER(ctypes.c_int), vp]
    lib.mla_decode_all_shards.restype = ctypes.c_int
    lib.mla_decode_all_shards_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.mla_decode_all_shards_workspace_bytes.restype = sz
    lib.mla_merge_partials.argtypes = [ctypes.POINTER(MergeArgs), vp]
    lib.mla_merge_partials.restype = ctypes.c_int
    lib.mla_append_kv.argtypes = [ctypes.POINTER(AppendArgs), vp]
    lib.mla_append_kv.restype = ctypes.c_int
    i64 = ctypes.c_int64
    lib.mla_quantize_q.argtypes = [vp, vp, i64, i64, i64, ctypes.c_float, vp, vp]
    lib.mla_quantize_q.restype = ctypes.c_int
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_last_error.argtypes = []
    lib.mla_last_error.restype = ctypes.c_char_p
    lib.mla_abi_version.restype = i32
    lib.mla_sizeof_decode_args.restype = sz
    lib.mla_sizeof_merge_args.restype = sz
    lib.mla_sizeof_append_args.restype = sz
    if lib.mla_sizeof_decode_args() != ctypes.sizeof(DecodeArgs):
        raise RuntimeError("mla_decode_args_t layout mismatch between library and binding")
    if lib.mla_sizeof_merge_args() != ctypes.sizeof(MergeArgs):
        raise RuntimeError("mla_merge_args_t layout mismatch between library and binding")
    if lib.mla_sizeof_append_args() != ctypes.sizeof(AppendArgs):
        raise RuntimeError("mla_append_args_t layout mismatch between library and binding")
    _lib = lib
    return lib


class MlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def _check(st: int) -> None:
    if st != STATUS_OK:
        lib = load()
        raise MlaError(st, lib.mla_last_error().decode() or lib.mla_status_string(st).decode())


def _stream_ptr(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype in (torch.uint8, getattr(torch, "float8_e4m3fn", None)):
        return DTYPE_FP8_E4M3
    raise ValueError(f"unsupported dtype {t.dtype}")


# --------------------------------------------------------------------------
# entry points (same names as the C ABI)
# --------------------------------------------------------------------------
def mla_build_shard_metadata(seq_lens, block_table, max_seq_len: int, shard_id: int, num_shards: int,
                             local_seq_lens, local_kv_indices=None, stream=None) -> int:
    """Fill local_seq_lens [B] (and local_kv_indices [B, stride]); returns the local max."""
    lib = load()
    B = int(seq_lens.shape[0])
    stride = int(local_kv_indices.shape[1]) if local_kv_indices is not None else 0
    lmax = ctypes.c_int32(0)
    _check(lib.mla_build_shard_metadata(_ptr(seq_lens), _ptr(block_table), B, int(block_table.shape[1]),
                                        PAGE_SIZE, int(max_seq_len), int(shard_id), int(num_shards),
                                        _ptr(local_seq_lens), _ptr(local_kv_indices), stride,
                                        ctypes.byref(lmax), _stream_ptr(stream)))
    return int(lmax.value)


def mla_shard_local_max(max_seq_len: int, shard_id: int, num_shards: int) -> int:
    """The shard-local length bound (the local max) for a step whose longest
    request has ``max_seq_len`` tokens, from mla_build_shard_metadata with an
    empty batch (host only: nothing is enqueued and no device memory read)."""
    lib = load()
    lmax = ctypes.c_int32(0)
    _check(lib.mla_build_shard_metadata(None, None, 0, 1, PAGE_SIZE, int(max_seq_len), int(shard_id),
                                        int(num_shards), None, None, 0, ctypes.byref(lmax), None))
    return int(lmax.value)


def mla_decode_workspace_bytes(batch: int, num_heads: int, q_len: int) -> int:
    return int(load().mla_decode_workspace_bytes(int(batch), int(num_heads), int(q_len)))


def mla_decode_all_shards_workspace_bytes(batch: int, num_heads: int, q_len: int, num_shards: int) -> int:
    return int(load().mla_decode_all_shards_workspace_bytes(int(batch), int(num_heads), int(q_len),
                                                            int(num_shards)))


def _row_stride(t, dims: int, what: str) -> int:
    """Elements between consecutive query rows of a [B, q_len, H, dims] view
    whose rows are evenly spaced (the last dim contiguous)."""
    if t.dim() != 4 or int(t.shape[3]) != dims or t.stride(3) != 1:
        raise ValueError(f"{what} must be a [B, q_len, H, {dims}] view with a contiguous last dim")
    B, ql, H = int(t.shape[0]), int(t.shape[1]), int(t.shape[2])
    rs = t.stride(2)
    if (ql > 1 and t.stride(1) != H * rs) or (B > 1 and t.stride(0) != ql * H * rs):
        raise ValueError(f"{what}: query rows must be evenly spaced in (b, i, h) order")
    return int(rs)


def _decode_args(q, kv_pages, block_table, seq_lens, shard_id, num_shards, q_len, out, lse, workspace,
                 kv_scale, softmax_scale, lse_base, local_seq_lens, local_kv_indices, split_target, events,
                 reuse_plan, q_lens=None, q_rope=None, q_scale=0.0):
    import torch
    a = DecodeArgs()
    B, ql, H = int(q.shape[0]), int(q.shape[1]), int(q.shape[2])
    if ql != q_len:
        raise ValueError("q.shape[1] must equal q_len")
    if q.dtype == torch.uint8:
        # e4m3 query codes [B, q_len, H, 576] with their dequant scale
        if not q_scale > 0.0 or q_rope is not None:
            raise ValueError("an e4m3 query (uint8 codes) needs q_scale > 0 and no q_rope")
        a.q_row_stride = _row_stride(q, D_QK, "q (e4m3 codes)")
        a.q_scale = float(q_scale)
    elif q_scale != 0.0:
        raise ValueError("q_scale applies to an e4m3 query (uint8 codes) only")
    elif q_rope is None:
        a.q_row_stride = _row_stride(q, D_QK, "q")
    else:
        if tuple(q_rope.shape[:3]) != (B, ql, H):
            raise ValueError("q and q_rope must agree in [B, q_len, H]")
        a.q_row_stride = _row_stride(q, 512, "q (latent part)")
        a.q_rope_row_stride = _row_stride(q_rope, D_QK - 512, "q_rope")
        a.q_rope = _ptr(q_rope)
    a.q, a.kv_pages, a.block_table, a.seq_lens = _ptr(q), _ptr(kv_pages), _ptr(block_table), _ptr(seq_lens)
    a.local_seq_lens, a.local_kv_indices = _ptr(local_seq_lens), _ptr(local_kv_indices)
    a.local_kv_stride = int(local_kv_indices.shape[1]) if local_kv_indices is not None else 0
    a.batch, a.num_heads, a.q_len = B, H, int(q_len)
    a.max_pages, a.num_pages, a.page_size = int(block_table.shape[1]), int(kv_pages.shape[0]), PAGE_SIZE
    a.shard_id, a.num_shards = int(shard_id), int(num_shards)
    a.kv_dtype = _dtype_code(kv_pages)
    a.kv_scale, a.softmax_scale = float(kv_scale), float(softmax_scale)
    a.lse_base = int(lse_base)
    a.out, a.out_dtype, a.lse = _ptr(out), _dtype_code(out), _ptr(lse)
    if workspace is not None:
        a.workspace, a.workspace_bytes = _ptr(workspace), int(workspace.numel() * workspace.element_size())
    a.split_target = int(split_target)
    if events is not None:
        a.event_begin, a.event_end = int(events[0].cuda_event), int(events[1].cuda_event)
    a.reuse_plan = 1 if reuse_plan else 0
    a.q_lens = _ptr(q_lens)
    return a


def mla_decode_partial(q, kv_pages, block_table, seq_lens, shard_id: int, num_shards: int, q_len: int,
                       out, lse, workspace, *, kv_scale: float = 1.0, softmax_scale: float,
                       lse_base: int = LSE_BASE_E, local_seq_lens=None, local_kv_indices=None,
                       split_target: int = 0, events=None, reuse_plan: bool = False, q_lens=None,
                       q_rope=None, q_scale: float = 0.0, stream=None) -> int:
    """Rank-local (out, lse) of one shard; returns the LSE base written.

    q [B, q_len, H, 576] bf16; kv_pages [P, 64, 576] bf16 or uint8 (e4m3);
    block_table [B, max_pages] i32; seq_lens [B] i32; out [B, q_len, H, 512]
    f32 or bf16; lse [B, q_len, H] f32; workspace uint8 of at least
    mla_decode_workspace_bytes(B, H, q_len). ``events`` = optional pair of
    timing events recorded around the attention kernel. ``reuse_plan``: the
    workspace holds the schedule mla_decode_plan built for the same inputs.
    ``q_lens``: optional [B] i32 decode depth per request (rows past it are
    padding, written (0, -inf)). ``q_rope``: optional [B, q_len, H, 64] bf16
    rope part of the query; then ``q`` is the [B, q_len, H, 512] latent part
    (either may be a strided view, e.g. two slices of one buffer). A uint8
    ``q`` [B, q_len, H, 576] holds e4m3 query codes (mla_quantize_q) whose
    values are code x ``q_scale`` (fp8 KV only).
    """
    lib = load()
    a = _decode_args(q, kv_pages, block_table, seq_lens, shard_id, num_shards, q_len, out, lse, workspace,
                     kv_scale, softmax_scale, lse_base, local_seq_lens, local_kv_indices, split_target, events,
                     reuse_plan, q_lens, q_rope, q_scale)
    written = ctypes.c_int(-1)
    _check(lib.mla_decode_partial(ctypes.byref(a), ctypes.byref(written), _stream_ptr(stream)))
    return int(written.value)


def mla_decode_partial_noalloc(q, kv_pages, block_table, seq_lens, shard_id: int, num_shards: int, q_len: int,
                               out, lse, *, kv_scale: float = 1.0, softmax_scale: float,
                               lse_base: int = LSE_BASE_E, local_seq_lens=None, local_kv_indices=None,
                               split_target: int = 0, events=None, q_lens=None, q_rope=None,
                               q_scale: float = 0.0, stream=None) -> int:
    """mla_decode_partial without a workspace: the library's own device
    scratch holds the schedule and partials (calls on one device must not
    overlap). Returns the LSE base written."""
    lib = load()
    a = _decode_args(q, kv_pages, block_table, seq_lens, shard_id, num_shards, q_len, out, lse, None,
                     kv_scale, softmax_scale, lse_base, local_seq_lens, local_kv_indices, split_target, events,
                     False, q_lens, q_rope, q_scale)
    written = ctypes.c_int(-1)
    _check(lib.mla_decode_partial_noalloc(ctypes.byref(a), ctypes.byref(written), _stream_ptr(stream)))
    return int(written.value)


def mla_decode_all_shards(q, kv_pages, block_table, seq_lens, num_shards: int, q_len: int, out, lse, workspace,
                          *, kv_scale: float = 1.0, softmax_scale: float, lse_base: int = LSE_BASE_E,
                          split_target: int = 0, events=None, reuse_plan: bool = False, q_lens=None,
                          q_rope=None, q_scale: float = 0.0, stream=None) -> int:
    """Every shard of the cyclic split in one launch, merged: out / lse get
    the full-context result. Shapes as mla_decode_partial; workspace of at
    least mla_decode_all_shards_workspace_bytes(B, H, q_len, num_shards).
    ``reuse_plan``: the workspace holds the schedule an earlier call built
    for the same inputs. ``q_rope``: as for mla_decode_partial. Returns the
    LSE base written."""
    lib = load()
    a = _decode_args(q, kv_pages, block_table, seq_lens, 0, num_shards, q_len, out, lse, workspace,
                     kv_scale, softmax_scale, lse_base, None, None, split_target, events, reuse_plan, q_lens,
                     q_rope, q_scale)
    written = ctypes.c_int(-1)
    _check(lib.mla_decode_all_shards(ctypes.byref(a), ctypes.byref(written), _stream_ptr(stream)))
    return int(written.value)


def mla_decode_plan(q, kv_pages, block_table, seq_lens, shard_id: int, num_shards: int, q_len: int,
                    out, lse, workspace, *, kv_scale: float = 1.0, softmax_scale: float,
                    lse_base: int = LSE_BASE_E, local_seq_lens=None, local_kv_indices=None,
                    split_target: int = 0, q_scale: float = 0.0, stream=None) -> None:
    """The work schedule of mla_decode_partial with the same arguments, into
    ``workspace`` (built once per decode step, reused with reuse_plan)."""
    lib = load()
    a = _decode_args(q, kv_pages, block_table, seq_lens, shard_id, num_shards, q_len, out, lse, workspace,
                     kv_scale, softmax_scale, lse_base, local_seq_lens, local_kv_indices, split_target, None,
                     False, q_scale=q_scale)
    _check(lib.mla_decode_plan(ctypes.byref(a), _stream_ptr(stream)))


def mla_merge_partials(outs: Sequence, lses: Sequence, bases: Sequence[int], out, lse_out=None,
                       lse_out_base: int = LSE_BASE_E, stream=None, events=None) -> None:
    """LSE-weighted merge of S partials: outs[r] [N, H, Dv], lses[r] [N, H] f32.

    ``events``: optional pair of timing events that receive the merge
    kernel's dispatch start and end."""
    lib = load()
    S = len(outs)
    a = MergeArgs()
    out_ptrs = (ctypes.c_void_p * S)(*[_ptr(o) for o in outs])
    lse_ptrs = (ctypes.c_void_p * S)(*[_ptr(l) for l in lses])
    base_arr = (ctypes.c_int * S)(*[int(b) for b in bases])
    a.outs, a.lses, a.bases = out_ptrs, lse_ptrs, base_arr
    a.num_shards = S
    a.rows, a.num_heads, a.dv = int(out.shape[0]), int(out.shape[1]), int(out.shape[2])
    a.in_dtype = _dtype_code(outs[0])
    a.out, a.out_dtype = _ptr(out), _dtype_code(out)
    a.lse_out, a.lse_out_base = _ptr(lse_out), int(lse_out_base)
    if events is not None:
        a.event_begin, a.event_end = int(events[0].cuda_event), int(events[1].cuda_event)
    _check(lib.mla_merge_partials(ctypes.byref(a), _stream_ptr(stream)))


def mla_quantize_q(q, out, q_scale: float, q_rope=None, stream=None) -> None:
    """e4m3 codes of a bf16 query into ``out`` [B, q_len, H, 576] uint8
    (contiguous): the nearest e4m3 value to q / q_scale, ties to even,
    saturating. ``q`` [B, q_len, H, 576] bf16, or its [.., 512] latent part
    with ``q_rope`` [.., 64] (strided views allowed, as for the decode)."""
    lib = load()
    if out.dim() != 4 or int(out.shape[3]) != D_QK or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, q_len, H, 576] uint8 tensor")
    rows = int(out.shape[0]) * int(out.shape[1]) * int(out.shape[2])
    if q_rope is None:
        qs, rs = _row_stride(q, D_QK, "q"), 0
    else:
        qs, rs = _row_stride(q, 512, "q (latent part)"), _row_stride(q_rope, D_QK - 512, "q_rope")
    if tuple(q.shape[:3]) != tuple(out.shape[:3]):
        raise ValueError("q and out must agree in [B, q_len, H]")
    _check(lib.mla_quantize_q(_ptr(q), _ptr(q_rope), qs, rs, rows, float(q_scale), _ptr(out), _stream_ptr(stream)))


def mla_append_kv(k_nope, k_rope, seq_lens, block_table, kv_pages, shard_id: int, num_shards: int, *,
                  kv_scale: float = 1.0, stream=None) -> None:
    """Write the newest n_new tokens of each request into the pool, on the
    shard that owns each token (token L - n_new + i belongs to shard
    (L - n_new + i) mod S); fp8 pools get the row quantised with kv_scale.

    k_nope [B, n_new, 512] bf16; k_rope [B, n_new, 64] bf16; seq_lens [B] i32
    (new global lengths); block_table [B, max_pages] i32; kv_pages
    [P, 64, 576] bf16 or uint8 (e4m3), written in place.
    """
    lib = load()
    if k_nope.dim() != 3 or k_nope.shape[2] != 512 or k_rope.dim() != 3 or k_rope.shape[2] != 64:
        raise ValueError("k_nope must be [B, n_new, 512] and k_rope [B, n_new, 64]")
    if tuple(k_nope.shape[:2]) != tuple(k_rope.shape[:2]):
        raise ValueError("k_nope and k_rope must agree in [B, n_new]")
    if not (k_nope.is_contiguous() and k_rope.is_contiguous()):
        raise ValueError("k_nope and k_rope must be contiguous")
    a = AppendArgs()
    a.k_nope, a.k_rope = _ptr(k_nope), _ptr(k_rope)
    a.seq_lens, a.block_table, a.kv_pages = _ptr(seq_lens), _ptr(block_table), _ptr(kv_pages)
    a.batch, a.n_new = int(k_nope.shape[0]), int(k_nope.shape[1])
    a.max_pages, a.num_pages = int(block_table.shape[1]), int(kv_pages.shape[0])
    a.shard_id, a.num_shards = int(shard_id), int(num_shards)
    a.kv_dtype = _dtype_code(kv_pages)
    a.kv_scale = float(kv_scale)
    _check(lib.mla_append_kv(ctypes.byref(a), _stream_ptr(stream)))
