"""One sharded decode step on the GPU through the C ABI.

A step is: for every shard r, the rank-local partial decode (out_r, lse_r)
over the tokens the shard owns, then the LSE-weighted merge of the S
partials into the full-context result. PyTorch only allocates device
memory; all arithmetic runs in the library's kernels.

The partials read their KV rows through the block table by default
(``use_metadata=False``): the kernel applies the cyclic owner rule itself
and one table entry serves 64 tokens, shared through L2, where the
shard-local KV indices (``use_metadata=True``, built by run_metadata) cost
a private table line per tile that misses to HBM — measured 3-7% slower per
attention launch and 1.5-4% per step on the named workloads. Both gathers
give the same rows and are parity-tested.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

from . import _lib as L


@dataclasses.dataclass
class DeviceWorkload:
    """Device copies of a workload's input bytes (and the scalars to use them)."""
    batch: int
    heads: int
    q_len: int
    shards: int
    kv_fp8: bool
    kv_scale: float
    softmax_scale: float
    lse_base: int
    out_bf16: bool
    max_seq_len: int
    q: torch.Tensor            # [B, q_len, H, 576] bf16
    kv_pages: torch.Tensor     # [P, 64, 576] bf16 | uint8
    block_table: torch.Tensor  # [B, max_pages] i32
    seq_lens: torch.Tensor     # [B] i32
    q_lens: Optional[torch.Tensor] = None   # [B] i32 decode depth per request, or None
    # e4m3 query codes [B, q_len, H, 576] and their scale (fp8 KV only): the
    # decode reads these instead of the bf16 query when q_scale > 0
    q8: Optional[torch.Tensor] = None
    q_scale: float = 0.0

    @staticmethod
    def upload(wl, device="cuda", out_dtype: Optional[str] = None) -> "DeviceWorkload":
        q = torch.from_numpy(np.ascontiguousarray(wl.q)).view(torch.bfloat16).to(device)
        if wl.kv_dtype == "bf16":
            kv = torch.from_numpy(np.ascontiguousarray(wl.kv_pages)).view(torch.bfloat16).to(device)
        else:
            kv = torch.from_numpy(np.ascontiguousarray(wl.kv_pages)).to(device)
        return DeviceWorkload(
            batch=wl.batch, heads=wl.heads, q_len=wl.q_len, shards=wl.shards,
            kv_fp8=wl.kv_dtype == "fp8", kv_scale=wl.kv_scale, softmax_scale=wl.softmax_scale,
            lse_base=L.LSE_BASE_2 if wl.lse_base == "2" else L.LSE_BASE_E,
            out_bf16=(out_dtype or wl.out_dtype) == "bf16", max_seq_len=wl.max_seq_len,
            q=q, kv_pages=kv,
            block_table=torch.from_numpy(np.ascontiguousarray(wl.block_table)).to(device),
            seq_lens=torch.from_numpy(np.ascontiguousarray(wl.seq_lens)).to(device),
            q_lens=(torch.from_numpy(np.ascontiguousarray(wl.q_lens)).to(device)
                    if getattr(wl, "q_lens", None) is not None else None),
            q8=(torch.from_numpy(np.ascontiguousarray(wl.q_codes)).to(device)
                if getattr(wl, "q_codes", None) is not None else None),
            q_scale=float(getattr(wl, "q_scale", 0.0)) if getattr(wl, "q_codes", None) is not None else 0.0)

    def quantize_query(self, q_scale: float, stream=None) -> None:
        """The e4m3 codes of the bf16 query on device (the concat-and-quantise
        prep of the fp8 KV path); later decode calls read them."""
        if self.q8 is None:
            self.q8 = torch.empty(self.q.shape, dtype=torch.uint8, device=self.q.device)
        L.mla_quantize_q(self.q, self.q8, q_scale, stream=stream)
        self.q_scale = float(q_scale)

    def query(self):
        """(query tensor, q_scale) the decode calls pass."""
        return (self.q8, self.q_scale) if self.q_scale > 0 else (self.q, 0.0)

    def local_max(self, shard: int) -> int:
        return L.mla_shard_local_max(self.max_seq_len, shard, self.shards)


class StepBuffers:
    """Outputs, metadata and workspace of one step, allocated once."""

    def __init__(self, dw: DeviceWorkload, merged_out_bf16: Optional[bool] = None):
        dev = dw.q.device
        B, q, H, S = dw.batch, dw.q_len, dw.heads, dw.shards
        odt = torch.bfloat16 if dw.out_bf16 else torch.float32
        self.outs = [torch.empty((B, q, H, L.D_V), dtype=odt, device=dev) for _ in range(S)]
        self.lses = [torch.empty((B, q, H), dtype=torch.float32, device=dev) for _ in range(S)]
        mdt = odt if merged_out_bf16 is None else (torch.bfloat16 if merged_out_bf16 else torch.float32)
        self.out = torch.empty((B, q, H, L.D_V), dtype=mdt, device=dev)
        self.lse = torch.empty((B, q, H), dtype=torch.float32, device=dev)
        self.local_seq_lens = [torch.empty((B,), dtype=torch.int32, device=dev) for _ in range(S)]
        self.local_kv_indices = [torch.empty((B, dw.local_max(r)), dtype=torch.int32, device=dev)
                                 for r in range(S)]
        nbytes = L.mla_decode_workspace_bytes(B, H, q)
        self.workspace = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=dev)
        self._nbytes = max(nbytes, 1)
        self.workspaces = [self.workspace]

    def per_shard_workspaces(self) -> None:
        """One workspace per shard, so that shard partials may run concurrently."""
        dev = self.workspace.device
        while len(self.workspaces) < len(self.outs):
            self.workspaces.append(torch.empty((self._nbytes,), dtype=torch.uint8, device=dev))

    def fill_nan(self) -> None:
        for t in self.outs + self.lses + [self.out, self.lse]:
            t.fill_(float("nan"))


def run_metadata(dw: DeviceWorkload, bufs: StepBuffers, shard: int, stream=None) -> int:
    return L.mla_build_shard_metadata(dw.seq_lens, dw.block_table, dw.max_seq_len, shard, dw.shards,
                                      bufs.local_seq_lens[shard], bufs.local_kv_indices[shard],
                                      stream=stream)


def _workspace(bufs: StepBuffers, shard: int):
    return bufs.workspaces[shard] if shard < len(bufs.workspaces) else bufs.workspace


def run_plan(dw: DeviceWorkload, bufs: StepBuffers, shard: int, use_metadata: bool = False,
             split_target: int = 0, stream=None) -> None:
    """The shard's work schedule into its workspace (once per decode step)."""
    q, q_scale = dw.query()
    L.mla_decode_plan(
        q, dw.kv_pages, dw.block_table, dw.seq_lens, shard, dw.shards, dw.q_len,
        bufs.outs[shard], bufs.lses[shard], _workspace(bufs, shard), kv_scale=dw.kv_scale,
        softmax_scale=dw.softmax_scale, lse_base=dw.lse_base,
        local_seq_lens=bufs.local_seq_lens[shard] if use_metadata else None,
        local_kv_indices=bufs.local_kv_indices[shard] if use_metadata else None,
        split_target=split_target, q_scale=q_scale, stream=stream)


def run_partial(dw: DeviceWorkload, bufs: StepBuffers, shard: int, use_metadata: bool = False,
                split_target: int = 0, events=None, reuse_plan: bool = False, stream=None) -> int:
    q, q_scale = dw.query()
    return L.mla_decode_partial(
        q, dw.kv_pages, dw.block_table, dw.seq_lens, shard, dw.shards, dw.q_len,
        bufs.outs[shard], bufs.lses[shard], _workspace(bufs, shard), kv_scale=dw.kv_scale,
        softmax_scale=dw.softmax_scale, lse_base=dw.lse_base,
        local_seq_lens=bufs.local_seq_lens[shard] if use_metadata else None,
        local_kv_indices=bufs.local_kv_indices[shard] if use_metadata else None,
        split_target=split_target, events=events, reuse_plan=reuse_plan, q_lens=dw.q_lens, q_scale=q_scale,
        stream=stream)


def run_merge(dw: DeviceWorkload, bufs: StepBuffers, out_base: int = L.LSE_BASE_E, stream=None,
              events=None) -> None:
    N = dw.batch * dw.q_len
    outs = [o.view(N, dw.heads, L.D_V) for o in bufs.outs]
    lses = [l.view(N, dw.heads) for l in bufs.lses]
    L.mla_merge_partials(outs, lses, [dw.lse_base] * dw.shards, bufs.out.view(N, dw.heads, L.D_V),
                         bufs.lse.view(N, dw.heads), lse_out_base=out_base, stream=stream, events=events)


def run_step(dw: DeviceWorkload, bufs: StepBuffers, use_metadata: bool = False, split_target: int = 0,
             out_base: int = L.LSE_BASE_E, stream=None) -> None:
    """Metadata, partial decode of every shard, then the merge."""
    for r in range(dw.shards):
        if use_metadata:
            run_metadata(dw, bufs, r, stream=stream)
        run_partial(dw, bufs, r, use_metadata=use_metadata, split_target=split_target, stream=stream)
    run_merge(dw, bufs, out_base=out_base, stream=stream)


def run_step_concurrent(dw: DeviceWorkload, bufs: StepBuffers, streams, use_metadata: bool = False,
                        out_base: int = L.LSE_BASE_E, reuse_plan: bool = False) -> None:
    """Partials of all shards on their own streams (one workspace each), joined
    on the current stream, then the merge. Capturable as one HIP graph.
    ``reuse_plan``: every shard's workspace holds its schedule (run_plan)."""
    import torch
    bufs.per_shard_workspaces()
    cur = torch.cuda.current_stream()
    for r in range(dw.shards):
        s = streams[r]
        s.wait_stream(cur)
        with torch.cuda.stream(s):
            run_partial(dw, bufs, r, use_metadata=use_metadata, reuse_plan=reuse_plan, stream=s)
    for r in range(dw.shards):
        cur.wait_stream(streams[r])
    run_merge(dw, bufs, out_base=out_base, stream=cur)


def all_shards_workspace(dw: DeviceWorkload, bufs: StepBuffers):
    """Workspace of the single-launch decode of every shard (allocated once)."""
    import torch
    if getattr(bufs, "all_workspace", None) is None:
        n = L.mla_decode_all_shards_workspace_bytes(dw.batch, dw.heads, dw.q_len, dw.shards)
        bufs.all_workspace = torch.empty((max(n, 1),), dtype=torch.uint8, device=dw.q.device)
    return bufs.all_workspace


def run_all_shards(dw: DeviceWorkload, bufs: StepBuffers, out_base: int = L.LSE_BASE_E, split_target: int = 0,
                   events=None, reuse_plan: bool = False, stream=None) -> int:
    """Every shard in one launch with the merge fused, into bufs.out / bufs.lse."""
    ws = all_shards_workspace(dw, bufs)
    q, q_scale = dw.query()
    return L.mla_decode_all_shards(q, dw.kv_pages, dw.block_table, dw.seq_lens, dw.shards, dw.q_len,
                                   bufs.out, bufs.lse, ws, kv_scale=dw.kv_scale, softmax_scale=dw.softmax_scale,
                                   lse_base=out_base, split_target=split_target, events=events,
                                   reuse_plan=reuse_plan, q_lens=dw.q_lens, q_scale=q_scale, stream=stream)
