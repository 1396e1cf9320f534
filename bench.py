#!/usr/bin/env python3
"""Benchmark: sharded paged-MLA decode step + LSE merge on one MI355X.

A step is one pass of the whole path over one batch: for each of the S
shards the rank-local partial decode, then the LSE-weighted merge of the S
partials. Each shard's work schedule (mla_decode_plan) is built once per
decode step (not per layer) and timed separately (plan_us_per_shard in the
details); every partial of the step reuses it and reads KV rows through the
block table. The shard-local metadata (local lengths and KV indices, an
alternative gather the library also takes) is timed on its own too
(metadata_us_per_shard); the step does not use it. Inputs are synthetic (seeded, shaped
like the pages' workloads) and already resident in HBM when timing starts;
two copies of the KV pool and queries are alternated so the 256 MB
Infinity Cache cannot serve repeated reads.

Default: the Kimi-K2.5-like workload (batch 64, 64 heads, q_len 1, 4 shards,
bf16 KV, lengths uniform in [4096, 8192]) is the headline (`value`,
`roofline`); the other four workloads (tiny; DeepSeek-like fp8, 8 shards;
MTP q_len 4; skewed lengths, 8 shards, base-2 LSE) are measured the same way
and reported per workload under `configs`; plus the merge-only sweep (4
partials of T x 64 heads x 512 bf16 + fp32 LSE, T in 1..128). Prints ONE JSON
line on stdout. ``--configs`` narrows the per-workload list (e.g. for a
profiler run of one workload).

Reported:
  value         KV-GB/s of the step = bytes of every visible token's latent
                row read once / step time;
  tflops        2 * rows * (576 + 512) flops per visible (row, token) / time;
  roofline      the attention kernel alone, timed with HIP events recorded by
                the library around its launch: algorithmic bytes per launch
                (the shard's KV rows + Q + partial out + LSE) / mean duration,
                against 8 TB/s;
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload;
  hbm_measured  on-box HBM references from library kernels (a 1 GiB device
                copy and a 1 GiB read), against the larger of which the
                HBM-bound kernels' fractions are also given.

The fp8-KV workload is also timed with its query quantised to e4m3 codes
(mla_quantize_q, then the decode reads the codes): `e4m3_query` under its
entry in `configs`, beside the bf16-query figures, which stay its main ones.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "MLA split-KV decode KV-GB/s + TFLOP/s vs roofline; merge μs (64 heads, D=512)"
KERNEL_SRC_DIR = os.path.join(ROOT, "decode_attention_paged_amd", "csrc")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


class HipEvent:
    """A hipEvent_t created through the HIP runtime (timing enabled), so the
    library can record it around one kernel launch on the caller's stream."""
    _hip = None

    @classmethod
    def _rt(cls):
        if cls._hip is None:
            import ctypes
            import torch  # noqa: F401  (loads the HIP runtime)
            cls._hip = ctypes.CDLL("libamdhip64.so")
        return cls._hip

    def __init__(self):
        import ctypes
        self.handle = ctypes.c_void_p()
        if self._rt().hipEventCreate(ctypes.byref(self.handle)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.cuda_event = self.handle.value

    def elapsed_ms(self, end: "HipEvent") -> float:
        import ctypes
        ms = ctypes.c_float()
        err = self._rt().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if err != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({err})")
        return float(ms.value)

    def __del__(self):
        try:
            self._rt().hipEventDestroy(self.handle)
        except Exception:
            pass


# --------------------------------------------------------------------------
# algorithmic work of a workload
# --------------------------------------------------------------------------
def workload_work(wl):
    import numpy as np
    row_bytes = 576 * (1 if wl.kv_dtype == "fp8" else 2)
    lens = wl.seq_lens.astype(np.int64)
    kv_bytes = int(lens.sum()) * row_bytes
    q = wl.q_len
    vis = (q * lens - q * (q - 1) // 2).clip(min=0)        # sum over draft rows of visible tokens
    flops = 2.0 * wl.heads * (576 + 512) * float(vis.sum())
    out_elt = 2 if wl.out_dtype == "bf16" else 4
    per_shard = []
    for r in range(wl.shards):
        loc = lens // wl.shards + (r < lens % wl.shards)
        rows = wl.batch * q * wl.heads
        b = int(loc.sum()) * row_bytes + rows * 576 * 2 + rows * 512 * out_elt + rows * 4
        locvis = 0
        for i in range(q):
            Lv = (lens - q + i + 1).clip(min=0)
            locvis += int((Lv // wl.shards + (r < Lv % wl.shards)).sum())
        per_shard.append((b, 2.0 * wl.heads * (576 + 512) * locvis))
    return kv_bytes, flops, per_shard


# the attention kernel's translation unit and the headers it includes: the
# committed counter summary applies while these are unchanged
KERNEL_SOURCES = ("mla_device.h", "mla_internal.h", "mla_stream.hip")


def kernel_sha() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(KERNEL_SRC_DIR, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per attention-kernel launch from the committed counter summary
    (null unless it was taken on the current kernel sources)."""
    path = os.path.join(ROOT, "profiles", f"attn_kernel_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_sources_sha256_16") != kernel_sha():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# --------------------------------------------------------------------------
# GPU timing
# --------------------------------------------------------------------------
def bench_workload(index: int, steps: int, warmup: int, rotate: bool = True, split_target: int = 0,
                   use_graph: bool = True):
    import torch

    from decode_attention_paged_amd import step as ST
    from workloads import make_config

    log(f"[bench] config {index}: generating inputs")
    wl = make_config(index)
    kv_bytes, flops, per_shard = workload_work(wl)
    dws = [ST.DeviceWorkload.upload(wl)]
    if rotate and kv_bytes < 600e6:
        d0 = dws[0]
        import dataclasses
        dws.append(dataclasses.replace(d0, q=d0.q.clone(), kv_pages=d0.kv_pages.clone()))
    bufs = ST.StepBuffers(dws[0])
    S = wl.shards
    ev = [[(HipEvent(), HipEvent()) for _ in range(S)] for _ in range(steps)]
    mev = [(HipEvent(), HipEvent()) for _ in range(steps)]      # the merge kernel's own dispatch

    # shard-local metadata (built once per decode step, not per layer) is
    # timed on its own; the step below reads KV rows through the block table
    # (the step driver's default), so it does not depend on it
    mdev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(S)]
    for r in range(S):
        ST.run_metadata(dws[0], bufs, r)
    torch.cuda.synchronize()
    for r in range(S):
        mdev[r][0].record()
        ST.run_metadata(dws[0], bufs, r)
        mdev[r][1].record()
    torch.cuda.synchronize()
    metadata_us = statistics.median(1e3 * a.elapsed_time(b) for a, b in mdev)
    # so is each shard's work schedule (one per workspace, reused by every
    # layer's partial decode): built and timed here, reused by the steps
    bufs.per_shard_workspaces()
    for r in range(S):
        ST.run_plan(dws[0], bufs, r, split_target=split_target)
    torch.cuda.synchronize()
    for r in range(S):
        mdev[r][0].record()
        ST.run_plan(dws[0], bufs, r, split_target=split_target)
        mdev[r][1].record()
    torch.cuda.synchronize()
    plan_us = statistics.median(1e3 * a.elapsed_time(b) for a, b in mdev)

    def one_step(k, timed):
        dw = dws[k % len(dws)]
        for r in range(S):
            ST.run_partial(dw, bufs, r, split_target=split_target, events=ev[k][r] if timed else None,
                           reuse_plan=True)
        ST.run_merge(dw, bufs, events=mev[k] if timed else None)

    # kernel timing: eager steps, the attention kernel bracketed by events
    # that take its own dispatch start and end
    log(f"[bench] config {index}: warmup {warmup}")
    for k in range(warmup):
        one_step(k, False)
    torch.cuda.synchronize()
    log(f"[bench] config {index}: kernel timing over {steps} eager steps")
    t0 = time.perf_counter()
    for k in range(steps):
        one_step(k, True)
    torch.cuda.synchronize()
    eager_ms_step = 1e3 * (time.perf_counter() - t0) / steps

    # step timing: the step (every shard's partial on a stream of its own,
    # joined for the merge) captured as one HIP graph per input set and
    # replayed; checked bit for bit against the eager step first
    step_timing = "graph replay, shard partials on concurrent streams"
    ms_step = None
    if split_target == 0 and use_graph:
        try:
            streams = [torch.cuda.Stream() for _ in range(S)]
            graphs = []
            for dw in dws:
                ST.run_step_concurrent(dw, bufs, streams, reuse_plan=True)   # warm the path before capture
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    ST.run_step_concurrent(dw, bufs, streams, reuse_plan=True)
                graphs.append(g)
            torch.cuda.synchronize()
            for i, dw in enumerate(dws):
                bufs.fill_nan()
                for r in range(S):
                    ST.run_partial(dw, bufs, r, reuse_plan=True)
                ST.run_merge(dw, bufs)
                torch.cuda.synchronize()
                ref_out, ref_lse = bufs.out.clone(), bufs.lse.clone()
                for _ in range(2):
                    bufs.fill_nan()
                    graphs[i].replay()
                    torch.cuda.synchronize()
                    if not (torch.equal(bufs.out.view(torch.uint8), ref_out.view(torch.uint8))
                            and torch.equal(bufs.lse.view(torch.uint8), ref_lse.view(torch.uint8))):
                        raise RuntimeError("graph replay differs from the eager step")
            for k in range(warmup):
                graphs[k % len(graphs)].replay()
            torch.cuda.synchronize()
            log(f"[bench] config {index}: timing {steps} steps (graph replay)")
            t0 = time.perf_counter()
            for k in range(steps):
                graphs[k % len(graphs)].replay()
            torch.cuda.synchronize()
            ms_step = 1e3 * (time.perf_counter() - t0) / steps
            del graphs
        except Exception as e:  # noqa: BLE001 - fall back to the eager step time
            log(f"[bench] config {index}: graph step unavailable ({e}); eager step time reported")
            ms_step = None
    if ms_step is None:
        ms_step = eager_ms_step
        step_timing = "eager launches"
    attn_ms = [[ev[k][r][0].elapsed_ms(ev[k][r][1]) for r in range(S)] for k in range(steps)]
    merge_ms = [mev[k][0].elapsed_ms(mev[k][1]) for k in range(steps)]
    # merge bytes: every shard's partial (out + f32 LSE) read, the merged out
    # and its LSE written
    n_vec = wl.batch * wl.q_len * wl.heads
    part_b = 2 if wl.out_dtype == "bf16" else 4
    merge_bytes = S * n_vec * (512 * part_b + 4) + n_vec * (512 * part_b + 4)
    tot_bytes = sum(b for b, _ in per_shard)
    tot_flops = sum(f for _, f in per_shard)
    attn_total_ms = statistics.mean(sum(row) for row in attn_ms)
    mean_launch_ms = attn_total_ms / S
    achieved_gbs = tot_bytes / (attn_total_ms * 1e-3) / 1e9
    achieved_tflops = tot_flops / (attn_total_ms * 1e-3) / 1e12
    res = dict(
        index=index, name=wl.name, batch=wl.batch, heads=wl.heads, q_len=wl.q_len, shards=S,
        kv_dtype=wl.kv_dtype, lse_base=wl.lse_base, tokens=int(wl.seq_lens.sum()),
        ms_per_step=ms_step, kv_gbs=kv_bytes / (ms_step * 1e-3) / 1e9,
        tflops=flops / (ms_step * 1e-3) / 1e12,
        attn_kernel_mean_us=1e3 * mean_launch_ms, attn_kernel_bytes_per_launch=tot_bytes / S,
        attn_kernel_gbs=achieved_gbs, attn_kernel_tflops=achieved_tflops,
        merge_us=1e3 * statistics.median(merge_ms), merge_bytes=merge_bytes,
        merge_gbs=merge_bytes / (statistics.median(merge_ms) * 1e-3) / 1e9,
        merge_hbm_frac=merge_bytes / (statistics.median(merge_ms) * 1e-3) / 1e9 / HBM_PEAK_GBS,
        steps=steps, warmup=warmup, rotated=len(dws),
        metadata_us_per_shard=metadata_us, plan_us_per_shard=plan_us, step_timing=step_timing,
        eager_ms_per_step=eager_ms_step,
    )
    if split_target == 0:
        res["all_shards"] = bench_all_shards(wl, dws, bufs, steps, warmup, kv_bytes, flops, use_graph)
        if wl.kv_dtype == "fp8":
            res["e4m3_query"] = bench_e4m3_query(wl, dws, bufs, steps, warmup, kv_bytes, per_shard, use_graph)
    # the contraction runs on bf16 MFMAs for both KV types (fp8 pages are
    # converted to bf16 exactly, in registers), so its peak is the bf16 one
    peak_tf = BF16_PEAK_TFLOPS
    res["attn_kernel_hbm_frac"] = achieved_gbs / HBM_PEAK_GBS
    res["attn_kernel_mfma_frac"] = achieved_tflops / peak_tf
    del dws, bufs
    torch.cuda.empty_cache()
    return wl, res


def bench_all_shards(wl, dws, bufs, steps: int, warmup: int, kv_bytes: int, flops: float,
                     use_graph: bool = True):
    """The same step as one call: every shard in one launch, the merge fused
    into the piece combine (mla_decode_all_shards). Its schedule is built
    once per decode step and reused; the call is captured as a HIP graph per
    input set, checked bit for bit against the eager call and against the
    separate step's merged output (within the KV type's tolerance plus one
    ulp of the output type), then
    replayed for the step time (use_graph False: timed as eager calls). The
    attention kernel is timed on its own dispatch in eager calls."""
    import torch

    from decode_attention_paged_amd import step as ST

    tol = 6e-2 if wl.kv_dtype == "fp8" else 2e-2
    sep_out, sep_lse = bufs.out.clone(), bufs.lse.clone()     # the separate step's last result
    log(f"[bench] {wl.name}: single-launch step of all shards")
    ST.run_all_shards(dws[0], bufs)                              # builds the schedule
    torch.cuda.synchronize()
    a, b = bufs.out.float(), sep_out.float()
    diff = (a - b).abs()
    d_out = diff.max().item()
    # both results are rounded to the output type: two values within the
    # tolerance of the exact one may round one bf16 ulp apart
    if bufs.out.dtype == torch.bfloat16:
        mag = torch.maximum(a.abs(), b.abs())
        ulp = torch.where(mag > 0, torch.exp2(torch.floor(torch.log2(mag)) - 7), torch.zeros_like(mag))
        out_ok = bool((diff <= tol + ulp).all())
    else:
        out_ok = d_out <= tol
    fin = torch.isfinite(sep_lse)
    d_lse = (bufs.lse[fin] - sep_lse[fin]).abs().max().item() if bool(fin.any()) else 0.0
    if not (out_ok and d_lse <= tol and torch.equal(torch.isfinite(bufs.lse), fin)):
        raise RuntimeError(f"single-launch step differs from the separate step ({d_out}, {d_lse})")
    aev = [(HipEvent(), HipEvent()) for _ in range(steps)]
    for k in range(warmup):
        ST.run_all_shards(dws[k % len(dws)], bufs, reuse_plan=True)
    t0 = time.perf_counter()
    for k in range(steps):
        ST.run_all_shards(dws[k % len(dws)], bufs, reuse_plan=True, events=aev[k])
    torch.cuda.synchronize()
    eager_ms = 1e3 * (time.perf_counter() - t0) / steps
    attn_ms = statistics.mean(a.elapsed_ms(b) for a, b in aev)
    if not use_graph:
        return _all_shards_result(wl, kv_bytes, flops, eager_ms, attn_ms, d_out, d_lse, "eager calls")
    graphs = []
    for dw in dws:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            ST.run_all_shards(dw, bufs, reuse_plan=True)
        graphs.append(g)
    torch.cuda.synchronize()
    for i, dw in enumerate(dws):
        ST.run_all_shards(dw, bufs, reuse_plan=True)
        torch.cuda.synchronize()
        ref_out, ref_lse = bufs.out.clone(), bufs.lse.clone()
        bufs.fill_nan()
        graphs[i].replay()
        torch.cuda.synchronize()
        if not (torch.equal(bufs.out.view(torch.uint8), ref_out.view(torch.uint8))
                and torch.equal(bufs.lse.view(torch.uint8), ref_lse.view(torch.uint8))):
            raise RuntimeError("graph replay of the single-launch step differs from the eager call")
    for k in range(warmup):
        graphs[k % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        graphs[k % len(graphs)].replay()
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / steps
    del graphs
    return _all_shards_result(wl, kv_bytes, flops, ms, attn_ms, d_out, d_lse, "graph replay")


QUANT_REPEAT = 8


def bench_e4m3_query(wl, dws, bufs, steps: int, warmup: int, kv_bytes: int, per_shard, use_graph: bool = True):
    """The fp8-KV step with the query quantised too: mla_quantize_q turns the
    bf16 query into e4m3 codes (q_scale = max |q| / 448, one per step), then
    every shard's partial decode reads the codes (scores on the fp8 matrix
    cores) and the merge follows. Timed: the attention kernel per shard (HIP
    events around its launch), the quantise kernel (events around it, queued
    behind an attention launch so the host's launch latency falls outside,
    QUANT_REPEAT launches back to back per pair of events, so the figure is
    a launch's share of a back-to-back run),
    the step (quantise + partials on concurrent streams + merge) and the
    single launch of every shard (quantise + one call), both as graph
    replays checked bit for bit against the eager call. Also reported: the
    largest difference from the bf16-query step (the quantisation error)."""
    import torch

    from decode_attention_paged_amd import step as ST

    for dw in dws:
        dw.q_scale = 0.0
    ST.run_step(dws[0], bufs)
    torch.cuda.synchronize()
    ref_out, ref_lse = bufs.out.float().clone(), bufs.lse.clone()
    q_scale = float(dws[0].q.float().abs().max().item()) / 448.0
    log(f"[bench] {wl.name}: e4m3 query (q_scale {q_scale:.5f})")
    for dw in dws:
        dw.quantize_query(q_scale)
    torch.cuda.synchronize()
    try:
        ST.run_step(dws[0], bufs)
        torch.cuda.synchronize()
        fin = torch.isfinite(ref_lse)
        d_out = (bufs.out.float() - ref_out).abs().max().item()
        d_lse = (bufs.lse[fin] - ref_lse[fin]).abs().max().item() if bool(fin.any()) else 0.0
        S = wl.shards
        ev = [[(HipEvent(), HipEvent()) for _ in range(S)] for _ in range(steps)]
        qev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for k in range(warmup + steps):
            dw = dws[k % len(dws)]
            timed = k >= warmup
            for r in range(S):
                ST.run_partial(dw, bufs, r, reuse_plan=True, events=ev[k - warmup][r] if timed else None)
            if timed:
                qev[k - warmup][0].record()
            for _ in range(QUANT_REPEAT):
                dw.quantize_query(q_scale)
            if timed:
                qev[k - warmup][1].record()
            ST.run_merge(dw, bufs)
        torch.cuda.synchronize()
        attn_us = 1e3 * statistics.mean(a.elapsed_ms(b) for row in ev for a, b in row)
        quant_us = 1e3 * statistics.mean(a.elapsed_time(b) for a, b in qev) / QUANT_REPEAT
        rows = wl.batch * wl.q_len * wl.heads
        # algorithmic bytes per launch: the bf16-query figure less the query's
        # halved size (576 code bytes per row instead of 1152)
        launch_bytes = statistics.mean(b for b, _ in per_shard) - rows * 576
        launch_flops = statistics.mean(f for _, f in per_shard)
        quant_bytes = rows * 576 * 3
        out = dict(q_scale=q_scale, attn_kernel_us_per_shard=attn_us,
                   attn_kernel_bytes_per_launch=launch_bytes,
                   attn_kernel_gbs=launch_bytes / (attn_us * 1e-6) / 1e9,
                   attn_kernel_hbm_frac=launch_bytes / (attn_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                   attn_kernel_mfma_frac=launch_flops / (attn_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS,
                   quantize_us=quant_us, quantize_bytes=quant_bytes,
                   quantize_gbs=quant_bytes / (quant_us * 1e-6) / 1e9,
                   max_abs_diff_vs_bf16_query=dict(out=d_out, lse=d_lse))

        def step_fn(dw, streams):
            dw.quantize_query(q_scale)
            ST.run_step_concurrent(dw, bufs, streams, reuse_plan=True)

        def single_fn(dw, streams):
            dw.quantize_query(q_scale)
            ST.run_all_shards(dw, bufs, reuse_plan=True)

        streams = [torch.cuda.Stream() for _ in range(S)]
        for tag, fn in (("step", step_fn), ("all_shards_step", single_fn)):
            for dw in dws:
                fn(dw, streams)
            torch.cuda.synchronize()
            if use_graph:
                graphs = []
                for dw in dws:
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        fn(dw, streams)
                    graphs.append(g)
                torch.cuda.synchronize()
                for i, dw in enumerate(dws):
                    fn(dw, streams)
                    torch.cuda.synchronize()
                    eo, el = bufs.out.clone(), bufs.lse.clone()
                    bufs.fill_nan()
                    graphs[i].replay()
                    torch.cuda.synchronize()
                    if not (torch.equal(bufs.out.view(torch.uint8), eo.view(torch.uint8))
                            and torch.equal(bufs.lse.view(torch.uint8), el.view(torch.uint8))):
                        raise RuntimeError(f"graph replay of the e4m3-query {tag} differs from the eager call")
                run = lambda k: graphs[k % len(graphs)].replay()   # noqa: E731
            else:
                run = lambda k: fn(dws[k % len(dws)], streams)    # noqa: E731
            for k in range(warmup):
                run(k)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for k in range(steps):
                run(k)
            torch.cuda.synchronize()
            ms = 1e3 * (time.perf_counter() - t0) / steps
            out[tag] = dict(ms_per_step=ms, kv_gbs=kv_bytes / (ms * 1e-3) / 1e9,
                            timing="graph replay" if use_graph else "eager calls")
            if use_graph:
                del graphs
        return out
    finally:
        for dw in dws:
            dw.q_scale = 0.0


def _all_shards_result(wl, kv_bytes, flops, ms, attn_ms, d_out, d_lse, timing):
    # algorithmic bytes of the call: every visible KV row once, the queries
    # once, the merged out and LSE (the queries the kernel reads again for
    # each shard's segments are overhead, as piece partials are)
    rows = wl.batch * wl.q_len * wl.heads
    out_elt = 2 if wl.out_dtype == "bf16" else 4
    call_bytes = kv_bytes + rows * 576 * 2 + rows * (512 * out_elt + 4)
    return dict(ms_per_step=ms, kv_gbs=kv_bytes / (ms * 1e-3) / 1e9, tflops=flops / (ms * 1e-3) / 1e12,
                attn_kernel_us=1e3 * attn_ms, call_bytes=call_bytes,
                attn_kernel_gbs=call_bytes / (attn_ms * 1e-3) / 1e9,
                attn_kernel_hbm_frac=call_bytes / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                attn_kernel_mfma_frac=flops / (attn_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                step_timing=timing, max_abs_diff_vs_separate=dict(out=d_out, lse=d_lse))


def measure_copy_peak(nbytes: int = 1 << 30, reps: int = 10):
    """On-box HBM references from library kernels, timed by events over
    `reps` back-to-back runs: a device-to-device copy of `nbytes` (read and
    written once: 2 x nbytes per run) and a sum over `nbytes` of fp32 (read
    once), both sequential streams. `gbs` is the larger of the two; the
    HBM-bound kernels' fractions of it are reported next to those of the
    8 TB/s spec. They are references, not the chip's ceiling: LDS-DMA streams
    written for this library move more (6.0-6.9 TB/s sequential)."""
    import torch

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3

    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    copy_gbs = 2 * nbytes * reps / timed(lambda: dst.copy_(src)) / 1e9
    del src, dst
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    out = torch.empty((), dtype=torch.float32, device="cuda")
    read_gbs = nbytes * reps / timed(lambda: torch.sum(x, dim=0, out=out)) / 1e9
    del x, out
    torch.cuda.empty_cache()
    return dict(gbs=round(max(copy_gbs, read_gbs), 1), copy_gbs=round(copy_gbs, 1), read_gbs=round(read_gbs, 1),
                bytes=nbytes, runs=reps,
                method="events around back-to-back runs of a device-to-device copy (torch copy_, read + "
                       "write bytes) and an fp32 sum (torch sum, read bytes) of 1 GiB")


def bench_merge_sweep(replays: int = 20, warmup: int = 5):
    """Merge-only: 4 partials of [T, 64, 512] bf16 + fp32 LSE -> [T, 64, 512] bf16.

    Two timings per size: the kernel's own dispatch (HIP events recorded with
    the launch, eager launches over rotated input sets, so the MALL holds at
    most a fraction of them) — the roofline figure — and graph replays (one
    merge per input set in the graph): replay time / sets, i.e. back-to-back
    launches without host overhead, gaps between dispatches included."""
    import torch

    from decode_attention_paged_amd import _lib as L
    from workloads import MERGE_TOKENS, make_merge_inputs

    out = {}
    for T in MERGE_TOKENS:
        mi = make_merge_inputs(T, seed=4000 + T)
        set_bytes = 4 * T * 64 * (512 * 2 + 4) + T * 64 * 512 * 2 + T * 64 * 4
        nsets = max(2, min(64, int(math.ceil(600e6 / set_bytes))))
        sets = []
        for s_ in range(nsets):
            outs = [torch.from_numpy(o).view(torch.bfloat16).cuda() for o in mi.outs]
            lses = [torch.from_numpy(l).cuda() for l in mi.lses]
            sets.append((outs, lses, torch.empty((T, 64, 512), dtype=torch.bfloat16, device="cuda"),
                         torch.empty((T, 64), dtype=torch.float32, device="cuda")))
        for k in range(warmup):
            o, l, y, yl = sets[k % nsets]
            L.mla_merge_partials(o, l, [L.LSE_BASE_E] * 4, y, yl)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for o, l, y, yl in sets:
                L.mla_merge_partials(o, l, [L.LSE_BASE_E] * 4, y, yl)
        graph.replay()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(replays)]
        for a, b in evs:
            a.record()
            graph.replay()
            b.record()
        torch.cuda.synchronize()
        per = sorted(1e3 * a.elapsed_time(b) / nsets for a, b in evs)
        med = statistics.median(per)
        kevs = [(HipEvent(), HipEvent()) for _ in range(max(replays, nsets))]
        for k, ev in enumerate(kevs):
            o, l, y, yl = sets[k % nsets]
            L.mla_merge_partials(o, l, [L.LSE_BASE_E] * 4, y, yl, events=ev)
        torch.cuda.synchronize()
        kus = [1e3 * a.elapsed_ms(b) for a, b in kevs]
        kmean = statistics.mean(kus)
        out[str(T)] = dict(us_median=med, us_min=per[0], bytes=set_bytes,
                           gbs=set_bytes / (med * 1e-6) / 1e9, sets=nsets, timing="graph replay",
                           kernel_us_mean=kmean, kernel_us_min=min(kus), kernel_gbs=set_bytes / (kmean * 1e-6) / 1e9,
                           kernel_launches=len(kus))
        del sets, graph
    torch.cuda.empty_cache()
    return out


def bench_append(calls: int = 16, replays: int = 10):
    """KV append of one decode step's newest tokens (one token per request)
    into the owning shard's pool, at the bf16 default workload's shape (B 64,
    S 4) and the fp8 one's (B 32, S 8): µs per shard call, from graph replays
    of `calls` rounds of every shard's call (back-to-back dispatches without
    host overhead; the median replay / calls). A few hundred bytes per
    request: the call is latency bound, reported in µs only."""
    import numpy as np
    import torch

    from decode_attention_paged_amd import _lib as L
    from workloads import make_append_inputs

    out = {}
    for tag, B, S, kv_dtype in (("bf16 B64 S4", 64, 4, "bf16"), ("fp8 B32 S8", 32, 8, "fp8")):
        inp = make_append_inputs(batch=B, n_new=1, max_pages=64, num_pages=B * 64, kv_dtype=kv_dtype,
                                 kv_scale=0.05, seed=6000 + B)
        if kv_dtype == "bf16":
            pool = torch.from_numpy(inp.kv_pages.view(np.int16)).cuda().view(torch.bfloat16)
        else:
            pool = torch.from_numpy(inp.kv_pages).cuda()
        k_nope = torch.from_numpy(inp.k_nope.view(np.int16)).cuda().view(torch.bfloat16)
        k_rope = torch.from_numpy(inp.k_rope.view(np.int16)).cuda().view(torch.bfloat16)
        lens = torch.from_numpy(inp.seq_lens).cuda()
        bt = torch.from_numpy(inp.block_table).cuda()
        for r in range(S):
            L.mla_append_kv(k_nope, k_rope, lens, bt, pool, r, S, kv_scale=inp.kv_scale)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(calls):
                for r in range(S):
                    L.mla_append_kv(k_nope, k_rope, lens, bt, pool, r, S, kv_scale=inp.kv_scale)
        graph.replay()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(replays)]
        for a, b in evs:
            a.record()
            graph.replay()
            b.record()
        torch.cuda.synchronize()
        per = [1e3 * a.elapsed_time(b) / (calls * S) for a, b in evs]
        out[tag] = round(statistics.median(per), 2)
        del pool, graph
    torch.cuda.empty_cache()
    return out


# --------------------------------------------------------------------------
# CPU oracle baseline
# --------------------------------------------------------------------------
def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(wl, seconds: float, repeats: int = 3):
    """The fp64 oracle on the first requests of the workload (all shard
    partials + merge), on as many requests as fit in about seconds / repeats,
    timed `repeats` times; the median rate."""
    import numpy as np  # noqa: F401

    from oracle import mla_oracle as O
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = ",".join(sorted({str(i.get("internal_api")) for i in info})) or "unknown"
    except Exception:  # pragma: no cover
        threads, blas = 1, "unknown"
    row_bytes = 576 * (1 if wl.kv_dtype == "fp8" else 2)
    # size the sample with a first pass, then time it `repeats` times
    budget = seconds / repeats
    sample, t0 = [], time.perf_counter()
    for b in range(wl.batch):
        O.decode_step(wl, [b])
        sample.append(b)
        if time.perf_counter() - t0 >= budget:
            break
    nbytes = sum(int(wl.seq_lens[b]) for b in sample) * row_bytes
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        O.decode_step(wl, sample)
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    return dict(value=nbytes / med / 1e9, unit="GB/s", cores=int(threads), kind="oracle",
                cpu_model=cpu_model(), blas=blas, os_cpu_count=os.cpu_count(),
                sample=f"first {len(sample)} of {wl.batch} requests "
                       f"({sum(int(wl.seq_lens[b]) for b in sample)} tokens) of the {wl.name} workload: "
                       f"all {wl.shards} shard partials + merge, fp64 NumPy, median of {repeats} runs "
                       f"({', '.join(f'{t:.2f}' for t in times)} s)",
                seconds=med)


def binding_roof(r):
    """The attention kernel against the roof that binds it: HBM bytes or bf16
    MFMA flops (both KV types run bf16 MFMAs), whichever fraction is larger."""
    if r["attn_kernel_mfma_frac"] > r["attn_kernel_hbm_frac"]:
        return dict(bound="mfma", achieved=round(r["attn_kernel_tflops"], 2), peak=BF16_PEAK_TFLOPS,
                    unit="TFLOP/s", frac=round(r["attn_kernel_mfma_frac"], 4))
    return dict(bound="hbm", achieved=round(r["attn_kernel_gbs"], 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(r["attn_kernel_hbm_frac"], 4))


def config_summary(r):
    """One workload's figures for the JSON line (`traffic`: HBM bytes per
    attention launch from the committed counter summary of that workload,
    null unless it was taken on the current kernel sources)."""
    roof = binding_roof(r)
    roof["traffic"] = traffic_from_profile(r["name"])
    roof["algorithmic_bytes_per_launch"] = int(r["attn_kernel_bytes_per_launch"])
    out = dict(
        workload=f"batch {r['batch']}, {r['heads']} heads, q_len {r['q_len']}, {r['shards']} shards, "
                 f"{r['kv_dtype']} KV, {r['tokens']} tokens",
        ms_per_step=round(r["ms_per_step"], 5), kv_gbs=round(r["kv_gbs"], 1), tflops=round(r["tflops"], 2),
        attn_kernel_us_per_shard=round(r["attn_kernel_mean_us"], 2),
        attn_kernel=roof,
        merge_step=dict(us=round(r["merge_us"], 2), gbs=round(r["merge_gbs"], 1),
                        frac=round(r["merge_hbm_frac"], 4)),
        step_timing=r["step_timing"])
    if "all_shards" in r:
        a = r["all_shards"]
        out["all_shards_step"] = dict(ms_per_step=round(a["ms_per_step"], 5), kv_gbs=round(a["kv_gbs"], 1),
                                      attn_kernel_us=round(a["attn_kernel_us"], 2),
                                      attn_kernel_hbm_frac=round(a["attn_kernel_hbm_frac"], 4),
                                      attn_kernel_mfma_frac=round(a.get("attn_kernel_mfma_frac", 0.0), 4),
                                      algorithmic_bytes_per_launch=int(a["call_bytes"]),
                                      traffic=traffic_from_profile("all_shards_" + r["name"]),
                                      step_timing=a.get("step_timing", "graph replay"))
    if "e4m3_query" in r:
        e = r["e4m3_query"]
        out["e4m3_query"] = dict(
            q_scale=round(e["q_scale"], 6),
            attn_kernel_us_per_shard=round(e["attn_kernel_us_per_shard"], 2),
            attn_kernel=dict(bound="hbm", achieved=round(e["attn_kernel_gbs"], 1), peak=HBM_PEAK_GBS, unit="GB/s",
                             frac=round(e["attn_kernel_hbm_frac"], 4),
                             algorithmic_bytes_per_launch=int(e["attn_kernel_bytes_per_launch"]),
                             traffic=traffic_from_profile("e4m3_query_" + r["name"])),
            quantize_kernel=dict(us=round(e["quantize_us"], 2), bytes=int(e["quantize_bytes"]),
                                 gbs=round(e["quantize_gbs"], 1)),
            step=dict(ms_per_step=round(e["step"]["ms_per_step"], 5), kv_gbs=round(e["step"]["kv_gbs"], 1),
                      timing=e["step"]["timing"] + ", quantise + shard partials on concurrent streams + merge"),
            all_shards_step=dict(ms_per_step=round(e["all_shards_step"]["ms_per_step"], 5),
                                 kv_gbs=round(e["all_shards_step"]["kv_gbs"], 1),
                                 timing=e["all_shards_step"]["timing"] + ", quantise + one call"),
            max_abs_diff_vs_bf16_query={k: float(f"{v:.3e}") for k, v in e["max_abs_diff_vs_bf16_query"].items()})
    return out


def assemble_line(args, wl, res, merge, append, per_config, cpu, hbm_measured) -> dict:
    """The JSON line: the headline workload's step and attention kernel, the
    merge sweep and append timing, every workload under `configs`, the CPU
    baseline and the on-box HBM references."""
    mfma_bound = res["attn_kernel_mfma_frac"] > res["attn_kernel_hbm_frac"]
    if mfma_bound:
        peak = BF16_PEAK_TFLOPS
        roof = dict(bound="mfma", achieved=res["attn_kernel_tflops"], peak=peak, unit="TFLOP/s",
                    frac=res["attn_kernel_tflops"] / peak)
    else:
        roof = dict(bound="hbm", achieved=res["attn_kernel_gbs"], peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=res["attn_kernel_gbs"] / HBM_PEAK_GBS)
    roof["traffic"] = traffic_from_profile(wl.name)
    kname = "attn_ws_kernel<block table, %s KV> (mla_stream.hip)" % wl.kv_dtype
    roof["kernel"] = kname + ", mean of %d launches" % (args.steps * wl.shards)
    roof["mean_launch_us"] = res["attn_kernel_mean_us"]
    roof["algorithmic_bytes_per_launch"] = res["attn_kernel_bytes_per_launch"]
    if roof["bound"] == "hbm":
        roof["measured_reference"] = hbm_measured["gbs"]
        roof["frac_of_measured_reference"] = roof["achieved"] / hbm_measured["gbs"]

    line = {
        "metric": METRIC,
        "value": round(res["kv_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",            # MFMA contraction type (fp8 KV is converted to bf16)
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: batch {wl.batch}, {wl.heads} heads, q_len {wl.q_len}, "
                               f"{wl.shards} cyclic shards, {wl.kv_dtype} KV, page 64, "
                               f"{res['tokens']} context tokens, partials + merge",
                   "global_batch": wl.batch, "shards": wl.shards, "step": res["step_timing"],
                   "per_decode_step": "schedule %.1f us per shard, not in the step (shard metadata, not used by the step: %.1f us)"
                                      % (res["plan_us_per_shard"], res["metadata_us_per_shard"])},
        "tflops": round(res["tflops"], 3),
        "merge_us": {T: round(v["us_median"], 2) for T, v in merge.items()} if merge else None,
        "merge_kernel_us": {T: round(v["kernel_us_mean"], 2) for T, v in merge.items()} if merge else None,
        "merge_roofline": (dict(bound="hbm", T=128, achieved=round(merge["128"]["kernel_gbs"], 1), peak=HBM_PEAK_GBS,
                                unit="GB/s", frac=round(merge["128"]["kernel_gbs"] / HBM_PEAK_GBS, 4),
                                kernel_us=round(merge["128"]["kernel_us_mean"], 2))
                           if merge and "128" in merge else None),
        "merge_step": dict(us=round(res["merge_us"], 2), bytes=int(res["merge_bytes"]),
                           gbs=round(res["merge_gbs"], 1), frac=round(res["merge_hbm_frac"], 4),
                           shards=wl.shards, timing="the step's merge kernel, its own dispatch (eager)"),
        "append_us": append,
        "all_shards_step": (dict(ms_per_step=round(res["all_shards"]["ms_per_step"], 5),
                                 kv_gbs=round(res["all_shards"]["kv_gbs"], 1),
                                 attn_kernel_us=round(res["all_shards"]["attn_kernel_us"], 2),
                                 attn_kernel_hbm_frac=round(res["all_shards"]["attn_kernel_hbm_frac"], 4),
                                 timing="mla_decode_all_shards: every shard in one launch, merge fused, "
                                        + res["all_shards"].get("step_timing", "graph replay")
                                        + "; schedule built once per step")
                            if "all_shards" in res else None),
        "roofline": roof,
        "hbm_measured": hbm_measured,
        "configs": per_config,
        "cpu_baseline": cpu,
    }
    if line["merge_roofline"]:
        line["merge_roofline"]["frac_of_measured_reference"] = round(
            line["merge_roofline"]["achieved"] / hbm_measured["gbs"], 4)
    return line


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="workload index 1..5 for the headline line")
    ap.add_argument("--configs", default="1,2,3,4,5",
                    help="comma list of workloads measured under `configs` (the headline one always runs)")
    ap.add_argument("--details", default=None, help="write per-workload results (JSON) here")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-merge-sweep", action="store_true", help="skip the merge-only sweep and the append timing")
    ap.add_argument("--no-graph", action="store_true", help="time the step as eager launches")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--split-target", type=int, default=0,
                    help="KV chunks per launch per row block (0 = library default)")
    ap.add_argument("--sweep-split", default=None,
                    help="comma list of split targets to time on the headline workload (details only)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes 5 times and exit "
                         "(reference kernel for scaling the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_calibration:
        n = int(args.copy_calibration)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)
        return 0
    from decode_attention_paged_amd import _lib as L
    L.load()

    wl, res = bench_workload(args.config, args.steps, args.warmup, split_target=args.split_target,
                             use_graph=not args.no_graph)
    details = {"headline": res}
    if args.sweep_split:
        for tgt in [int(x) for x in args.sweep_split.split(",")]:
            _, r = bench_workload(args.config, args.steps, args.warmup, split_target=tgt)
            details[f"split{tgt}"] = r
            log(f"[bench] split {tgt}: {r['ms_per_step']:.3f} ms/step, attn {r['attn_kernel_mean_us']:.1f} us "
                f"({100 * r['attn_kernel_hbm_frac']:.1f}% HBM)")
    merge = None if args.no_merge_sweep else bench_merge_sweep()
    if merge:
        details["merge_only"] = merge
    append = None if args.no_merge_sweep else bench_append()
    if append:
        details["append_us_per_shard_call"] = append
    per_config = {}
    for idx in [int(x) for x in args.configs.split(",") if x.strip()]:
        if idx == args.config:
            r = res
        else:
            _, r = bench_workload(idx, args.steps, args.warmup, use_graph=not args.no_graph)
            details[f"config{idx}"] = r
        per_config[r["name"]] = config_summary(r)
        log(f"[bench] config {idx} {r['name']}: {r['ms_per_step']:.3f} ms/step, "
            f"{r['kv_gbs']:.0f} KV-GB/s, {r['tflops']:.1f} TFLOP/s, attn kernel "
            f"{r['attn_kernel_gbs']:.0f} GB/s ({100 * r['attn_kernel_hbm_frac']:.1f}% HBM, "
            f"{100 * r['attn_kernel_mfma_frac']:.1f}% MFMA), merge {r['merge_us']:.1f} us "
            f"({r['merge_gbs']:.0f} GB/s, {100 * r['merge_hbm_frac']:.1f}% HBM)")
        if "all_shards" in r:
            a = r["all_shards"]
            log(f"[bench] config {idx} {r['name']} single launch: {a['ms_per_step']:.3f} ms/step, "
                f"{a['kv_gbs']:.0f} KV-GB/s, attn kernel {a['attn_kernel_us']:.1f} us "
                f"({100 * a['attn_kernel_hbm_frac']:.1f}% HBM)")
        if "e4m3_query" in r:
            e = r["e4m3_query"]
            log(f"[bench] config {idx} {r['name']} e4m3 query: step {e['step']['ms_per_step']:.3f} ms, single "
                f"launch {e['all_shards_step']['ms_per_step']:.3f} ms, attn kernel "
                f"{e['attn_kernel_us_per_shard']:.1f} us/shard, quantise {e['quantize_us']:.1f} us, "
                f"vs bf16 query out {e['max_abs_diff_vs_bf16_query']['out']:.2e}")

    cpu = None if args.no_cpu else cpu_baseline(wl, args.cpu_seconds)
    hbm_measured = measure_copy_peak()
    log(f"[bench] on-box HBM references: copy {hbm_measured['copy_gbs']:.0f} GB/s, "
        f"read {hbm_measured['read_gbs']:.0f} GB/s")
    for r in per_config.values():
        ak = r["attn_kernel"]
        if ak["bound"] == "hbm":
            ak["frac_of_measured_reference"] = round(ak["achieved"] / hbm_measured["gbs"], 4)
    line = assemble_line(args, wl, res, merge, append, per_config, cpu, hbm_measured)
    if args.details:
        os.makedirs(os.path.dirname(os.path.abspath(args.details)), exist_ok=True)
        with open(args.details, "w") as f:
            json.dump(details, f, indent=1)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
