"""GPU parity of the single-launch decode of every shard with the merge fused
(mla_decode_all_shards through the C ABI) against the oracle: the S shard
partials of the cyclic split followed by their LSE-weighted merge, and the
unsharded attention they must equal. Covers every workload shape scaled
down, shard counts 1-16, q_len 4 with per-request depths, both LSE bases and
output dtypes, zero-length requests, more segments than the schedule keeps
in LDS, sampled requests at the full kimi-like, fp8 and skewed sizes, the
reused schedule and HIP-graph replays.
"""
import numpy as np
import pytest
import torch

import gpu_util as U
from oracle import mla_oracle as O
from workloads import make_config, make_workload

pytestmark = pytest.mark.gpu

if U.gpu_available():
    from decode_attention_paged_amd import _lib as L
    from decode_attention_paged_amd import step as ST

SMALL = {
    "tiny": dict(index=1),
    "kimi_like": dict(index=2, batch=3, lens=("uniform", 300, 700)),
    "deepseek_like_fp8": dict(index=3, batch=2, lens=("uniform", 700, 1500)),
    "mtp_q4": dict(index=4, batch=2, lens=("uniform", 100, 400)),
    "skewed": dict(index=5, batch=14, lens=("skewed", 1, 1500)),
}


def _flush(msg):
    print(msg, flush=True)


def _small(name, **extra):
    spec = dict(SMALL[name])
    idx = spec.pop("index")
    spec.update(extra)
    return make_config(idx, **spec)


def _check(wl, bufs, what, out_base="e"):
    ref_o, ref_l, _ = O.decode_step(wl, out_base=out_base)
    U.assert_partial_close(bufs.out, bufs.lse, ref_o, ref_l, out_base, U.TOL[wl.kv_dtype], f"merged {what}")
    full_o, full_l = O.decode_full(wl)
    U.assert_partial_close(bufs.out, bufs.lse, full_o, O.to_base(full_l, out_base), out_base,
                           U.TOL[wl.kv_dtype], f"unsharded {what}")


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("split_target", [0, 7, 64])
def test_all_shards_parity(name, split_target):
    wl = _small(name)
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    bufs.fill_nan()
    _flush(f"all shards {name} S={wl.shards} split={split_target}")
    written = ST.run_all_shards(dw, bufs, split_target=split_target)
    torch.cuda.synchronize()
    assert written == L.LSE_BASE_E
    _check(wl, bufs, name)


@pytest.mark.parametrize("shards", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_all_shards_shard_counts(shards, kv_dtype):
    wl = make_workload("counts", batch=5, heads=64, q_len=1, shards=shards, kv_dtype=kv_dtype,
                       lens=("uniform", 1, 900), seed=40 + shards, out_dtype="bf16")
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    bufs.fill_nan()
    _flush(f"all shards S={shards} {kv_dtype}")
    ST.run_all_shards(dw, bufs)
    torch.cuda.synchronize()
    _check(wl, bufs, f"S={shards} {kv_dtype}")


@pytest.mark.parametrize("var_q", [False, True])
@pytest.mark.parametrize("shards", [2, 4])
def test_all_shards_draft_rows(var_q, shards):
    """q_len 4 under S > 1: row i of request b sees the tokens up to
    L - q_b + i of every shard; with per-request depths, rows past q_b are
    (0, -inf) after the merge too."""
    wl = make_workload("mtp", batch=6, heads=32, q_len=4, shards=shards, kv_dtype="bf16",
                       lens=("uniform", 1, 500), seed=60 + shards, var_q=var_q)
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    bufs.fill_nan()
    _flush(f"all shards draft rows S={shards} var_q={var_q}")
    ST.run_all_shards(dw, bufs)
    torch.cuda.synchronize()
    _check(wl, bufs, f"draft S={shards}")


def test_all_shards_lse_base_two_and_f32_out():
    wl = _small("skewed")
    dw = ST.DeviceWorkload.upload(wl, out_dtype="f32")
    bufs = ST.StepBuffers(dw)
    bufs.fill_nan()
    _flush("all shards base 2, f32 out")
    assert ST.run_all_shards(dw, bufs, out_base=L.LSE_BASE_2) == L.LSE_BASE_2
    torch.cuda.synchronize()
    assert bufs.out.dtype == torch.float32
    _check(wl, bufs, "base 2", out_base="2")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_all_shards_zero_length_and_tiny_requests(kv_dtype):
    """Lengths 0, 1 and 2 next to a longer request, q_len 2: rows that see no
    token on any shard are exactly (+0, -inf)."""
    wl = make_workload("zero", batch=6, heads=16, q_len=2, shards=3, kv_dtype=kv_dtype,
                       lens=("fixed", [0, 1, 0, 65, 2, 0]), seed=3, out_dtype="bf16")
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    bufs.fill_nan()
    _flush(f"all shards zero-length {kv_dtype}")
    ST.run_all_shards(dw, bufs)
    torch.cuda.synchronize()
    _check(wl, bufs, f"zero {kv_dtype}")
    lse = bufs.lse.cpu().numpy()
    out = bufs.out.float().cpu().numpy()
    for b in (0, 2, 5):
        assert np.all(np.isneginf(lse[b])) and np.all(out[b] == 0) and not np.any(np.signbit(out[b]))
    assert np.all(np.isneginf(lse[1, 0])) and np.all(np.isfinite(lse[1, 1]))


def test_all_shards_many_segments_and_reused_schedule():
    """6300 requests x 2 shards = 12600 segments (offset tables in the
    workspace); NaN-prefilled outputs must be fully written, sampled requests
    must match the oracle and the reused schedule must give the same bytes."""
    wl = make_workload("many", batch=6300, heads=16, q_len=1, shards=2, kv_dtype="bf16",
                       lens=("uniform", 1, 60), seed=778, out_dtype="bf16")
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    bufs.fill_nan()
    _flush("all shards many segments")
    ST.run_all_shards(dw, bufs)
    torch.cuda.synchronize()
    assert not torch.isnan(bufs.out.float()).any() and not torch.isnan(bufs.lse).any()
    rng = np.random.default_rng(6)
    sample = sorted(rng.choice(wl.batch, size=300, replace=False).tolist() + [0, wl.batch - 1])
    full_o, full_l = O.decode_full(wl, requests=sample)
    U.assert_partial_close(bufs.out[sample], bufs.lse[sample], full_o, full_l, "e", U.TOL["bf16"], "many")
    first_o, first_l = bufs.out.clone(), bufs.lse.clone()
    bufs.fill_nan()
    ST.run_all_shards(dw, bufs, reuse_plan=True)
    torch.cuda.synchronize()
    assert torch.equal(bufs.out.view(torch.int16), first_o.view(torch.int16))
    assert torch.equal(bufs.lse.view(torch.int32), first_l.view(torch.int32))


@pytest.mark.parametrize("index", [2, 3, 5])
def test_all_shards_full_size_sampled(index):
    """The full kimi-like (S 4), fp8 (S 8) and skewed (S 8) workloads in the
    launch configuration the benchmark times; sampled requests against the
    unsharded oracle (skewed: its eight shortest requests, whose outputs are
    close to single V rows and so the largest, the longest and the median
    too), every row written."""
    wl = make_config(index)
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    bufs.fill_nan()
    _flush(f"all shards full size config {wl.name}")
    ST.run_all_shards(dw, bufs)
    torch.cuda.synchronize()
    assert not torch.isnan(bufs.out.float()).any() and not torch.isnan(bufs.lse).any()
    sample = [0, 7, wl.batch - 1]
    if index == 5:
        order = np.argsort(wl.seq_lens, kind="stable")
        sample = sorted({int(x) for x in order[:8]} | {int(order[-1]), int(order[len(order) // 2])})
    full_o, full_l = O.decode_full(wl, requests=sample)
    U.assert_partial_close(bufs.out[sample], bufs.lse[sample], full_o, full_l, "e", U.TOL[wl.kv_dtype],
                           f"full {wl.name}")


def test_all_shards_matches_the_separate_step_and_graph_replays():
    """The one-launch result agrees with the per-shard partials + merge, and
    a HIP graph of the call replayed three times (fresh NaN outputs and eager
    work in between) writes the eager bytes every time."""
    wl = _small("deepseek_like_fp8")
    dw = ST.DeviceWorkload.upload(wl)
    sep = ST.StepBuffers(dw)
    ST.run_step(dw, sep)
    bufs = ST.StepBuffers(dw)
    _flush("all shards vs separate step, graph replays")
    ST.run_all_shards(dw, bufs)
    torch.cuda.synchronize()
    tol = U.TOL[wl.kv_dtype]
    assert (bufs.out.float() - sep.out.float()).abs().max().item() <= tol
    assert (bufs.lse - sep.lse).abs().max().item() <= tol
    eager_o, eager_l = bufs.out.clone(), bufs.lse.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ST.run_all_shards(dw, bufs)
    torch.cuda.synchronize()
    for rep in range(3):
        bufs.fill_nan()
        scratch = torch.randn(1 << 16, device="cuda").sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs.out.view(torch.int16) if bufs.out.dtype == torch.bfloat16 else bufs.out.view(torch.int32),
                           eager_o.view(torch.int16) if eager_o.dtype == torch.bfloat16 else eager_o.view(torch.int32)), rep
        assert torch.equal(bufs.lse.view(torch.int32), eager_l.view(torch.int32)), rep
        del scratch


def test_all_shards_short_requests_with_empty_shards():
    """Lengths 0..7 with S = 8: most shards own nothing; the merged rows match
    the oracle and the request of length 0 is exactly (+0, -inf)."""
    wl = make_workload("short", batch=8, heads=32, q_len=1, shards=8, kv_dtype="bf16",
                       lens=("fixed", (1, 2, 3, 4, 5, 6, 7, 0)), seed=5, out_dtype="bf16")
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    bufs.fill_nan()
    _flush("all shards short requests, S 8")
    ST.run_all_shards(dw, bufs, out_base=L.LSE_BASE_2)
    torch.cuda.synchronize()
    _check(wl, bufs, "short", out_base="2")
    mo, ml = bufs.out.float().cpu().numpy(), bufs.lse.cpu().numpy()
    assert np.all(mo[7] == 0) and not np.signbit(mo[7]).any() and np.all(np.isneginf(ml[7]))
    assert np.all(np.isfinite(ml[:7]))


@pytest.mark.parametrize("split_target", [8, 64])
def test_all_shards_bad_page_ids_poison_instead_of_faulting(split_target):
    """A page id outside the pool (and a negative one) reads the NaN row: the
    request that owns it comes out NaN in every row, out and LSE (the fused
    merge must not take a poisoned shard for an empty one), whether its
    shards' segments are whole or cut into pieces; the other requests match
    the oracle."""
    wl = make_workload("bad", batch=16, heads=16, q_len=1, shards=2, kv_dtype="bf16",
                       lens=("fixed", (200,) * 15 + (130,)), seed=9)
    ok = list(range(1, wl.batch - 1))
    ok_o, ok_l = O.decode_full(wl, requests=ok)
    wl.block_table[0, 1] = 10_000          # outside the pool
    wl.block_table[15, 2] = -5             # negative
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    bufs.fill_nan()
    _flush(f"all shards bad page ids split={split_target}")
    ST.run_all_shards(dw, bufs, split_target=split_target)
    torch.cuda.synchronize()
    o, l = bufs.out.float().cpu().numpy(), bufs.lse.cpu().numpy()
    for b in (0, 15):
        assert np.isnan(o[b]).all() and np.isnan(l[b]).all(), f"request {b} not poisoned"
    U.assert_partial_close(bufs.out[ok], bufs.lse[ok], ok_o, ok_l, "e", U.TOL["bf16"], "untouched requests")
