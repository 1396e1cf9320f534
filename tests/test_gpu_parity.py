"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Inputs are the seeded workloads of ``workloads`` (the five workload shapes,
scaled down so the oracle finishes in seconds while still spanning several
32-token tiles, several KV chunks per request and ragged tails; the full
sizes are checked on sampled requests in test_gpu_fullsize.py). Outputs are
pre-filled with NaN so an unwritten row fails.
Tolerances: out and LSE max-abs 2e-2 (bf16 KV) / 6e-2 (fp8 KV), LSE in nats;
neutral rows exactly (+0, -inf); metadata bit-exact. Merge: fp32 output
within 1e-5 of each (row, head) vector's largest magnitude, LSE within
1e-5 * max(1, |lse|); bf16 output within one bf16 ulp of the fp64 result plus
that same fp32 bound (the kernel accumulates in fp32, so its error is relative
to the vector's largest term, which can exceed a small result's ulp under
cancellation, and then rounds once to bf16).
"""
import math

import numpy as np
import pytest
import torch

import gpu_util as U
from oracle import mla_oracle as O
from workloads import make_config, make_merge_inputs, make_workload

pytestmark = pytest.mark.gpu

if U.gpu_available():
    from decode_attention_paged_amd import _lib as L
    from decode_attention_paged_amd import step as ST


def _flush(msg):
    print(msg, flush=True)


# scaled-down instances of the five workload shapes
SMALL = {
    "tiny": dict(index=1),
    "kimi_like": dict(index=2, batch=3, lens=("uniform", 300, 700)),
    "deepseek_like_fp8": dict(index=3, batch=2, lens=("uniform", 700, 1500)),
    "mtp_q4": dict(index=4, batch=2, lens=("uniform", 100, 400)),
    "skewed": dict(index=5, batch=14, lens=("skewed", 1, 1500)),
}


def _small(name, **extra):
    spec = dict(SMALL[name])
    idx = spec.pop("index")
    spec.update(extra)
    return make_config(idx, **spec)


# --------------------------------------------------------------------------
# metadata
# --------------------------------------------------------------------------
@pytest.mark.parametrize("S", [1, 2, 3, 4, 8])
def test_metadata_bit_exact(S):
    rng = np.random.default_rng(100 + S)
    B = 9
    seq_lens = rng.integers(0, 400, size=B).astype(np.int32)
    seq_lens[0] = 0
    seq_lens[1] = 1
    maxp = int(max(1, ((seq_lens.max() + 63) // 64)))
    npages = int(sum((L_ + 63) // 64 for L_ in seq_lens))
    perm = rng.permutation(max(npages, 1)).astype(np.int32)
    bt = np.full((B, maxp), -1, np.int32)
    off = 0
    for b, L_ in enumerate(seq_lens):
        k = (int(L_) + 63) // 64
        bt[b, :k] = perm[off:off + k]
        off += k
    M = int(seq_lens.max())
    d_sl = torch.from_numpy(seq_lens).cuda()
    d_bt = torch.from_numpy(bt).cuda()
    for r in range(S):
        _flush(f"metadata S={S} r={r}")
        lens, lmax, idx = O.shard_metadata(seq_lens, bt, 64, M, r, S)
        out_l = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        out_i = torch.full((B, lmax + 3), -7, dtype=torch.int32, device="cuda")
        got_max = L.mla_build_shard_metadata(d_sl, d_bt, M, r, S, out_l, out_i)
        torch.cuda.synchronize()
        assert got_max == lmax
        assert np.array_equal(out_l.cpu().numpy(), lens)
        gi = out_i.cpu().numpy()
        assert np.array_equal(gi[:, :lmax], idx)
        assert (gi[:, lmax:] == -1).all()


def test_metadata_pages_sweep():
    """The pages' layout sweep (sizes 1,2,3,4,8; lengths 0..40) as one batch."""
    lens = np.arange(0, 41, dtype=np.int32)
    bt = np.zeros((41, 1), np.int32)
    d_sl, d_bt = torch.from_numpy(lens).cuda(), torch.from_numpy(bt).cuda()
    for S in (1, 2, 3, 4, 8):
        tot = np.zeros(41, np.int64)
        per = []
        for r in range(S):
            out_l = torch.empty((41,), dtype=torch.int32, device="cuda")
            L.mla_build_shard_metadata(d_sl, d_bt, 40, r, S, out_l, None)
            torch.cuda.synchronize()
            got = out_l.cpu().numpy().astype(np.int64)
            per.append(got)
            tot += got
        assert np.array_equal(tot, lens)
        for Lg in range(1, 41):
            grew = [int(per[r][Lg] - per[r][Lg - 1]) for r in range(S)]
            assert sum(grew) == 1 and grew[(Lg - 1) % S] == 1


# --------------------------------------------------------------------------
# partial decode, per shard
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("use_metadata", [True, False])
@pytest.mark.parametrize("split_target", [0, 1, 37])
def test_partial_parity(name, use_metadata, split_target):
    wl = _small(name)
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    bufs.fill_nan()
    tol = U.TOL[wl.kv_dtype]
    for r in range(wl.shards):
        _flush(f"partial {name} meta={use_metadata} split={split_target} shard={r}/{wl.shards}")
        if use_metadata:
            ST.run_metadata(dw, bufs, r)
        base = ST.run_partial(dw, bufs, r, use_metadata=use_metadata, split_target=split_target)
        assert base == dw.lse_base
        torch.cuda.synchronize()
        ref_o, ref_l = O.decode_partial(wl, r, wl.shards, wl.lse_base)
        U.assert_partial_close(bufs.outs[r], bufs.lses[r], ref_o, ref_l, wl.lse_base, tol,
                               f"{name} shard {r}")


@pytest.mark.parametrize("kv_dtype,heads,q_len,shards,out_dtype", [
    ("bf16", 16, 4, 1, "f32"), ("bf16", 64, 4, 4, "bf16"), ("fp8", 128, 3, 2, "bf16"), ("bf16", 32, 2, 3, "f32")])
def test_partial_parity_per_request_depth(kv_dtype, heads, q_len, shards, out_dtype):
    """A decode depth per request (0 .. q_len, drawn): real rows against the
    oracle, padding rows exactly (+0, -inf); then the merged step."""
    wl = make_workload("var_q", batch=6, heads=heads, q_len=q_len, shards=shards, kv_dtype=kv_dtype,
                       lens=("uniform", 1, 700), seed=61 + heads + q_len, out_dtype=out_dtype, var_q=True)
    assert wl.q_lens is not None and (wl.q_lens < q_len).any()
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    bufs.fill_nan()
    tol = U.TOL[kv_dtype]
    parts = []
    for r in range(wl.shards):
        _flush(f"per-request depth {kv_dtype} H={heads} q={q_len} q_lens={wl.q_lens.tolist()} shard={r}/{shards}")
        ST.run_metadata(dw, bufs, r)
        ST.run_partial(dw, bufs, r)
        torch.cuda.synchronize()
        ref_o, ref_l = O.decode_partial(wl, r, wl.shards, wl.lse_base)
        parts.append((ref_o, ref_l))
        U.assert_partial_close(bufs.outs[r], bufs.lses[r], ref_o, ref_l, wl.lse_base, tol, f"var_q shard {r}")
    ST.run_merge(dw, bufs)
    torch.cuda.synchronize()
    mo, ml = O.merge([p_[0] for p_ in parts], [p_[1] for p_ in parts], [wl.lse_base] * wl.shards)
    U.assert_partial_close(bufs.out, bufs.lse, mo, ml, "e", tol, "var_q merged")


@pytest.mark.parametrize("kv_dtype,q_len", [("bf16", 1), ("fp8", 1), ("bf16", 2)])
def test_max_shard_count(kv_dtype, q_len):
    """S = 16 (the largest supported): a wave's eight owned tokens span 128
    positions and up to three pages on the block-table path. Every shard
    through both gather paths, the metadata bit-exact, then the 16-way
    merge against the unsharded oracle."""
    S = 16
    wl = make_workload("s16", batch=3, heads=16, q_len=q_len, shards=S, kv_dtype=kv_dtype,
                       lens=("uniform", 1, 2600), seed=160 + q_len, out_dtype="bf16")
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    tol = U.TOL[kv_dtype]
    for use_metadata in (False, True):
        bufs.fill_nan()
        for r in range(S):
            _flush(f"max shards {kv_dtype} q={q_len} meta={use_metadata} shard={r}/{S}")
            if use_metadata:
                lmax = ST.run_metadata(dw, bufs, r)
                ref_len, ref_max, ref_idx = O.shard_metadata(wl.seq_lens, wl.block_table, 64, wl.max_seq_len, r, S)
                torch.cuda.synchronize()
                assert lmax == ref_max
                assert np.array_equal(bufs.local_seq_lens[r].cpu().numpy(), ref_len)
                got_idx = bufs.local_kv_indices[r].cpu().numpy()
                assert np.array_equal(got_idx[:, :ref_idx.shape[1]], ref_idx)
            ST.run_partial(dw, bufs, r, use_metadata=use_metadata)
            torch.cuda.synchronize()
            ref_o, ref_l = O.decode_partial(wl, r, S, wl.lse_base)
            U.assert_partial_close(bufs.outs[r], bufs.lses[r], ref_o, ref_l, wl.lse_base, tol,
                                   f"S16 shard {r} meta={use_metadata}")
    ST.run_merge(dw, bufs)
    torch.cuda.synchronize()
    full_o, full_l = O.decode_full(wl)
    U.assert_partial_close(bufs.out, bufs.lse, full_o, full_l, "e", tol, "S16 merged")


@pytest.mark.parametrize("kv_dtype,heads,q_len,out_dtype", [
    ("bf16", 48, 1, "f32"), ("fp8", 80, 1, "bf16"), ("bf16", 16, 3, "bf16"), ("fp8", 112, 2, "f32")])
def test_partial_parity_partial_row_blocks(kv_dtype, heads, q_len, out_dtype):
    """Row counts that leave part of a 64-row block empty (48, 80, 48, 224
    rows): the empty rows are computed on zero queries and never stored."""
    wl = make_workload("rows", batch=3, heads=heads, q_len=q_len, shards=3, kv_dtype=kv_dtype,
                       lens=("uniform", 1, 900), seed=31 + heads, out_dtype=out_dtype)
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    bufs.fill_nan()
    tol = U.TOL[wl.kv_dtype]
    for r in range(wl.shards):
        _flush(f"partial rows={heads * q_len} {kv_dtype} shard={r}")
        ST.run_metadata(dw, bufs, r)
        ST.run_partial(dw, bufs, r, split_target=7)
        torch.cuda.synchronize()
        ref_o, ref_l = O.decode_partial(wl, r, wl.shards, wl.lse_base)
        U.assert_partial_close(bufs.outs[r], bufs.lses[r], ref_o, ref_l, wl.lse_base, tol,
                               f"rows {heads * q_len} shard {r}")


def test_maximum_heads_fill_the_workgroup_tables():
    """num_heads at its maximum (16384) with q_len 4: one request is 1024
    row blocks, so its row-block group takes all 1024 workgroups that the
    schedule's tables hold. Each shard's partial and the single launch of
    every shard match the oracle; the merged reference is the oracle's merge
    of its own shard partials."""
    wl = make_workload("maxheads", batch=2, heads=L.MAX_HEADS, q_len=4, shards=2, kv_dtype="bf16",
                       lens=("uniform", 40, 160), seed=91)
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    bufs.fill_nan()
    tol = U.TOL[wl.kv_dtype]
    parts = []
    for r in range(wl.shards):
        _flush(f"max heads {L.MAX_HEADS} x q_len 4, shard {r}")
        ST.run_partial(dw, bufs, r)
        torch.cuda.synchronize()
        ref_o, ref_l = O.decode_partial(wl, r, wl.shards, wl.lse_base)
        U.assert_partial_close(bufs.outs[r], bufs.lses[r], ref_o, ref_l, wl.lse_base, tol, f"max heads shard {r}")
        parts.append((ref_o, ref_l))
    _flush(f"max heads {L.MAX_HEADS} x q_len 4, every shard in one launch")
    bufs.fill_nan()
    ST.run_all_shards(dw, bufs)
    torch.cuda.synchronize()
    ref_o, ref_l = O.merge([o for o, _ in parts], [l for _, l in parts], [wl.lse_base] * wl.shards)
    U.assert_partial_close(bufs.out, bufs.lse, ref_o, ref_l, "e", tol, "max heads, every shard in one launch")


def test_partial_bf16_output():
    wl = _small("kimi_like")
    dw = ST.DeviceWorkload.upload(wl, out_dtype="bf16")
    bufs = ST.StepBuffers(dw)
    bufs.fill_nan()
    for r in range(wl.shards):
        ST.run_metadata(dw, bufs, r)
        ST.run_partial(dw, bufs, r, split_target=5)
        torch.cuda.synchronize()
        ref_o, ref_l = O.decode_partial(wl, r, wl.shards, wl.lse_base)
        assert bufs.outs[r].dtype == torch.bfloat16
        U.assert_partial_close(bufs.outs[r], bufs.lses[r], ref_o, ref_l, wl.lse_base, 2e-2, f"bf16 out shard {r}")


def test_empty_shards_are_exactly_neutral():
    # lengths 1..7 with S = 8: shards >= L own nothing
    wl = make_workload("short", batch=8, heads=32, q_len=1, shards=8, kv_dtype="bf16",
                       lens=("fixed", (1, 2, 3, 4, 5, 6, 7, 0)), seed=5, lse_base="2")
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    bufs.fill_nan()
    ST.run_step(dw, bufs)
    torch.cuda.synchronize()
    for r in range(8):
        lse = bufs.lses[r].cpu().numpy()
        out = bufs.outs[r].cpu().numpy()
        for b, Lb in enumerate(wl.seq_lens):
            if r >= Lb:
                assert np.all(np.isneginf(lse[b])) and np.all(out[b] == 0) and not np.signbit(out[b]).any()
            else:
                assert np.all(np.isfinite(lse[b]))
    # the request of length 0 merges to (0, -inf)
    mo, ml = bufs.out.cpu().numpy(), bufs.lse.cpu().numpy()
    assert np.all(mo[7] == 0) and np.all(np.isneginf(ml[7]))
    ref_o, ref_l, _ = O.decode_step(wl)
    U.assert_partial_close(bufs.out, bufs.lse, ref_o, ref_l, "e", 2e-2, "merged short")


def _poisoned_workload(S):
    """16 requests of 200 tokens; request 0's second page id lies outside the
    pool, so every shard's share of it reads the NaN row."""
    wl = make_workload("bad", batch=16, heads=16, q_len=1, shards=S, kv_dtype="bf16",
                       lens=("fixed", (200,) * 16), seed=9, out_dtype="bf16")
    wl.block_table[0, 1] = 10_000
    return wl


@pytest.mark.parametrize("split_target", [8, 64])
@pytest.mark.parametrize("use_metadata", [False, True])
def test_bad_page_ids_poison_out_and_lse_per_shard_and_merged(split_target, use_metadata):
    """A page id outside the pool reads as NaN instead of faulting, and the
    NaN reaches both the partial out and its LSE on every shard that owns a
    token of that page, then the merged row (a NaN LSE must not be taken for
    an empty shard). With 8 workgroups every segment is held whole by one
    workgroup (finalised in place); with 64 each is cut into pieces that the
    combine merges. The other requests match the oracle."""
    S = 2
    wl = _poisoned_workload(S)
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    bufs.fill_nan()
    ok = list(range(1, wl.batch))
    parts = []
    for r in range(S):
        _flush(f"bad page shard {r}/{S} split={split_target} meta={use_metadata}")
        if use_metadata:
            ST.run_metadata(dw, bufs, r)
        ST.run_partial(dw, bufs, r, use_metadata=use_metadata, split_target=split_target)
        torch.cuda.synchronize()
        o, l = bufs.outs[r].float().cpu().numpy(), bufs.lses[r].cpu().numpy()
        assert np.isnan(o[0]).all() and np.isnan(l[0]).all(), f"shard {r}: poisoned request not NaN"
        ref_o, ref_l = O.decode_partial(wl, r, S, wl.lse_base, requests=ok)
        parts.append((ref_o, ref_l))
        U.assert_partial_close(bufs.outs[r][ok], bufs.lses[r][ok], ref_o, ref_l, wl.lse_base, U.TOL["bf16"],
                               f"untouched requests shard {r}")
    ST.run_merge(dw, bufs)
    torch.cuda.synchronize()
    mo, ml = bufs.out.float().cpu().numpy(), bufs.lse.cpu().numpy()
    assert np.isnan(mo[0]).all() and np.isnan(ml[0]).all(), "merged poisoned request not NaN"
    ref_o, ref_l = O.merge([p_[0] for p_ in parts], [p_[1] for p_ in parts], [wl.lse_base] * S)
    U.assert_partial_close(bufs.out[ok], bufs.lse[ok], ref_o, ref_l, "e", U.TOL["bf16"], "merged untouched")


# --------------------------------------------------------------------------
# whole step: metadata -> partials -> merge
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(SMALL))
def test_step_parity(name):
    wl = _small(name)
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    bufs.fill_nan()
    _flush(f"step {name}")
    ST.run_step(dw, bufs)
    torch.cuda.synchronize()
    ref_o, ref_l, _ = O.decode_step(wl)
    U.assert_partial_close(bufs.out, bufs.lse, ref_o, ref_l, "e", U.TOL[wl.kv_dtype], f"step {name}")
    full_o, full_l = O.decode_full(wl)
    U.assert_partial_close(bufs.out, bufs.lse, full_o, full_l, "e", U.TOL[wl.kv_dtype], f"unsharded {name}")


def test_step_is_deterministic():
    wl = _small("skewed")
    dw = ST.DeviceWorkload.upload(wl)
    a, b = ST.StepBuffers(dw), ST.StepBuffers(dw)
    ST.run_step(dw, a)
    ST.run_step(dw, b)
    torch.cuda.synchronize()
    assert torch.equal(a.out.view(torch.int32), b.out.view(torch.int32))
    assert torch.equal(a.lse.view(torch.int32), b.lse.view(torch.int32))


@pytest.mark.parametrize("name", ["kimi_like", "deepseek_like_fp8", "mtp_q4", "skewed"])
def test_gather_paths_agree_bit_for_bit(name):
    """The shard-local KV indices and the block table name the same rows, and
    the owned counts and the schedule are the same, so every shard's partial
    (out, lse) and the merged result must be bit-identical between the two
    gathers (the step driver reads the block table by default)."""
    wl = _small(name)
    dw = ST.DeviceWorkload.upload(wl)
    a, b = ST.StepBuffers(dw), ST.StepBuffers(dw)
    a.fill_nan()
    b.fill_nan()
    _flush(f"gather paths {name}")
    ST.run_step(dw, a, use_metadata=True)
    ST.run_step(dw, b, use_metadata=False)
    torch.cuda.synchronize()
    for r in range(wl.shards):
        assert torch.equal(a.outs[r].view(torch.uint8), b.outs[r].view(torch.uint8)), f"out shard {r}"
        assert torch.equal(a.lses[r].view(torch.uint8), b.lses[r].view(torch.uint8)), f"lse shard {r}"
    assert torch.equal(a.out.view(torch.uint8), b.out.view(torch.uint8))
    assert torch.equal(a.lse.view(torch.uint8), b.lse.view(torch.uint8))


# --------------------------------------------------------------------------
# merge
# --------------------------------------------------------------------------
def _merge_ref(mi):
    outs = [O.decode_bf16(o) if o.dtype == np.uint16 else o.astype(np.float64) for o in mi.outs]
    return O.merge(outs, [l.astype(np.float64) for l in mi.lses], mi.bases)


@pytest.mark.parametrize("T", [1, 8, 16, 32, 64, 128])
def test_merge_bf16_parity(T):
    mi = make_merge_inputs(T, neutral_frac=0.05, seed=3000 + T)
    outs = [torch.from_numpy(o).view(torch.bfloat16).cuda() for o in mi.outs]
    lses = [torch.from_numpy(l).cuda() for l in mi.lses]
    out = torch.full((T, 64, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, 64), float("nan"), dtype=torch.float32, device="cuda")
    L.mla_merge_partials(outs, lses, [L.LSE_BASE_E] * 4, out, lse)
    torch.cuda.synchronize()
    ro, rl = _merge_ref(mi)
    go = U.to_np(out)
    # one bf16 ulp of the result plus the fp32 accumulation error, which is
    # relative to the (row, head) vector's magnitude (cancellation can leave
    # a result far smaller than its terms)
    vec = np.abs(ro).max(axis=-1, keepdims=True)
    assert np.all(np.abs(go - ro) <= U.bf16_ulp(ro) + 1e-5 * vec), "bf16 merge beyond one ulp"
    gl = U.to_np(lse)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
    assert np.all(np.abs(gl[fin] - rl[fin]) <= 1e-5 * np.maximum(1.0, np.abs(rl[fin])))


@pytest.mark.parametrize("bases", [("e", "e", "e"), ("2", "e", "2"), ("2", "2", "2")])
def test_merge_fp32_relative(bases):
    mi = make_merge_inputs(24, shards=3, heads=16, dv=512, dtype="f32", bases=bases,
                           neutral_frac=0.1, seed=77)
    outs = [torch.from_numpy(o).cuda() for o in mi.outs]
    lses = [torch.from_numpy(l).cuda() for l in mi.lses]
    code = {"e": L.LSE_BASE_E, "2": L.LSE_BASE_2}
    out = torch.full((24, 16, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((24, 16), float("nan"), dtype=torch.float32, device="cuda")
    L.mla_merge_partials(outs, lses, [code[b] for b in bases], out, lse, lse_out_base=L.LSE_BASE_2)
    torch.cuda.synchronize()
    ro, rl = _merge_ref(mi)
    go = U.to_np(out)
    scale = np.maximum(np.abs(ro).max(axis=-1, keepdims=True), 1e-30)
    assert np.all(np.abs(go - ro) <= 1e-5 * scale)
    gl = U.to_np(lse) * math.log(2)       # requested base 2
    fin = np.isfinite(rl)
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
    assert np.all(np.abs(gl[fin] - rl[fin]) <= 1e-5 * np.maximum(1.0, np.abs(rl[fin])))


def test_merge_single_shard_and_neutral_extra():
    mi = make_merge_inputs(4, shards=1, heads=8, dtype="f32", seed=5)
    o = torch.from_numpy(mi.outs[0]).cuda()
    l = torch.from_numpy(mi.lses[0]).cuda()
    out = torch.empty_like(o)
    lse = torch.empty_like(l)
    L.mla_merge_partials([o], [l], [L.LSE_BASE_E], out, lse)
    z_o = torch.zeros_like(o)
    z_l = torch.full_like(l, float("-inf"))
    out2 = torch.empty_like(o)
    lse2 = torch.empty_like(l)
    L.mla_merge_partials([o, z_o], [l, z_l], [L.LSE_BASE_E] * 2, out2, lse2)
    torch.cuda.synchronize()
    assert torch.allclose(out, o, rtol=1e-6, atol=0)
    assert torch.equal(out2, out) and torch.equal(lse2, lse)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_merge_propagates_nan(dtype):
    """A shard whose LSE is NaN (it read a poisoned KV row) poisons the merged
    vector, out and LSE, as the fp64 definition does; a NaN output element
    with a finite LSE poisons that element of the out only; all-NaN vectors stay NaN (they are not
    the neutral state). Vectors without NaN are unchanged."""
    S, T, H = 4, 6, 16
    mi = make_merge_inputs(T, shards=S, heads=H, dtype=dtype, neutral_frac=0.1, seed=91)
    lses = mi.lses.copy()
    outs = mi.outs.copy()
    lses[1, 0, 3] = np.nan                 # one shard
    lses[:, 2, 5] = np.nan                 # every shard
    lses[0, 4, 0] = -np.inf                # a neutral shard next to a NaN one
    lses[2, 4, 0] = np.nan
    nan_bits = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
    outs[3, 5, 7, 11] = nan_bits           # NaN out, finite LSE
    lses[3, 5, 7] = 9.0
    if dtype == "bf16":
        d_outs = [torch.from_numpy(outs[r]).view(torch.bfloat16).cuda() for r in range(S)]
        ref_outs = [O.decode_bf16(outs[r]) for r in range(S)]
        odt = torch.bfloat16
    else:
        d_outs = [torch.from_numpy(outs[r]).cuda() for r in range(S)]
        ref_outs = [outs[r].astype(np.float64) for r in range(S)]
        odt = torch.float32
    d_lses = [torch.from_numpy(lses[r]).cuda() for r in range(S)]
    out = torch.zeros((T, H, 512), dtype=odt, device="cuda")
    lse = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    L.mla_merge_partials(d_outs, d_lses, [L.LSE_BASE_E] * S, out, lse)
    torch.cuda.synchronize()
    ro, rl = O.merge(ref_outs, [lses[r].astype(np.float64) for r in range(S)], ["e"] * S)
    go, gl = U.to_np(out), U.to_np(lse)
    assert np.array_equal(np.isnan(go), np.isnan(ro)), "NaN pattern of out differs from the definition"
    assert np.array_equal(np.isnan(gl), np.isnan(rl)), "NaN pattern of lse differs from the definition"
    assert np.isnan(go[0, 3]).all() and np.isnan(gl[0, 3]) and np.isnan(go[2, 5]).all() and np.isnan(gl[2, 5])
    assert np.isnan(go[4, 0]).all() and np.isnan(gl[4, 0])
    assert np.isnan(go[5, 7, 11]) and np.isfinite(np.delete(go[5, 7], 11)).all() and np.isfinite(gl[5, 7])
    fin = ~np.isnan(ro)
    vec = np.abs(np.where(fin, ro, 0)).max(axis=-1, keepdims=True)
    bound = (U.bf16_ulp(ro) if dtype == "bf16" else 0) + 1e-5 * vec
    assert np.all(np.abs(go - ro)[fin] <= np.broadcast_to(bound, ro.shape)[fin])


def test_many_segments_plan_in_workspace():
    """More segments (request x 64-row block) than the schedule keeps in LDS
    (6144): 6300 short requests over 2 shards, so the plan's offset tables
    live in the workspace. Every output row must be written (NaN-prefilled
    buffers) and sampled requests must match the oracle; the reused
    schedule must give the same bytes."""
    S = 2
    wl = make_workload("many", batch=6300, heads=16, q_len=1, shards=S, kv_dtype="bf16",
                       lens=("uniform", 1, 60), seed=777, out_dtype="bf16")
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    bufs.fill_nan()
    rng = np.random.default_rng(5)
    sample = sorted(rng.choice(wl.batch, size=400, replace=False).tolist() + [0, wl.batch - 1])
    for r in range(S):
        _flush(f"many segments shard {r}/{S}")
        ST.run_metadata(dw, bufs, r)
        ST.run_partial(dw, bufs, r)
        torch.cuda.synchronize()
        assert not torch.isnan(bufs.outs[r].float()).any() and not torch.isnan(bufs.lses[r]).any()
        ref_o, ref_l = O.decode_partial(wl, r, S, wl.lse_base, requests=sample)
        U.assert_partial_close(bufs.outs[r][sample], bufs.lses[r][sample], ref_o, ref_l, wl.lse_base,
                               U.TOL["bf16"], f"many shard {r}")
        first = bufs.outs[r].clone()
        bufs.per_shard_workspaces()
        ST.run_plan(dw, bufs, r)
        ST.run_partial(dw, bufs, r, reuse_plan=True)
        torch.cuda.synchronize()
        assert torch.equal(bufs.outs[r].view(torch.int16), first.view(torch.int16))


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_zero_length_and_tiny_requests(kv_dtype):
    """Requests of length 0 (no token on any shard), 1 and 2 next to a
    longer one, q_len 2 (the first draft row of a length-1 request sees
    nothing): every such row is exactly (+0, -inf) per shard and after the
    merge, on both gather paths."""
    S = 3
    wl = make_workload("zero", batch=6, heads=16, q_len=2, shards=S, kv_dtype=kv_dtype,
                       lens=("fixed", [0, 1, 0, 65, 2, 0]), seed=3, out_dtype="bf16")
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    tol = U.TOL[kv_dtype]
    for use_metadata in (True, False):
        bufs.fill_nan()
        parts = []
        for r in range(S):
            _flush(f"zero-length {kv_dtype} meta={use_metadata} shard {r}/{S}")
            if use_metadata:
                ST.run_metadata(dw, bufs, r)
            ST.run_partial(dw, bufs, r, use_metadata=use_metadata)
            torch.cuda.synchronize()
            ref_o, ref_l = O.decode_partial(wl, r, S, wl.lse_base)
            parts.append((ref_o, ref_l))
            U.assert_partial_close(bufs.outs[r], bufs.lses[r], ref_o, ref_l, wl.lse_base, tol, f"zero shard {r}")
        ST.run_merge(dw, bufs)
        torch.cuda.synchronize()
        full_o, full_l = O.decode_full(wl)
        U.assert_partial_close(bufs.out, bufs.lse, full_o, full_l, "e", tol, "zero merged")


# --------------------------------------------------------------------------
# split query: q_nope and q_rope read in place
# --------------------------------------------------------------------------
@pytest.mark.parametrize("layout", ["slices_of_one_buffer", "separate_tensors"])
@pytest.mark.parametrize("name", ["kimi_like", "deepseek_like_fp8", "mtp_q4"])
def test_split_query_matches_concatenated(name, layout):
    """The query given as its 512 latent dims and its 64 rope dims, each read
    in place with its own row stride (no concatenation pass), gives the same
    bytes as the concatenated [.., 576] query, per shard and in the single
    launch of every shard, and matches the oracle."""
    wl = _small(name)
    dw = ST.DeviceWorkload.upload(wl)
    B, q, H = wl.batch, wl.q_len, wl.heads
    if layout == "slices_of_one_buffer":
        # rows of 704 elements: [pad 64 | rope 64 | pad 32 | nope 512 | pad 32]
        buf = torch.full((B, q, H, 704), float("nan"), dtype=torch.bfloat16, device="cuda")
        buf[..., 64:128] = dw.q[..., 512:]
        buf[..., 160:672] = dw.q[..., :512]
        q_nope, q_rope = buf[..., 160:672], buf[..., 64:128]
    else:
        q_nope, q_rope = dw.q[..., :512].contiguous(), dw.q[..., 512:].contiguous()
    ref = ST.StepBuffers(dw)
    got = ST.StepBuffers(dw)
    tol = U.TOL[wl.kv_dtype]
    for r in range(wl.shards):
        _flush(f"split query {name} {layout} shard {r}/{wl.shards}")
        ST.run_metadata(dw, ref, r)
        ST.run_metadata(dw, got, r)
        ST.run_partial(dw, ref, r)
        L.mla_decode_partial(q_nope, dw.kv_pages, dw.block_table, dw.seq_lens, r, wl.shards, q,
                             got.outs[r], got.lses[r], got.workspace, kv_scale=dw.kv_scale,
                             softmax_scale=dw.softmax_scale, lse_base=dw.lse_base,
                             local_seq_lens=got.local_seq_lens[r], local_kv_indices=got.local_kv_indices[r],
                             q_rope=q_rope)
        torch.cuda.synchronize()
        assert torch.equal(got.outs[r].view(torch.int16 if got.outs[r].dtype == torch.bfloat16 else torch.int32),
                           ref.outs[r].view(torch.int16 if ref.outs[r].dtype == torch.bfloat16 else torch.int32))
        assert torch.equal(got.lses[r].view(torch.int32), ref.lses[r].view(torch.int32))
        ref_o, ref_l = O.decode_partial(wl, r, wl.shards, wl.lse_base)
        U.assert_partial_close(got.outs[r], got.lses[r], ref_o, ref_l, wl.lse_base, tol, f"split q shard {r}")
    ws = ST.all_shards_workspace(dw, got)
    got.fill_nan()
    L.mla_decode_all_shards(q_nope, dw.kv_pages, dw.block_table, dw.seq_lens, wl.shards, q, got.out, got.lse, ws,
                            kv_scale=dw.kv_scale, softmax_scale=dw.softmax_scale, q_rope=q_rope)
    torch.cuda.synchronize()
    full_o, full_l = O.decode_full(wl)
    U.assert_partial_close(got.out, got.lse, full_o, full_l, "e", tol, f"split q all shards {name}")
