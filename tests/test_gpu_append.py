"""GPU parity of the KV append (mla_append_kv through the C ABI) against the
oracle, bit for bit on the whole pool: only the owning shard writes a new
token's row, bf16 rows are copied, fp8 rows are quantised exactly as the
oracle's nearest-value encoder does (ties to even, saturation at 448, signed
NaN); rows of skipped tokens (before the request start, past the table, page
ids outside the pool) and every other row stay untouched. Then an end-to-end
check: a pool whose newest rows are poisoned, repaired by the append on each
owner, decodes like the original workload.
"""
import numpy as np
import pytest
import torch

import gpu_util as U
from oracle import mla_oracle as O
from workloads import make_append_inputs, make_workload

pytestmark = pytest.mark.gpu

if U.gpu_available():
    from decode_attention_paged_amd import _lib as L
    from decode_attention_paged_amd import step as ST


def _e4m3_midpoints():
    """Every midpoint between neighbouring positive e4m3 values (exact in
    bf16: at most 5 significant bits)."""
    v = O.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    return (v[:-1] + v[1:]) / 2


def _run(inp, shard, S):
    dev = torch.device("cuda")
    if inp.kv_dtype == "bf16":
        pool = torch.from_numpy(inp.kv_pages.view(np.int16).copy()).to(dev).view(torch.bfloat16)
    else:
        pool = torch.from_numpy(inp.kv_pages.copy()).to(dev)
    k_nope = torch.from_numpy(inp.k_nope.view(np.int16)).to(dev).view(torch.bfloat16)
    k_rope = torch.from_numpy(inp.k_rope.view(np.int16)).to(dev).view(torch.bfloat16)
    lens = torch.from_numpy(inp.seq_lens).to(dev)
    bt = torch.from_numpy(inp.block_table).to(dev)
    L.mla_append_kv(k_nope, k_rope, lens, bt, pool, shard, S, kv_scale=inp.kv_scale)
    torch.cuda.synchronize()
    if inp.kv_dtype == "bf16":
        return pool.view(torch.int16).cpu().numpy().view(np.uint16)
    return pool.cpu().numpy()


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("S,n_new", [(1, 1), (3, 1), (4, 1), (8, 1), (1, 4), (4, 4), (2, 3)])
def test_append_matches_oracle_bit_exact(kv_dtype, S, n_new):
    print(f"append {kv_dtype} S={S} n_new={n_new}", flush=True)
    special = [np.nan, -np.nan, np.inf, -np.inf, 1e4, -1e4, 0.0, -0.0, 1e-38, 3e-39]
    inp = make_append_inputs(batch=40, n_new=n_new, kv_dtype=kv_dtype, kv_scale=0.3711, seed=100 + 7 * S + n_new,
                             special=special)
    for r in range(S):
        got = _run(inp, r, S)
        ref = O.append_kv(inp.kv_pages, inp.k_nope, inp.k_rope, inp.seq_lens, inp.block_table, r, S, kv_dtype,
                          inp.kv_scale)
        assert np.array_equal(got, ref), f"shard {r}: {int((got != ref).any(axis=-1).sum())} rows differ"


def test_append_fp8_rounding_at_every_midpoint():
    """kv_scale 0.5 makes the division exact, so every planted value lands on
    an exact e4m3 midpoint (or the saturation boundary) and the tie rule
    decides the code."""
    print("append fp8 midpoints", flush=True)
    mids = _e4m3_midpoints()
    special = np.concatenate([mids, -mids, [448.0, 464.0, 480.0, 1e6]]) * 0.5
    inp = make_append_inputs(batch=40, n_new=4, kv_dtype="fp8", kv_scale=0.5, seed=77, special=special)
    assert np.isin(O.decode_bf16(inp.k_nope).ravel(), special).sum() > 100
    got = _run(inp, 0, 1)
    ref = O.append_kv(inp.kv_pages, inp.k_nope, inp.k_rope, inp.seq_lens, inp.block_table, 0, 1, "fp8", 0.5)
    assert np.array_equal(got, ref)


def test_append_then_decode_matches_the_original_workload():
    """The newest token's row of every request is poisoned with NaN, then
    appended back by its owning shard; every shard's decode must match the
    oracle on the original workload (bf16 KV: the append restores the bytes)."""
    print("append then decode", flush=True)
    wl = make_workload("append_e2e", batch=5, heads=16, q_len=1, shards=4, kv_dtype="bf16",
                       lens=("uniform", 60, 300), seed=515)
    B = wl.batch
    rows = np.zeros((B, 1, 576), dtype=np.uint16)
    poisoned = wl.kv_pages.copy()
    for b in range(B):
        t = int(wl.seq_lens[b]) - 1
        page = int(wl.block_table[b, t // 64])
        rows[b, 0] = wl.kv_pages[page, t % 64]
        poisoned[page, t % 64] = 0x7FC0                    # bf16 NaN
    dev = torch.device("cuda")
    pool = torch.from_numpy(poisoned.view(np.int16)).to(dev).view(torch.bfloat16)
    k_nope = torch.from_numpy(rows[..., :512].copy().view(np.int16)).to(dev).view(torch.bfloat16)
    k_rope = torch.from_numpy(rows[..., 512:].copy().view(np.int16)).to(dev).view(torch.bfloat16)
    lens = torch.from_numpy(wl.seq_lens).to(dev)
    bt = torch.from_numpy(wl.block_table).to(dev)
    for r in range(wl.shards):
        L.mla_append_kv(k_nope, k_rope, lens, bt, pool, r, wl.shards)
    torch.cuda.synchronize()
    assert np.array_equal(pool.view(torch.int16).cpu().numpy().view(np.uint16), wl.kv_pages)
    d = ST.DeviceWorkload.upload(wl)
    d.kv_pages.copy_(pool)
    bufs = ST.StepBuffers(d)
    for r in range(wl.shards):
        ST.run_metadata(d, bufs, r)
        ST.run_partial(d, bufs, r)
    torch.cuda.synchronize()
    for r in range(wl.shards):
        ref_o, ref_l = O.decode_partial(wl, r, wl.shards, wl.lse_base)
        U.assert_partial_close(bufs.outs[r], bufs.lses[r], ref_o, ref_l, wl.lse_base, U.TOL["bf16"], f"shard {r}")


def test_append_in_a_graph_matches_eager_on_every_replay():
    """The append captured in a HIP graph (all shards' calls), replayed three
    times on fresh pool contents with eager work and synchronisation in
    between, writes the same pool as the eager calls each time."""
    print("append graph replays", flush=True)
    S = 4
    inp = make_append_inputs(batch=32, n_new=2, kv_dtype="fp8", kv_scale=0.29, seed=91,
                             special=[np.nan, np.inf, 1e4])
    dev = torch.device("cuda")
    pool0 = torch.from_numpy(inp.kv_pages.copy()).to(dev)
    pool = pool0.clone()
    k_nope = torch.from_numpy(inp.k_nope.view(np.int16)).to(dev).view(torch.bfloat16)
    k_rope = torch.from_numpy(inp.k_rope.view(np.int16)).to(dev).view(torch.bfloat16)
    lens = torch.from_numpy(inp.seq_lens).to(dev)
    bt = torch.from_numpy(inp.block_table).to(dev)
    for r in range(S):
        L.mla_append_kv(k_nope, k_rope, lens, bt, pool, r, S, kv_scale=inp.kv_scale)
    torch.cuda.synchronize()
    eager = pool.cpu().numpy()
    ref = inp.kv_pages
    for r in range(S):
        ref = O.append_kv(ref, inp.k_nope, inp.k_rope, inp.seq_lens, inp.block_table, r, S, "fp8", inp.kv_scale)
    assert np.array_equal(eager, ref)
    pool.copy_(pool0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for r in range(S):
            L.mla_append_kv(k_nope, k_rope, lens, bt, pool, r, S, kv_scale=inp.kv_scale)
    torch.cuda.synchronize()
    for rep in range(3):
        pool.copy_(pool0)
        scratch = torch.randn(1 << 16, device=dev).sum()     # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(pool.cpu().numpy(), eager), f"replay {rep}"
        del scratch
