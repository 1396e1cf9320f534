"""The allocation-free decode (mla_decode_partial_noalloc, scratch held by
the library) against the workspace decode (mla_decode_partial) through the
C ABI: the same bytes, and within the oracle's tolerance, on two calls in a
row on one device, the second with a smaller input (the scratch keeps the
first call's contents, which must not leak into the second); the fp8 call
also from e4m3 query codes."""
import dataclasses

import pytest
import torch

import gpu_util as U
from oracle import mla_oracle as O
from workloads import make_config

pytestmark = pytest.mark.gpu

if U.gpu_available():
    from decode_attention_paged_amd import _lib as L
    from decode_attention_paged_amd import step as ST


def _noalloc(dw, bufs, r, use_metadata):
    q, q_scale = dw.query()
    return L.mla_decode_partial_noalloc(
        q, dw.kv_pages, dw.block_table, dw.seq_lens, r, dw.shards, dw.q_len, bufs.outs[r], bufs.lses[r],
        kv_scale=dw.kv_scale, softmax_scale=dw.softmax_scale, lse_base=dw.lse_base,
        local_seq_lens=bufs.local_seq_lens[r] if use_metadata else None,
        local_kv_indices=bufs.local_kv_indices[r] if use_metadata else None, q_lens=dw.q_lens,
        q_scale=q_scale)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("use_metadata,e4m3_query", [(True, False), (False, False), (False, True)])
def test_noalloc_matches_workspace_decode_twice(use_metadata, e4m3_query):
    big = make_config(3, batch=4, lens=("uniform", 1500, 2500))                 # fp8, 128 heads, 8 shards
    small = make_config(2, batch=3, lens=("uniform", 100, 300))                 # bf16, 64 heads, 4 shards
    if e4m3_query:                                                             # the fp8 call from e4m3 query codes
        big = dataclasses.replace(big, q_codes=O.quantize_query(big.q, 0.25), q_scale=0.25)
    for n, wl in enumerate((big, small)):
        dw = ST.DeviceWorkload.upload(wl)
        ref, got = ST.StepBuffers(dw), ST.StepBuffers(dw)
        got.fill_nan()
        tol = U.TOL[wl.kv_dtype]
        for r in range(wl.shards):
            print(f"noalloc call {n} {wl.name} shard {r}/{wl.shards} meta={use_metadata} e4m3={e4m3_query}",
                  flush=True)
            if use_metadata:
                ST.run_metadata(dw, ref, r)
                ST.run_metadata(dw, got, r)
            ST.run_partial(dw, ref, r, use_metadata=use_metadata)
            base = _noalloc(dw, got, r, use_metadata)
            torch.cuda.synchronize()
            assert base == dw.lse_base
            assert torch.equal(_bits(got.outs[r]), _bits(ref.outs[r])), f"call {n} shard {r}: out differs"
            assert torch.equal(_bits(got.lses[r]), _bits(ref.lses[r])), f"call {n} shard {r}: lse differs"
            ref_o, ref_l = O.decode_partial(wl, r, wl.shards, wl.lse_base)
            U.assert_partial_close(got.outs[r], got.lses[r], ref_o, ref_l, wl.lse_base, tol, f"noalloc {n} shard {r}")


def test_noalloc_rejects_what_does_not_fit():
    wl = make_config(2, batch=2, lens=("uniform", 100, 200))
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    with pytest.raises(L.MlaError) as e:
        L.mla_decode_partial_noalloc(dw.q, dw.kv_pages, dw.block_table, dw.seq_lens, 0, dw.shards, dw.q_len,
                                     bufs.outs[0], bufs.lses[0], softmax_scale=dw.softmax_scale, split_target=1024)
    assert e.value.status == L.STATUS_WORKSPACE_TOO_SMALL and "scratch" in str(e.value)
