"""A decode step captured as one HIP graph (shard partials on concurrent
streams, joined for the merge) replays to the eager step's exact bytes.

The graph is replayed several times with the program's own eager work and
synchronisations in between, and every replay is compared with the eager
result (the kernels are deterministic, so the comparison is bit for bit).
"""
import pytest

pytestmark = pytest.mark.gpu


def test_graph_step_matches_eager():
    import torch
    from decode_attention_paged_amd import step as ST
    from workloads import make_workload

    wl = make_workload("graph", batch=6, heads=64, q_len=1, shards=4, kv_dtype="bf16",
                       lens=("uniform", 1, 3000), seed=11, out_dtype="bf16")
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    for r in range(wl.shards):
        ST.run_metadata(dw, bufs, r)
    # eager reference
    bufs.fill_nan()
    for r in range(wl.shards):
        ST.run_partial(dw, bufs, r)
    ST.run_merge(dw, bufs)
    torch.cuda.synchronize()
    ref_out, ref_lse = bufs.out.clone(), bufs.lse.clone()
    assert not torch.isnan(ref_out).any()

    streams = [torch.cuda.Stream() for _ in range(wl.shards)]
    ST.run_step_concurrent(dw, bufs, streams)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ST.run_step_concurrent(dw, bufs, streams)
    for rep in range(3):
        bufs.fill_nan()
        # unrelated eager work between replays
        x = torch.randn(1 << 16, device="cuda")
        (x * 2).sum().item()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs.out.view(torch.uint8), ref_out.view(torch.uint8)), rep
        assert torch.equal(bufs.lse.view(torch.uint8), ref_lse.view(torch.uint8)), rep
