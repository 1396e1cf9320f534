"""A schedule built once by mla_decode_plan and reused by several partial
decodes (as every layer of a decode step would) gives the exact bytes of
partial decodes that build their own schedule, for both KV types, a workload
whose requests are cut into pieces across workgroups, and a graph-captured
step that reuses the schedules.
"""
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv_dtype,heads,q_len,shards,split", [
    ("bf16", 64, 1, 4, 0), ("fp8", 128, 1, 2, 37), ("bf16", 32, 4, 1, 0), ("bf16", 16, 1, 3, 5)])
def test_reused_plan_matches_fresh_plan(kv_dtype, heads, q_len, shards, split):
    import torch
    from decode_attention_paged_amd import step as ST
    from workloads import make_workload

    wl = make_workload("plan", batch=5, heads=heads, q_len=q_len, shards=shards, kv_dtype=kv_dtype,
                       lens=("uniform", 1, 4000), seed=23, out_dtype="bf16")
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    bufs.per_shard_workspaces()
    for r in range(shards):
        ST.run_metadata(dw, bufs, r)
    bufs.fill_nan()
    for r in range(shards):
        ST.run_partial(dw, bufs, r, split_target=split)
    torch.cuda.synchronize()
    ref = [(o.clone(), l.clone()) for o, l in zip(bufs.outs, bufs.lses)]
    assert not any(torch.isnan(o).all() for o, _ in ref)

    for r in range(shards):
        ST.run_plan(dw, bufs, r, split_target=split)
    for layer in range(3):
        bufs.fill_nan()
        for r in range(shards):
            ST.run_partial(dw, bufs, r, split_target=split, reuse_plan=True)
        torch.cuda.synchronize()
        for r in range(shards):
            assert torch.equal(bufs.outs[r].view(torch.uint8), ref[r][0].view(torch.uint8)), (layer, r)
            assert torch.equal(bufs.lses[r].view(torch.uint8), ref[r][1].view(torch.uint8)), (layer, r)


def test_graph_step_with_reused_plans():
    import torch
    from decode_attention_paged_amd import step as ST
    from workloads import make_workload

    wl = make_workload("plan_graph", batch=6, heads=64, q_len=1, shards=4, kv_dtype="bf16",
                       lens=("uniform", 1, 3000), seed=12, out_dtype="bf16")
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    bufs.per_shard_workspaces()
    for r in range(wl.shards):
        ST.run_metadata(dw, bufs, r)
    bufs.fill_nan()
    for r in range(wl.shards):
        ST.run_partial(dw, bufs, r)
    ST.run_merge(dw, bufs)
    torch.cuda.synchronize()
    ref_out, ref_lse = bufs.out.clone(), bufs.lse.clone()

    for r in range(wl.shards):
        ST.run_plan(dw, bufs, r)
    streams = [torch.cuda.Stream() for _ in range(wl.shards)]
    ST.run_step_concurrent(dw, bufs, streams, reuse_plan=True)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ST.run_step_concurrent(dw, bufs, streams, reuse_plan=True)
    for rep in range(3):
        bufs.fill_nan()
        x = torch.randn(1 << 16, device="cuda")
        (x * 2).sum().item()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs.out.view(torch.uint8), ref_out.view(torch.uint8)), rep
        assert torch.equal(bufs.lse.view(torch.uint8), ref_lse.view(torch.uint8)), rep
