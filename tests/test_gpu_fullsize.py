"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark times (shard metadata on, default split schedule).

The oracle evaluates only sampled requests (all shards and the merge for
each), which covers the longest request, a short one and the first one.
"""
import numpy as np
import pytest
import torch

import gpu_util as U
from oracle import mla_oracle as O
from workloads import make_config

pytestmark = pytest.mark.gpu

if U.gpu_available():
    from decode_attention_paged_amd import step as ST


def _samples(wl):
    lens = wl.seq_lens
    picks = {0, int(np.argmax(lens)), int(np.argmin(lens)), int(np.argsort(lens)[len(lens) // 2])}
    return sorted(picks)


@pytest.mark.parametrize("index", [1, 2, 3, 4, 5])
def test_fullsize_sampled(index):
    print(f"full-size config {index}: generating", flush=True)
    wl = make_config(index)
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    bufs.fill_nan()
    print(f"full-size config {index}: running step B={wl.batch} H={wl.heads} S={wl.shards}", flush=True)
    ST.run_step(dw, bufs)
    torch.cuda.synchronize()
    reqs = _samples(wl)
    tol = U.TOL[wl.kv_dtype]
    for r in range(wl.shards):
        ref_o, ref_l = O.decode_partial(wl, r, wl.shards, wl.lse_base, reqs)
        U.assert_partial_close(bufs.outs[r][reqs], bufs.lses[r][reqs], ref_o, ref_l, wl.lse_base, tol,
                               f"config {index} shard {r} requests {reqs}")
    ref_o, ref_l, _ = O.decode_step(wl, reqs)
    U.assert_partial_close(bufs.out[reqs], bufs.lse[reqs], ref_o, ref_l, "e", tol,
                           f"config {index} merged requests {reqs}")
    # every row of every request was written and is finite or neutral
    lse = bufs.lse.cpu().numpy()
    assert not np.isnan(lse).any() and not np.isnan(bufs.out.float().cpu().numpy()).any()
