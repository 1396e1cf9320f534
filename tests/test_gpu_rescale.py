"""GPU parity on inputs that force the online-softmax rescale: keys planted
in owned tiles 2 and 5 of every shard raise each row's tile maximum far
above the first tile's (tests/test_rescale_inputs.py checks on the CPU that
most rows move their reference at least twice, some by more than 16 log2
units). Every shard through both gather paths and with the segments whole
or cut into pieces, the merged step, and the single launch of every shard,
against the oracle element by element (2e-2 bf16 KV, 6e-2 fp8 KV)."""
import pytest
import torch

import gpu_util as U
import rescale_util as R
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu

if U.gpu_available():
    from decode_attention_paged_amd import step as ST


def _flush(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("split_target", [0, 7, 64])
@pytest.mark.parametrize("name", sorted(R.SPECS))
def test_rescale_per_shard_and_merged(name, split_target):
    wl = R.rising_workload(name)
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    tol = U.TOL[wl.kv_dtype]
    refs = [O.decode_partial(wl, r, wl.shards, wl.lse_base) for r in range(wl.shards)]
    for use_metadata in (True, False):
        bufs.fill_nan()
        for r in range(wl.shards):
            _flush(f"rescale {name} split={split_target} meta={use_metadata} shard {r}/{wl.shards}")
            if use_metadata:
                ST.run_metadata(dw, bufs, r)
            ST.run_partial(dw, bufs, r, use_metadata=use_metadata, split_target=split_target)
            torch.cuda.synchronize()
            U.assert_partial_close(bufs.outs[r], bufs.lses[r], refs[r][0], refs[r][1], wl.lse_base, tol,
                                   f"rescale {name} shard {r}")
        ST.run_merge(dw, bufs)
        torch.cuda.synchronize()
        mo, ml = O.merge([p[0] for p in refs], [p[1] for p in refs], [wl.lse_base] * wl.shards)
        U.assert_partial_close(bufs.out, bufs.lse, mo, ml, "e", tol, f"rescale {name} merged")


@pytest.mark.parametrize("split_target", [0, 7, 64])
@pytest.mark.parametrize("name", sorted(R.SPECS))
def test_rescale_all_shards(name, split_target):
    wl = R.rising_workload(name)
    dw = ST.DeviceWorkload.upload(wl)
    bufs = ST.StepBuffers(dw)
    bufs.fill_nan()
    _flush(f"rescale all shards {name} split={split_target}")
    ST.run_all_shards(dw, bufs, split_target=split_target)
    torch.cuda.synchronize()
    full_o, full_l = O.decode_full(wl)
    U.assert_partial_close(bufs.out, bufs.lse, full_o, full_l, "e", U.TOL[wl.kv_dtype], f"rescale all {name}")
