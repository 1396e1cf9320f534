"""Host-side checks of bench.py (no GPU): the one-GPU refusal, the
algorithmic work it divides by, the choice of the binding roof, and the
JSON line's contract assembled from synthetic results."""
import argparse
import json
import math
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import make_config  # noqa: E402


def _run(*args):
    env = dict(os.environ, HIP_VISIBLE_DEVICES="")
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, env=env, timeout=300)


def test_more_than_one_gpu_is_refused_with_a_message():
    res = _run("--gpus", "2")
    assert res.returncode == 2
    assert "one GPU" in res.stderr and "Traceback" not in res.stderr


def test_without_a_gpu_it_exits_with_a_message():
    res = _run("--steps", "1", "--warmup", "0")
    if "needs a GPU" not in res.stderr:
        pytest.skip("a GPU is visible here")
    assert res.returncode == 2 and "Traceback" not in res.stderr


def test_workload_work_matches_closed_forms():
    # q_len 1: every owned token is visible; the shards' KV bytes add up to
    # the step's, and each launch also counts the queries, out and LSE
    wl = make_config(2, batch=5, lens=("uniform", 100, 300))
    kv, flops, per_shard = bench.workload_work(wl)
    L = wl.seq_lens.astype(np.int64)
    assert kv == int(L.sum()) * 1152
    assert flops == pytest.approx(2.0 * wl.heads * 1088 * float(L.sum()))
    rows = wl.batch * wl.heads
    extra = rows * 576 * 2 + rows * 512 * 2 + rows * 4
    assert sum(b for b, _ in per_shard) == kv + wl.shards * extra
    assert sum(f for _, f in per_shard) == pytest.approx(flops)
    # q_len 4: draft row i sees L - 3 + i tokens (per-shard counts by the
    # owner rule sum to the same)
    wl4 = make_config(4, batch=3, lens=("uniform", 50, 90), shards=2)
    _, f4, ps4 = bench.workload_work(wl4)
    vis = sum(int(Lb) - 3 + i for Lb in wl4.seq_lens for i in range(4))
    assert f4 == pytest.approx(2.0 * wl4.heads * 1088 * vis)
    assert sum(f for _, f in ps4) == pytest.approx(f4)


def test_the_binding_roof_is_the_larger_fraction():
    hbm = dict(attn_kernel_mfma_frac=0.1, attn_kernel_hbm_frac=0.4, attn_kernel_gbs=3200.0,
               attn_kernel_tflops=250.0)
    mfma = dict(hbm, attn_kernel_mfma_frac=0.3, attn_kernel_hbm_frac=0.1)
    a, b = bench.binding_roof(hbm), bench.binding_roof(mfma)
    assert a["bound"] == "hbm" and a["peak"] == 8000.0 and a["frac"] == pytest.approx(0.4)
    assert b["bound"] == "mfma" and b["peak"] == 2500.0 and b["unit"] == "TFLOP/s"


def _synthetic_result(name="kimi_like"):
    return dict(index=2, name=name, batch=64, heads=64, q_len=1, shards=4, kv_dtype="bf16", lse_base="e",
                tokens=386546, ms_per_step=0.16, kv_gbs=2780.0, tflops=333.0, attn_kernel_mean_us=32.3,
                attn_kernel_bytes_per_launch=120254528.0, attn_kernel_gbs=3720.0, attn_kernel_tflops=130.0,
                merge_us=7.4, merge_bytes=21053440, merge_gbs=2840.0, merge_hbm_frac=0.355, steps=20, warmup=5,
                rotated=2, metadata_us_per_shard=13.0, plan_us_per_shard=15.0, step_timing="graph replay",
                eager_ms_per_step=0.2, attn_kernel_hbm_frac=0.465, attn_kernel_mfma_frac=0.052,
                all_shards=dict(ms_per_step=0.106, kv_gbs=4200.0, attn_kernel_us=94.0, call_bytes=454000000,
                                attn_kernel_hbm_frac=0.6, attn_kernel_mfma_frac=0.23, step_timing="graph replay"))


def test_the_json_line_keeps_the_contract():
    args = argparse.Namespace(steps=20, warmup=5)
    wl = make_config(2, batch=4, lens=("uniform", 100, 200))
    res = _synthetic_result()
    per_config = {"kimi_like": bench.config_summary(res)}
    merge = {str(T): dict(us_median=3.0 + T / 20, kernel_us_mean=4.0 + T / 20, kernel_gbs=1000.0 + T)
             for T in (1, 8, 16, 32, 64, 128)}
    cpu = dict(value=0.05, unit="GB/s", cores=16, kind="oracle", sample="first 1 of 4 requests")
    hbm = dict(gbs=5100.0, copy_gbs=5100.0, read_gbs=4000.0)
    line = bench.assemble_line(args, wl, res, merge, {"bf16 B64 S4": 2.1}, per_config, cpu, hbm)
    text = json.dumps(line)                          # serialisable, one line
    assert "\n" not in text
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in line, k
    assert line["metric"] == bench.METRIC and line["unit"] == "GB/s"
    assert line["n_gpus"] == 1 and line["higher_is_better"] is True and line["vs_baseline"] is None
    assert line["value"] == pytest.approx(res["kv_gbs"]) and line["ms_per_step"] == pytest.approx(0.16)
    assert isinstance(line["config"]["workload"], str) and "model" not in line["config"]
    roof = line["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    assert roof["bound"] == "hbm" and roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"])
    assert roof["traffic"] is None or roof["traffic"] > 0
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in line["cpu_baseline"], k
    assert line["cpu_baseline"]["kind"] == "oracle"
    assert math.isclose(line["merge_roofline"]["frac"], (1000.0 + 128) / 8000.0, rel_tol=1e-3)
