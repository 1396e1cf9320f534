"""Pins of the oracle's e4m3 query path ([DCP decode] 实现拆解 step 3: with an
fp8 KV pool the query is prepared by a fused concat-and-quantise).

* the codes of a query that lies on the e4m3 grid (times the scale) are
  exactly those grid codes;
* in range, the codes equal a library cast of the fp32 quotient (torch's
  float8_e4m3fn, round to nearest even);
* decoding with grid codes and their scale equals decoding with the same
  values as a bf16 query (the fp64 query rows are identical), so a wrong
  scale, decode or row order in the fp8 query path fails;
* with codes present the decode reads them and not the bf16 query.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from workloads import make_config


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 values that bf16 holds exactly -> their bf16 patterns."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def _grid_codes(rng, shape):
    """Random finite e4m3 codes of both signs (no NaN)."""
    mag = rng.integers(0, 0x7F, size=shape)          # 0x00 .. 0x7E
    sign = rng.integers(0, 2, size=shape) << 7
    return (mag | sign).astype(np.uint8)


@pytest.mark.parametrize("q_scale", [0.25, 1.0, 2.0 ** -5])
def test_grid_query_codes_round_trip(q_scale):
    rng = np.random.default_rng(11)
    codes = _grid_codes(rng, (3, 1, 16, 576))
    vals = O.decode_e4m3(codes) * q_scale                 # powers-of-two scale: exact in bf16
    bits = _bf16_bits(vals.astype(np.float32))
    got = O.quantize_query(bits, q_scale)
    # +0 and -0 keep their codes; every other value its grid code
    assert np.array_equal(got, codes)


def test_query_codes_match_torch_cast_in_range():
    rng = np.random.default_rng(12)
    q = (rng.standard_normal((2, 4, 32, 576)) * 3.0).astype(np.float32)
    bits = (q.view(np.uint32) >> 16).astype(np.uint16)    # truncate to bf16 patterns
    q_scale = 0.37
    x = O.decode_bf16(bits).astype(np.float32) / np.float32(q_scale)
    assert np.abs(x).max() < 448.0
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.quantize_query(bits, q_scale), ref)


def _small_fp8(**kw):
    return make_config(3, batch=2, lens=("uniform", 40, 300), **kw)


def test_decode_with_grid_codes_equals_bf16_query():
    wl = _small_fp8()
    rng = np.random.default_rng(13)
    q_scale = 0.125
    # small codes (|value| <= 8 * q_scale) keep the scores moderate
    mag = rng.integers(0, 0x50, size=wl.q.shape)
    codes = (mag | (rng.integers(0, 2, size=wl.q.shape) << 7)).astype(np.uint8)
    bits = _bf16_bits((O.decode_e4m3(codes) * q_scale).astype(np.float32))
    wl_b = dataclasses.replace(wl, q=bits)
    wl_q = dataclasses.replace(wl, q=bits, q_codes=codes, q_scale=q_scale)
    for r in range(wl.shards):
        ob, lb = O.decode_partial(wl_b, r, wl.shards, wl.lse_base)
        oq, lq = O.decode_partial(wl_q, r, wl.shards, wl.lse_base)
        assert np.array_equal(ob, oq) and np.array_equal(lb, lq)
    # and a wrong scale is seen
    wl_w = dataclasses.replace(wl_q, q_scale=2 * q_scale)
    ow, _ = O.decode_partial(wl_w, 0, wl.shards, wl.lse_base)
    ob, _ = O.decode_partial(wl_b, 0, wl.shards, wl.lse_base)
    assert np.abs(ow - ob).max() > 1e-3


def test_decode_reads_the_codes_not_the_bf16_query():
    """With codes present, the bf16 query bits play no part: scrambling them
    leaves the decode unchanged, and changing one code changes its row."""
    wl = _small_fp8()
    codes = O.quantize_query(wl.q, 1.0)
    wl_q = dataclasses.replace(wl, q_codes=codes, q_scale=1.0)
    wl_s = dataclasses.replace(wl_q, q=np.zeros_like(wl.q))
    o1, l1 = O.decode_partial(wl_q, 0, wl.shards, "e")
    o2, l2 = O.decode_partial(wl_s, 0, wl.shards, "e")
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    c2 = codes.copy()
    c2[0, 0, 5, 7] ^= 0x08                               # one exponent bit of one element
    o3, l3 = O.decode_partial(dataclasses.replace(wl_q, q_codes=c2), 0, wl.shards, "e")
    diff = np.abs(l3 - l1)
    diff[~np.isfinite(diff)] = 0.0
    assert diff[0, 0, 5] > 0 and np.count_nonzero(diff) == 1
