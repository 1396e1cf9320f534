"""Input generator: determinism, structure of the page pool, encoders (CPU)."""
import collections
import math

import numpy as np

from oracle import mla_oracle as O
from workloads import (CONFIGS, f32_to_bf16_bits, f32_to_e4m3_bits, make_config,
                       make_merge_inputs, make_workload)


def test_deterministic_and_seed_sensitive():
    a = make_config(1)
    b = make_config(1)
    for f in ("seq_lens", "block_table", "kv_pages", "q"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = make_config(1, seed=99)
    assert not np.array_equal(a.q, c.q)


def test_page_pool_is_a_permutation_with_poisoned_tails():
    wl = make_config(2, batch=6)
    used = []
    for b, L in enumerate(wl.seq_lens):
        n = (int(L) + 63) // 64
        assert (wl.block_table[b, n:] == -1).all()
        used += wl.block_table[b, :n].tolist()
        if L % 64:
            tail = wl.kv_pages[wl.block_table[b, n - 1], L % 64:]
            assert np.isnan(O.decode_bf16(tail)).all()
        head = wl.kv_pages[wl.block_table[b, (int(L) - 1) // 64], (int(L) - 1) % 64]
        assert np.isfinite(O.decode_bf16(head)).all()
    assert sorted(used) == list(range(wl.num_pages))
    assert (4096 <= wl.seq_lens).all() and (wl.seq_lens <= 8192).all()


def test_skewed_lengths_have_short_requests():
    wl = make_config(5, lens=("skewed", 1, 4096), batch=40)
    short = collections.Counter(int(L) for L in wl.seq_lens if L < 8)
    # the eight forced short lengths are present (the log-uniform draw may add more)
    assert not (collections.Counter([1, 1, 2, 3, 4, 5, 6, 7]) - short)
    assert (wl.seq_lens >= 1).all() and (wl.seq_lens <= 4096).all()


def test_fp8_workload_scale_and_range():
    wl = make_config(3, batch=2, lens=("uniform", 100, 300))
    vals = O.decode_e4m3(wl.kv_pages)
    fin = vals[np.isfinite(vals)]
    assert np.abs(fin).max() == 448.0          # amax maps exactly to the top code
    assert 0.005 < wl.kv_scale < 0.02          # amax of N(0,1) draws / 448


def test_bf16_encoder_rounds_to_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 1e-40], np.float32)
    got = f32_to_bf16_bits(x)
    assert got.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, f32_to_bf16_bits(np.float32([1e-40]))[0]]
    rng = np.random.default_rng(1)
    y = rng.standard_normal(10000).astype(np.float32)
    back = O.decode_bf16(f32_to_bf16_bits(y))
    assert np.all(np.abs(back - y) <= np.abs(y) * 2.0 ** -8)


def _e4m3_nearest_even(v):
    """Exhaustive search over the 127 non-negative finite codes."""
    vals = O.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    a = abs(float(v))
    if a > 448.0:
        c = 0x7E
    else:
        d = np.abs(vals - a)
        cands = np.nonzero(d == d.min())[0]
        c = int(cands[0]) if len(cands) == 1 else int([k for k in cands if k % 2 == 0][0])
    return c | (0x80 if math.copysign(1.0, float(v)) < 0 else 0)


def test_e4m3_encoder_matches_exhaustive_search():
    rng = np.random.default_rng(0)
    vals = O.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    x = np.concatenate([rng.standard_normal(3000).astype(np.float32) * s for s in (1, 0.01, 100)]
                       + [mids, -mids, vals.astype(np.float32),
                          np.float32([448, 449, 464, 465, 1e6, 0.0, -0.0, 2**-10, 2**-10 * 3])])
    got = f32_to_e4m3_bits(x)
    want = np.array([_e4m3_nearest_even(v) for v in x], np.uint8)
    assert np.array_equal(got, want)


def test_merge_inputs_shapes_and_neutral_entries():
    mi = make_merge_inputs(8, neutral_frac=0.25)
    assert mi.outs.shape == (4, 8, 64, 512) and mi.outs.dtype == np.uint16
    assert mi.lses.shape == (4, 8, 64)
    neg = np.isneginf(mi.lses)
    assert neg.any() and (O.decode_bf16(mi.outs)[neg] == 0).all()


def test_config_table_matches_workload_shapes():
    assert CONFIGS[1]["batch"] == 2 and CONFIGS[1]["heads"] == 16 and CONFIGS[1]["shards"] == 4
    assert CONFIGS[3]["kv_dtype"] == "fp8" and CONFIGS[3]["shards"] == 8
    assert CONFIGS[4]["q_len"] == 4 and CONFIGS[4]["shards"] == 1
    assert CONFIGS[5]["lse_base"] == "2"
    wl = make_workload("x", batch=3, heads=16, q_len=4, shards=1, kv_dtype="bf16",
                       lens=("fixed", (5, 64, 65)), seed=1, extra_pages=2)
    assert wl.q.shape == (3, 4, 16, 576) and wl.kv_pages.shape == (1 + 1 + 2 + 2, 64, 576)
    assert np.isnan(O.decode_bf16(wl.kv_pages[-2:])).all()
