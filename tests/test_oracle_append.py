"""Pins of the oracle's KV append and its e4m3 encoder (CPU only).

The encoder is pinned against the format (every finite code round-trips,
every midpoint between neighbouring values goes to the even code, saturation
at 448, signed NaN), against a library cast (torch's float8_e4m3fn, round
to nearest even) and against the input generator's independent bit-level
encoder. The append is pinned against the layout invariant of the pages'
DCP key code (each appended token is written by exactly one shard, the
shard (L - 1) mod S for the newest) and against the shard-local KV index
table of the metadata oracle.
"""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from workloads import f32_to_e4m3_bits, make_append_inputs

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _values():
    return O.decode_e4m3(np.arange(0x7F, dtype=np.uint8))       # codes 0x00 .. 0x7E


def test_every_finite_code_round_trips():
    codes = np.arange(256, dtype=np.uint8)
    vals = O.decode_e4m3(codes)
    fin = ~np.isnan(vals)
    assert fin.sum() == 254
    assert np.array_equal(O.encode_e4m3(vals[fin].astype(np.float32)), codes[fin])


def test_midpoints_go_to_the_even_code():
    v = _values()
    for k in range(len(v) - 1):
        mid = np.float32((v[k] + v[k + 1]) / 2)        # 5 significant bits: exact in fp32
        assert float(mid) == (v[k] + v[k + 1]) / 2
        even = k if k % 2 == 0 else k + 1
        assert O.encode_e4m3(mid) == even, (k, float(mid))
        assert O.encode_e4m3(-mid) == (even | 0x80)
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(np.inf))
        assert O.encode_e4m3(below) == k and O.encode_e4m3(above) == k + 1


def test_saturation_zero_and_nan():
    enc = lambda x: int(O.encode_e4m3(np.float32(x)))    # noqa: E731
    assert enc(448.0) == 0x7E and enc(-448.0) == 0xFE
    assert enc(449.0) == 0x7E and enc(464.0) == 0x7E and enc(1e30) == 0x7E
    assert enc(np.inf) == 0x7E and enc(-np.inf) == 0xFE
    assert enc(0.0) == 0x00 and enc(-0.0) == 0x80
    assert enc(2.0 ** -10) == 0x00                        # half the smallest subnormal: tie to 0
    assert enc(3 * 2.0 ** -10) == 0x02                    # 1.5 subnormal steps: tie to even 2
    assert enc(np.nan) == 0x7F
    assert enc(-np.float32(np.nan)) == 0xFF


def test_matches_torch_cast_in_range():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (0.01, 1.0, 30.0, 150.0)]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.encode_e4m3(x), ref)


def test_matches_the_input_encoder_including_saturation():
    rng = np.random.default_rng(12)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (0.003, 1.0, 100.0, 1000.0)]).astype(np.float32)
    assert np.array_equal(O.encode_e4m3(x), f32_to_e4m3_bits(x))


@pytest.mark.parametrize("S", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("n_new", [1, 3])
def test_each_new_token_is_written_by_exactly_one_shard(S, n_new):
    inp = make_append_inputs(batch=24, n_new=n_new, kv_dtype="bf16", seed=40 + S)
    args = (inp.k_nope, inp.k_rope, inp.seq_lens, inp.block_table)
    written = np.zeros(inp.kv_pages.shape[:2], dtype=np.int32)
    for r in range(S):
        after = O.append_kv(inp.kv_pages, *args, r, S, "bf16")
        written += np.any(after != inp.kv_pages, axis=-1)
    unsharded = O.append_kv(inp.kv_pages, *args, 0, 1, "bf16")
    changed = np.any(unsharded != inp.kv_pages, axis=-1)
    assert written.max() <= 1
    assert np.array_equal(written.astype(bool), changed)
    # the newest token of request b goes to shard (L - 1) mod S
    for b in range(len(inp.seq_lens)):
        L = int(inp.seq_lens[b])
        pg = (L - 1) // 64
        if pg >= inp.block_table.shape[1]:
            continue
        page = int(inp.block_table[b, pg])
        if 0 <= page < inp.kv_pages.shape[0]:
            owner = (L - 1) % S
            after = O.append_kv(inp.kv_pages, *args, owner, S, "bf16")
            assert np.array_equal(after[page, (L - 1) % 64, :512], inp.k_nope[b, n_new - 1])


def test_written_row_is_the_metadata_row_of_the_newest_token():
    S = 4
    inp = make_append_inputs(batch=16, n_new=1, kv_dtype="bf16", num_pages=400, seed=7)
    ok = np.all((inp.block_table >= 0) & (inp.block_table < 400), axis=1) & (inp.seq_lens <= 6 * 64)
    lens, bt = inp.seq_lens[ok], inp.block_table[ok]
    for r in range(S):
        after = O.append_kv(inp.kv_pages, inp.k_nope[ok], inp.k_rope[ok], lens, bt, r, S, "bf16")
        ll, _, idx = O.shard_metadata(lens, bt, 64, int(lens.max()), r, S)
        flat_before = inp.kv_pages.reshape(-1, 576)
        flat_after = after.reshape(-1, 576)
        rows = np.flatnonzero(np.any(flat_after != flat_before, axis=1))
        newest = [int(idx[b, ll[b] - 1]) for b in range(len(lens)) if (int(lens[b]) - 1) % S == r]
        assert sorted(rows.tolist()) == sorted(set(newest))


def test_fp8_rows_are_within_half_a_step_of_the_scaled_input():
    inp = make_append_inputs(batch=12, n_new=2, kv_dtype="fp8", kv_scale=0.37, seed=9)
    after = O.append_kv(inp.kv_pages, inp.k_nope, inp.k_rope, inp.seq_lens, inp.block_table, 0, 1, "fp8",
                        inp.kv_scale)
    for b in range(12):
        for i in range(2):
            t = int(inp.seq_lens[b]) - 2 + i
            if t < 0 or t // 64 >= 6:
                continue
            page = int(inp.block_table[b, t // 64])
            if not 0 <= page < inp.kv_pages.shape[0]:
                continue
            x = O.decode_bf16(np.concatenate([inp.k_nope[b, i], inp.k_rope[b, i]])) / inp.kv_scale
            got = O.decode_e4m3(after[page, t % 64])
            a = np.minimum(np.abs(x), 448.0)
            # half a step of e4m3: 2^(floor(log2 a) - 4) for normals, 2^-10 below 2^-6
            half = np.where(a >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 4), 2.0 ** -10)
            assert np.all(np.abs(got - np.clip(x, -448, 448)) <= half * (1 + 1e-12))
