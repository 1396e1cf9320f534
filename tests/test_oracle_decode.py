"""Pins for the oracle's partial decode, LSE base handling and merge (CPU only).

Each pin is independent of the oracle's own code: a pure-Python brute force
(math.fsum / math.exp over explicit loops, its own bf16 / e4m3 decoding),
closed forms of softmax attention, the merge's defining identity (the
combine of all shard partials equals unsharded attention), and the neutral
state of an empty shard. Sizes are tiny so the whole file runs in seconds.
"""
import dataclasses
import math
import os
import struct

import numpy as np
import pytest

from oracle import mla_oracle as O
from workloads import make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# storage codecs against the format definitions
# --------------------------------------------------------------------------
def _table(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if line:
            c, v = line.split()
            out.append((int(c, 16), float(v)))
    return out


def test_e4m3_golden_codes():
    for code, val in _table("e4m3_codes.txt"):
        got = float(O.decode_e4m3(np.array([code], np.uint8))[0])
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_e4m3_monotone_and_symmetric():
    pos = O.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    neg = O.decode_e4m3(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -pos)


def test_bf16_golden_patterns():
    for pat, val in _table("bf16_patterns.txt"):
        got = float(O.decode_bf16(np.array([pat], np.uint16))[0])
        assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(pat)


# --------------------------------------------------------------------------
# pure-Python brute force (its own decoding, explicit loops)
# --------------------------------------------------------------------------
def _bf16_py(bits):
    return struct.unpack(">f", struct.pack(">I", int(bits) << 16))[0]


def _e4m3_py(code):
    code = int(code)
    s = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 15, code & 7
    return s * (math.ldexp(m, -9) if e == 0 else math.ldexp(8 + m, e - 10))


def brute_partial(wl, b, shard, S):
    """(out [q,H,512], lse_e [q,H]) by explicit loops; no numpy linear algebra."""
    L = int(wl.seq_lens[b])
    q, H = wl.q_len, wl.heads
    dec = _bf16_py if wl.kv_dtype == "bf16" else (lambda c: _e4m3_py(c) * wl.kv_scale)
    rows = {}
    for t in range(L):
        if t % S == shard:
            page = int(wl.block_table[b, t // 64])
            rows[t] = [dec(x) for x in wl.kv_pages[page, t % 64]]
    out = np.zeros((q, H, 512))
    lse = np.full((q, H), -math.inf)
    for i in range(q):
        for h in range(H):
            qv = [_bf16_py(x) for x in wl.q[b, i, h]]
            toks = [t for t in rows if t <= L - q + i]
            if not toks:
                continue
            s = {t: wl.softmax_scale * math.fsum(qv[d] * rows[t][d] for d in range(576)) for t in toks}
            m = max(s.values())
            p = {t: math.exp(s[t] - m) for t in toks}
            l = math.fsum(p.values())
            for d in range(512):
                out[i, h, d] = math.fsum(p[t] * rows[t][d] for t in toks) / l
            lse[i, h] = m + math.log(l)
    return out, lse


def _tiny(q_len=1, kv="bf16", lens=(37, 21), heads=2, seed=7):
    return make_workload("tiny_test", batch=len(lens), heads=heads, q_len=q_len, shards=1,
                         kv_dtype=kv, lens=("fixed", lens), seed=seed)


@pytest.mark.parametrize("q_len,kv,S", [(1, "bf16", 1), (1, "bf16", 3), (1, "fp8", 4),
                                         (4, "bf16", 1), (4, "bf16", 2)])
def test_partial_matches_brute_force(q_len, kv, S):
    wl = _tiny(q_len=q_len, kv=kv, lens=(37, 6))
    for r in range(S):
        out, lse = O.decode_partial(wl, r, S, "e")
        for b in range(wl.batch):
            bo, bl = brute_partial(wl, b, r, S)
            np.testing.assert_allclose(out[b], bo, rtol=1e-11, atol=1e-12)
            assert np.array_equal(np.isneginf(lse[b]), np.isneginf(bl))
            fin = np.isfinite(bl)
            np.testing.assert_allclose(lse[b][fin], bl[fin], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
def _owned_rows(wl, b, r, S):
    L = int(wl.seq_lens[b])
    pos = np.arange(r, L, S)
    pages = wl.block_table[b, pos // 64]
    return O.decode_bf16(wl.kv_pages[pages, pos % 64])


@pytest.mark.parametrize("S", [1, 2, 4])
def test_zero_query_gives_mean_and_log_count(S):
    wl = _tiny(lens=(37, 130, 5), heads=3)
    wl.q[...] = 0                      # bf16 +0.0
    for r in range(S):
        out, lse = O.decode_partial(wl, r, S, "e")
        for b in range(wl.batch):
            rows = _owned_rows(wl, b, r, S)
            n = rows.shape[0]
            if n == 0:
                assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b]))
                continue
            np.testing.assert_allclose(out[b, 0], np.broadcast_to(rows[:, :512].mean(0), (3, 512)),
                                       rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(lse[b, 0], math.log(n), rtol=1e-14)


def test_identical_keys_give_that_row():
    wl = _tiny(lens=(50, 9), heads=2)
    row = wl.kv_pages[wl.block_table[0, 0], 0].copy()
    for b in range(wl.batch):
        L = int(wl.seq_lens[b])
        for t in range(L):
            wl.kv_pages[wl.block_table[b, t // 64], t % 64] = row
    k = O.decode_bf16(row)
    for b in range(wl.batch):
        n = int(wl.seq_lens[b])
        out, lse = O.decode_full(wl, [b])
        for h in range(2):
            s = wl.softmax_scale * float(np.dot(O.decode_bf16(wl.q[b, 0, h]), k))
            np.testing.assert_allclose(out[0, 0, h], k[:512], rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(lse[0, 0, h], s + math.log(n), rtol=1e-13)


def test_single_token_and_two_tokens():
    wl = _tiny(lens=(1, 2), heads=2)
    out, lse = O.decode_full(wl)
    k0 = O.decode_bf16(wl.kv_pages[wl.block_table[0, 0], 0])
    for h in range(2):
        qv = O.decode_bf16(wl.q[0, 0, h])
        s0 = wl.softmax_scale * float(np.dot(qv, k0))
        np.testing.assert_allclose(out[0, 0, h], k0[:512], rtol=1e-15)
        np.testing.assert_allclose(lse[0, 0, h], s0, rtol=1e-14)
    ka = O.decode_bf16(wl.kv_pages[wl.block_table[1, 0], 0])
    kb = O.decode_bf16(wl.kv_pages[wl.block_table[1, 0], 1])
    for h in range(2):
        qv = O.decode_bf16(wl.q[1, 0, h])
        a, b = (wl.softmax_scale * float(np.dot(qv, k)) for k in (ka, kb))
        np.testing.assert_allclose(lse[1, 0, h], np.logaddexp(a, b), rtol=1e-14)
        wa = 1.0 / (1.0 + math.exp(b - a))
        np.testing.assert_allclose(out[1, 0, h], wa * ka[:512] + (1 - wa) * kb[:512], rtol=1e-12, atol=1e-14)


def test_shard_owning_nothing_is_neutral():
    wl = _tiny(lens=(3, 1), heads=2)
    S = 8
    for r in range(S):
        out, lse = O.decode_partial(wl, r, S, "2")
        for b, L in enumerate(wl.seq_lens):
            if r >= L:
                assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b]))
            else:
                assert np.all(np.isfinite(lse[b]))


def test_draft_rows_equal_single_row_decode_at_shorter_length():
    """Row i of a q_len=4 step sees exactly what a q_len=1 step of length
    L-3+i sees (the draft tokens sit at the tail of the sequence)."""
    wl4 = _tiny(q_len=4, lens=(70, 9, 4), heads=2, seed=11)
    for S in (1, 3):
        for r in range(S):
            o4, l4 = O.decode_partial(wl4, r, S, "e")
            for i in range(4):
                wl1 = dataclasses.replace(wl4, q_len=1, q=np.ascontiguousarray(wl4.q[:, i:i + 1]),
                                          seq_lens=(wl4.seq_lens - 3 + i).astype(np.int32))
                o1, l1 = O.decode_partial(wl1, r, S, "e")
                np.testing.assert_array_equal(o4[:, i], o1[:, 0])
                np.testing.assert_array_equal(l4[:, i], l1[:, 0])


def test_per_request_depth_rows_equal_single_row_decodes_and_padding_is_neutral():
    """With a decode depth q_b per request (the step's q_len = the largest),
    real row i < q_b of request b sees what a q_len=1 step of length
    L - q_b + 1 + i sees; rows i >= q_b are padding, exactly (0, -inf); all
    depths equal to q_len reproduce the fixed-depth result."""
    wl4 = _tiny(q_len=4, lens=(70, 9, 4, 33, 12), heads=2, seed=13)
    q_lens = np.array([4, 1, 0, 2, 3], dtype=np.int32)
    var = dataclasses.replace(wl4, q_lens=q_lens)
    full = dataclasses.replace(wl4, q_lens=np.full(5, 4, dtype=np.int32))
    for S in (1, 3):
        for r in range(S):
            o4, l4 = O.decode_partial(wl4, r, S, "e")
            of, lf = O.decode_partial(full, r, S, "e")
            np.testing.assert_array_equal(o4, of)
            np.testing.assert_array_equal(l4, lf)
            ov, lv = O.decode_partial(var, r, S, "e")
            for b in range(5):
                qb = int(q_lens[b])
                for i in range(4):
                    if i >= qb:
                        assert np.all(ov[b, i] == 0.0) and np.all(np.isneginf(lv[b, i]))
                        continue
                    wl1 = dataclasses.replace(wl4, batch=1, q_len=1, q=np.ascontiguousarray(wl4.q[b:b + 1, i:i + 1]),
                                              seq_lens=np.array([wl4.seq_lens[b] - qb + 1 + i], dtype=np.int32),
                                              block_table=wl4.block_table[b:b + 1])
                    o1, l1 = O.decode_partial(wl1, r, S, "e")
                    np.testing.assert_array_equal(ov[b, i], o1[0, 0])
                    np.testing.assert_array_equal(lv[b, i], l1[0, 0])


# --------------------------------------------------------------------------
# merge
# --------------------------------------------------------------------------
@pytest.mark.parametrize("S", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("q_len", [1, 4])
def test_merge_of_shards_equals_unsharded(S, q_len):
    wl = _tiny(q_len=q_len, lens=(130, 37, 5, 2), heads=2, seed=3 + S)
    full_o, full_l = O.decode_full(wl)
    parts = [O.decode_partial(wl, r, S, "e") for r in range(S)]
    mo, ml = O.merge([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(mo, full_o, rtol=1e-12, atol=1e-13)
    assert np.array_equal(np.isneginf(ml), np.isneginf(full_l))
    fin = np.isfinite(full_l)
    np.testing.assert_allclose(ml[fin], full_l[fin], rtol=1e-13)


def _random_parts(S=4, shape=(3, 5), dv=8, seed=0, neutral=0.2):
    rng = np.random.default_rng(seed)
    outs = [rng.standard_normal(shape + (dv,)) for _ in range(S)]
    lses = [rng.normal(3, 2, size=shape) for _ in range(S)]
    for r in range(S):
        m = rng.uniform(size=shape) < neutral
        lses[r][m] = -np.inf
        outs[r][m] = 0.0
    return outs, lses


def test_merge_single_shard_is_identity():
    outs, lses = _random_parts(S=1)
    mo, ml = O.merge(outs, lses)
    assert np.array_equal(mo, outs[0]) and np.array_equal(ml, lses[0])


def test_merge_extra_neutral_shard_is_bit_identical():
    outs, lses = _random_parts(S=3)
    mo, ml = O.merge(outs, lses)
    z_o, z_l = np.zeros_like(outs[0]), np.full_like(lses[0], -np.inf)
    for pos in (0, 3):
        o2, l2 = list(outs), list(lses)
        o2.insert(pos, z_o)
        l2.insert(pos, z_l)
        mo2, ml2 = O.merge(o2, l2)
        assert np.array_equal(mo2, mo) and np.array_equal(ml2, ml)


def test_zero_lse_for_an_empty_shard_would_corrupt_the_merge():
    # The idle-rank path of the DP-attention page returns a *zero* LSE for
    # zero-token rows; merged as a shard that weight e^0 = 1 drags the output.
    outs, lses = _random_parts(S=2, neutral=0.0)
    mo, _ = O.merge(outs, lses)
    mz, _ = O.merge(outs + [np.zeros_like(outs[0])], lses + [np.zeros_like(lses[0])])
    assert not np.allclose(mz, mo)


def test_merge_permutation_shift_and_associativity():
    outs, lses = _random_parts(S=5)
    mo, ml = O.merge(outs, lses)
    perm = [3, 0, 4, 1, 2]
    po, pl = O.merge([outs[i] for i in perm], [lses[i] for i in perm])
    np.testing.assert_allclose(po, mo, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(pl, ml, rtol=1e-14)
    so, sl = O.merge(outs, [l + 7.5 for l in lses])
    np.testing.assert_allclose(so, mo, rtol=1e-13, atol=1e-14)
    fin = np.isfinite(ml)
    np.testing.assert_allclose(sl[fin], ml[fin] + 7.5, rtol=1e-14)
    ao, al = O.merge(outs[:2], lses[:2])
    bo, bl = O.merge([ao] + outs[2:], [al] + lses[2:])
    np.testing.assert_allclose(bo, mo, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(bl[fin], ml[fin], rtol=1e-14)


def test_all_neutral_merge_is_neutral():
    z = [np.zeros((2, 4)) for _ in range(3)]
    mo, ml = O.merge(z, [np.full(2, -np.inf)] * 3)
    assert np.all(mo == 0) and np.all(np.isneginf(ml)) and not np.isnan(mo).any()


def test_base2_and_natural_agree_after_rebase():
    wl = _tiny(lens=(130, 37), heads=2, seed=5)
    S = 4
    pe = [O.decode_partial(wl, r, S, "e") for r in range(S)]
    p2 = [O.decode_partial(wl, r, S, "2") for r in range(S)]
    for (oe, le), (o2, l2) in zip(pe, p2):
        np.testing.assert_array_equal(oe, o2)
        fin = np.isfinite(le)
        # log2(x) * ln 2 = ln(x)
        np.testing.assert_allclose(l2[fin] * math.log(2), le[fin], rtol=1e-15)
        assert np.array_equal(np.isneginf(le), np.isneginf(l2))
    me = O.merge([p[0] for p in pe], [p[1] for p in pe], ["e"] * S)
    m2 = O.merge([p[0] for p in p2], [p[1] for p in p2], ["2"] * S)
    mixed = O.merge([p[0] for p in pe], [pe[0][1], p2[1][1], pe[2][1], p2[3][1]], ["e", "2", "e", "2"])
    for m in (m2, mixed):
        np.testing.assert_allclose(m[0], me[0], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(m[1], me[1], rtol=1e-14)
