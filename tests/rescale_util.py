"""Workloads whose scores rise tile after tile, and a CPU count of how often
an online softmax with a lazily moved reference must move it on them.

The attention kernels keep a per-row exponent reference that moves (and
rescales the row's accumulator) only when a 32-token tile's maximum exceeds
it by more than SLACK log2 units. Random N(0,1) inputs almost never do that
after the first tile, so these workloads plant keys aligned with the
queries in owned-token tiles 2 and 5 of every shard (``plant_rising_keys``)
and the helpers below check, from the scores computed here in float64, that
the reference really moves several times per row.
"""
import math

import numpy as np

from oracle import mla_oracle as O
from workloads import make_workload, plant_rising_keys

SLACK = 8.0          # log2 units, the kernels' rescale threshold
LOG2E = 1.0 / math.log(2.0)

# name -> make_workload arguments; every request is long enough to reach
# owned tile 5 of every shard
SPECS = {
    "bf16_h16_s2": dict(batch=3, heads=16, q_len=1, shards=2, kv_dtype="bf16", lens=("uniform", 520, 900)),
    "fp8_h32_s2": dict(batch=3, heads=32, q_len=1, shards=2, kv_dtype="fp8", lens=("uniform", 520, 900)),
    "bf16_h16_q4_s2": dict(batch=4, heads=16, q_len=4, shards=2, kv_dtype="bf16", lens=("uniform", 520, 900),
                           var_q=True),
    "bf16_h16_q4_s1": dict(batch=3, heads=16, q_len=4, shards=1, kv_dtype="bf16", lens=("uniform", 260, 500)),
    "bf16_h128_s2": dict(batch=2, heads=128, q_len=1, shards=2, kv_dtype="bf16", lens=("uniform", 520, 700)),
    "fp8_h128_q2_s1": dict(batch=2, heads=128, q_len=2, shards=1, kv_dtype="fp8", lens=("uniform", 300, 500)),
}


def rising_workload(name: str):
    spec = dict(SPECS[name])
    seed = 500 + sorted(SPECS).index(name)
    wl = make_workload("rising_" + name, seed=seed, out_dtype="bf16", **spec)
    return plant_rising_keys(wl)


def reference_moves(wl, b: int, shard: int):
    """Per query row of request b on one shard: the number of times the lazy
    reference moves after the first tile, and the largest single move
    (log2 units), with tiles of 32 owned visible tokens in order."""
    S, H, q = wl.shards, wl.heads, wl.q_len
    L = int(wl.seq_lens[b])
    qb = q if wl.q_lens is None else int(wl.q_lens[b])
    toks = np.asarray(O.owned_tokens(L, shard, S), dtype=np.int64)
    K = O.gather_kv_rows(wl.kv_pages, wl.block_table[b], toks, wl.kv_dtype, wl.kv_scale)
    Q = O.decode_bf16(wl.q[b]).reshape(q * H, -1)
    s = (Q @ K.T) * wl.softmax_scale * LOG2E
    moves = np.zeros(q * H, np.int64)
    biggest = np.zeros(q * H)
    for row in range(q * H):
        i = row // H
        if i >= qb:
            continue
        vis = toks <= L - qb + i
        sr = s[row, vis]
        ntile = (sr.size + 31) // 32
        if ntile == 0:
            continue
        ref = sr[:32].max()
        for k in range(1, ntile):
            tm = sr[32 * k:32 * k + 32].max()
            if tm > ref + SLACK:
                moves[row] += 1
                biggest[row] = max(biggest[row], tm - ref)
                ref = tm
    return moves, biggest


def check_crossings(wl):
    """Fraction of real rows (over requests and shards) whose reference moves
    at least twice, and the largest single move seen."""
    tot, twice, big = 0, 0, 0.0
    for b in range(wl.batch):
        for r in range(wl.shards):
            mv, bg = reference_moves(wl, b, r)
            qb = wl.q_len if wl.q_lens is None else int(wl.q_lens[b])
            real = np.arange(wl.q_len * wl.heads) // wl.heads < qb
            tot += int(real.sum())
            twice += int((mv[real] >= 2).sum())
            big = max(big, float(bg.max()) if bg.size else 0.0)
    return (twice / tot if tot else 0.0), big
