"""Pins for the oracle's shard-local metadata (CPU only).

The oracle counts owned tokens by enumeration; these tests hold it against
the pages' own invariants (the TestDcpDecodeLayout sweep in the key-code
section of the prhub digest of sglang PR 33926), the closed-form rank-local
length printed in that section's local-max helper, and hand-worked values.
"""
import os

import numpy as np
import pytest

from oracle import mla_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dcp_metadata.txt")
SIZES = [1, 2, 3, 4, 8]          # the pages' sweep
LENS = list(range(0, 41))


def _golden(kind):
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line.startswith(kind + " "):
            rows.append(line.split()[1:])
    return rows


def test_ranks_partition_the_global_length():
    for n in SIZES:
        for L in LENS:
            assert sum(O.local_len(L, r, n) for r in range(n)) == L, (n, L)


def test_newest_token_grows_exactly_its_owner():
    for n in SIZES:
        for L in LENS[1:]:
            grew = [O.local_len(L, r, n) - O.local_len(L - 1, r, n) for r in range(n)]
            assert sum(grew) == 1
            assert grew[(L - 1) % n] == 1


def test_enumeration_matches_printed_closed_form():
    # the local-max helper of the key-code section computes M // S + (r < M % S)
    for n in range(1, 10):
        for L in range(0, 200):
            for r in range(n):
                assert O.local_len(L, r, n) == L // n + int(r < L % n)


def test_local_max_is_positive_and_matches_helper():
    for n in SIZES:
        for M in LENS:
            for r in range(n):
                assert O.local_max_seq_len(M, r, n) == max(M // n + int(r < M % n), 1)
                assert O.local_max_seq_len(M, r, n) >= 1


def test_golden_local_len_and_max():
    for L, S, *vals in _golden("local_len"):
        L, S = int(L), int(S)
        assert [O.local_len(L, r, S) for r in range(S)] == [int(v) for v in vals]
    for M, S, *vals in _golden("local_max"):
        M, S = int(M), int(S)
        assert [O.local_max_seq_len(M, r, S) for r in range(S)] == [int(v) for v in vals]


def test_golden_kv_rows():
    for shard, S, pages, L, *rows in _golden("kv_rows"):
        shard, S, L = int(shard), int(S), int(L)
        bt = np.array([[int(p) for p in pages.split(",")]], dtype=np.int32)
        lens, lmax, idx = O.shard_metadata([L], bt, 64, L, shard, S)
        assert lens[0] == len(rows)
        assert idx[0, :lens[0]].tolist() == [int(x) for x in rows]
        assert (idx[0, lens[0]:] == -1).all()


@pytest.mark.parametrize("S", [1, 2, 3, 4, 8])
def test_kv_rows_follow_strided_positions(S):
    # independent formulation: the j-th owned token of shard r is t = j*S + r
    rng = np.random.default_rng(S)
    B = 5
    seq_lens = rng.integers(0, 300, size=B)
    npages = int(sum((L + 63) // 64 for L in seq_lens))
    perm = rng.permutation(max(npages, 1))
    maxp = max(1, max((L + 63) // 64 for L in seq_lens))
    bt = np.full((B, maxp), -1, dtype=np.int32)
    off = 0
    for b, L in enumerate(seq_lens):
        k = (L + 63) // 64
        bt[b, :k] = perm[off:off + k]
        off += k
    M = int(seq_lens.max())
    for r in range(S):
        lens, lmax, idx = O.shard_metadata(seq_lens, bt, 64, M, r, S)
        assert lmax == max(M // S + int(r < M % S), 1)
        assert idx.shape == (B, lmax)
        for b, L in enumerate(seq_lens):
            for j in range(lmax):
                t = j * S + r
                want = int(bt[b, t // 64]) * 64 + t % 64 if t < L else -1
                assert idx[b, j] == want
