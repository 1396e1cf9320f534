"""fp64 CPU oracle for paged MLA decode over a context-sharded KV cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: it is used by ``tests/``, by ``__graft_entry__.smoke()``
to check one small GPU result, and by ``bench.py``'s ``cpu_baseline`` leg.
It shares no code with the HIP path; the only thing both sides see is the
input bytes produced by ``workloads.gen``.

Pages cited (by address and section heading as printed):
  [DCP decode]  prhub.com.cn digest of sgl-project/sglang PR 33926 (the
                trtllm_mla decode path gains DCP support); sections
                "功能与动机" (motivation), "实现拆解" (implementation, numbered
                steps) and "关键源码片段" (key code: the DCP metadata helpers
                and the TestDcpDecodeLayout invariants).
  [symm_a2a]    github.com sgl-project/sglang PR 33364, "[Attention][DCP] Add
                symm_a2a: single-node symmetric-memory A2A backend for MLA
                decode"; sections Motivation and Modifications.

What it computes, and the passage each step follows:

* ``local_len`` / ``shard_metadata`` -- [DCP decode] key code: a request's
  tokens are dealt cyclically to ranks (token t belongs to rank t mod S);
  the rank-local length of a request; the rank-local scheduling upper bound
  max(M // S + (r < M % S), 1); the page table rebuilt on the rank's cyclic
  slice. The oracle *enumerates* owned tokens (t in range(L) if t % S == r)
  rather than using the closed form, so the closed form printed there is an
  independent pin in the tests.
* ``decode_partial`` -- [DCP decode] motivation and implementation step 3:
  each rank attends over only the tokens it owns and returns its rank-local
  (out, lse); a rank that owns no token is set to the neutral (0, -inf).
  For one query row this is plain softmax attention restricted to the owned,
  causally visible tokens. MLA geometry: the score uses all 576 dims
  (latent 512 + rope 64); V is the first 512 latent dims.
* LSE base -- [DCP decode] implementation step 4 (first fix) and the
  related-PR note on PR 34240: one kernel family reports base-2 LSE, another
  natural-log LSE, and the merge site rebases. ``to_base`` / ``rebase_to_e``.
* ``merge`` -- [symm_a2a] Modifications, the fourth kernel (and the ag_rs /
  a2a combines under Motivation): the LSE-weighted softmax reduction of all
  ranks' partial outputs into the full-context result.
* ``quantize_query`` -- [DCP decode] implementation step 3 (the fp8 KV path
  prepares the query with a fused concat-and-quantise): e4m3 codes of the
  query by the same rounding rule as the fp8 KV rows; ``decode_partial``
  then reads the query as those codes times the query scale.
* ``append_kv`` / ``encode_e4m3`` -- [DCP decode] key code (the layout test:
  each appended token grows exactly one rank's local length, rank
  (L - 1) mod S) and implementation steps 3-4 (the KV row is written with
  the pool's plain row write; fp8 pools hold it quantised): the owner of each
  new token writes its [k_nope | k_rope] row into its page slot. fp8 codes
  are the nearest e4m3 value to the fp32 quotient x / kv_scale, ties to the
  even code, saturating at 448; the oracle finds that value by searching the
  table of all codes it decodes itself.

Readings where the pages are silent (each is listed with its reason in the
design notes): owner indexing is 0-based; for q_len > 1 the sequence length
includes the draft rows and draft row i sees tokens t <= L - q_len + i (with a
per-request depth q_b in place of q_len when given; rows past it see none); the
softmax scale is 1/sqrt(192) unless given; fp8 is OCP e4m3 with a per-tensor
scale; an all-empty merge gives (0, -inf).
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

LN2 = math.log(2.0)
D_QK = 576
D_V = 512


# --------------------------------------------------------------------------
# storage decoding (exact, to fp64)
# --------------------------------------------------------------------------
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64. bf16 is the upper half of an IEEE
    binary32, so widening the pattern by 16 zero bits gives the exact value."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """OCP fp8 e4m3 ("fn") codes (uint8) -> fp64, from the format definition:
    sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0;
    exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no inf."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


# --------------------------------------------------------------------------
# shard-local metadata ([DCP decode] key code: the DCP metadata helpers)
# --------------------------------------------------------------------------
def owned_tokens(L: int, shard_id: int, num_shards: int) -> List[int]:
    """Global positions of request tokens owned by a shard: t mod S == r."""
    return [t for t in range(int(L)) if t % num_shards == shard_id]


def local_len(L: int, shard_id: int, num_shards: int) -> int:
    """Number of tokens of a length-L request that the shard owns (by counting)."""
    return len(owned_tokens(L, shard_id, num_shards))


def local_max_seq_len(max_seq_len: int, shard_id: int, num_shards: int) -> int:
    """Rank-local scheduling upper bound; positive even for an empty shard
    ([DCP decode] key code: the local-max helper never returns 0)."""
    return max(local_len(max_seq_len, shard_id, num_shards), 1)


def shard_metadata(seq_lens: Sequence[int], block_table: np.ndarray, page_size: int,
                   max_seq_len: int, shard_id: int, num_shards: int
                   ) -> Tuple[np.ndarray, int, np.ndarray]:
    """Shard-local lengths, local max and token-granular KV row indices.

    ``local_kv_indices[b, j]`` is the physical KV row (page * page_size +
    slot) of the shard's j-th owned token of request b, in increasing global
    position; entries past the request's local length are -1. Row stride is
    the local max. Pure Python integers throughout.
    """
    B = len(seq_lens)
    lmax = local_max_seq_len(max_seq_len, shard_id, num_shards)
    lens = np.zeros(B, dtype=np.int32)
    idx = np.full((B, lmax), -1, dtype=np.int32)
    for b in range(B):
        toks = owned_tokens(int(seq_lens[b]), shard_id, num_shards)
        lens[b] = len(toks)
        for j, t in enumerate(toks):
            page = int(block_table[b][t // page_size])
            idx[b, j] = page * page_size + t % page_size
    return lens, lmax, idx


# --------------------------------------------------------------------------
# attention for one request (definition of softmax attention, fp64)
# --------------------------------------------------------------------------
def gather_kv_rows(kv_pages: np.ndarray, block_row: np.ndarray, tokens: Sequence[int],
                   kv_dtype: str, kv_scale: float, page_size: int = 64) -> np.ndarray:
    """Decode the latent KV rows of the given global token positions to fp64."""
    toks = np.asarray(tokens, dtype=np.int64)
    if toks.size == 0:
        return np.zeros((0, kv_pages.shape[-1]), dtype=np.float64)
    pages = np.asarray(block_row, dtype=np.int64)[toks // page_size]
    raw = kv_pages[pages, toks % page_size, :]
    if kv_dtype == "bf16":
        return decode_bf16(raw)
    if kv_dtype == "fp8":
        return decode_e4m3(raw) * float(kv_scale)
    raise ValueError(kv_dtype)


def attend(qrows: np.ndarray, K: np.ndarray, scale: float, visible: np.ndarray
           ) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of each query row over the visible latent rows.

    qrows [R, 576], K [n, 576] (fp64), visible [R, n] bool. Returns
    out [R, 512] and natural-log lse [R]. A row with no visible token gives
    the neutral state (0, -inf).
    """
    R = qrows.shape[0]
    out = np.zeros((R, D_V), dtype=np.float64)
    lse = np.full(R, -np.inf, dtype=np.float64)
    if K.shape[0] == 0:
        return out, lse
    s = scale * (qrows @ K.T)                      # [R, n]
    V = K[:, :D_V]
    for i in range(R):
        vis = visible[i]
        if not vis.any():
            continue
        si = s[i, vis]
        m = si.max()
        p = np.exp(si - m)
        l = p.sum()
        out[i] = (p @ V[vis]) / l
        lse[i] = m + math.log(l)
    return out, lse


def _q_rows(wl, b: int) -> np.ndarray:
    """Query rows of request b in fp64: the bf16 query, or, when the workload
    carries e4m3 query codes, their values times the query scale."""
    codes = getattr(wl, "q_codes", None)
    if codes is not None:
        return (decode_e4m3(codes[b]) * float(wl.q_scale)).reshape(wl.q_len * wl.heads, D_QK)
    return decode_bf16(wl.q[b]).reshape(wl.q_len * wl.heads, D_QK)


def decode_partial(wl, shard_id: int, num_shards: int, base: str = "e",
                   requests: Optional[Sequence[int]] = None
                   ) -> Tuple[np.ndarray, np.ndarray]:
    """Rank-local (out, lse) of one shard for a decode step.

    ``wl`` is a ``workloads.gen.Workload`` (bytes). For request b with
    global length L, decode depth q_b (``wl.q_lens[b]``, else q_len) and
    query row (i, h), the shard attends over
    {t < L : t mod S == r and t <= L - q_b + i} for i < q_b; rows i >= q_b
    are padding and see nothing. Returns out [B', q_len, H, 512] and lse
    [B', q_len, H] (in ``base``) for the chosen requests (all by default).
    """
    reqs = list(range(wl.batch)) if requests is None else list(requests)
    q, H = wl.q_len, wl.heads
    q_lens = getattr(wl, "q_lens", None)
    out = np.zeros((len(reqs), q, H, D_V), dtype=np.float64)
    lse = np.full((len(reqs), q, H), -np.inf, dtype=np.float64)
    for n, b in enumerate(reqs):
        L = int(wl.seq_lens[b])
        qb = q if q_lens is None else int(q_lens[b])
        toks = owned_tokens(L, shard_id, num_shards)
        K = gather_kv_rows(wl.kv_pages, wl.block_table[b], toks, wl.kv_dtype, wl.kv_scale)
        t = np.asarray(toks, dtype=np.int64)
        rows_vis = (np.stack([(t <= L - qb + i) & (i < qb) for i in range(q)]) if t.size
                    else np.zeros((q, 0), bool))
        visible = np.repeat(rows_vis, H, axis=0)     # row index = i * H + h
        o, l = attend(_q_rows(wl, b), K, wl.softmax_scale, visible)
        out[n] = o.reshape(q, H, D_V)
        lse[n] = l.reshape(q, H)
    return out, to_base(lse, base)


def decode_full(wl, requests: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Unsharded attention over the whole visible context (S = 1)."""
    return decode_partial(wl, 0, 1, "e", requests)


# --------------------------------------------------------------------------
# LSE base and merge ([DCP decode] related note on PR 34240; [symm_a2a]
# Modifications, fourth kernel)
# --------------------------------------------------------------------------
def to_base(lse_e: np.ndarray, base: str) -> np.ndarray:
    """Express a natural-log LSE in base 2 (log2 x = ln x / ln 2) or keep it."""
    lse_e = np.asarray(lse_e, dtype=np.float64)
    if base == "e":
        return lse_e.copy()
    if base == "2":
        return lse_e / LN2
    raise ValueError(base)


def rebase_to_e(lse: np.ndarray, base: str) -> np.ndarray:
    """Natural-log LSE from an LSE in ``base``; -inf stays -inf."""
    lse = np.asarray(lse, dtype=np.float64)
    if base == "e":
        return lse.copy()
    if base == "2":
        return lse * LN2
    raise ValueError(base)


def merge(outs: Sequence[np.ndarray], lses: Sequence[np.ndarray],
          bases: Optional[Sequence[str]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """LSE-weighted softmax combine of S partials.

    outs[r] [..., Dv], lses[r] [...] (shard r's LSE in bases[r]). With
    lse_r rebased to natural log, M = max_r lse_r, w_r = exp(lse_r - M):
    out = sum_r w_r out_r / sum_r w_r and lse = M + ln sum_r w_r. Where every
    shard is neutral (all lse_r = -inf) the result is (0, -inf).
    Returns (out, natural-log lse) in fp64.
    """
    S = len(outs)
    bases = list(bases) if bases is not None else ["e"] * S
    L = np.stack([rebase_to_e(lses[r], bases[r]) for r in range(S)])     # [S, ...]
    O = np.stack([np.asarray(o, dtype=np.float64) for o in outs])         # [S, ..., Dv]
    M = L.max(axis=0)
    empty = np.isneginf(M)
    Msafe = np.where(empty, 0.0, M)
    w = np.exp(L - Msafe)                    # exp(-inf) = 0 for neutral shards
    wsum = w.sum(axis=0)
    wsafe = np.where(empty, 1.0, wsum)
    out = (w[..., None] * O).sum(axis=0) / wsafe[..., None]
    out = np.where(empty[..., None], 0.0, out)
    lse = np.where(empty, -np.inf, Msafe + np.log(wsafe))
    return out, lse


def decode_step(wl, requests: Optional[Sequence[int]] = None, out_base: str = "e"
                ) -> Tuple[np.ndarray, np.ndarray, List[Tuple[np.ndarray, np.ndarray]]]:
    """All S shard partials of a workload followed by their merge.

    Returns (merged out, merged natural-log lse, [(out_r, lse_r) per shard]),
    the shard LSEs in the workload's base.
    """
    parts = [decode_partial(wl, r, wl.shards, wl.lse_base, requests) for r in range(wl.shards)]
    out, lse = merge([p[0] for p in parts], [p[1] for p in parts], [wl.lse_base] * wl.shards)
    return out, to_base(lse, out_base), parts


# --------------------------------------------------------------------------
# KV append into the owning shard ([DCP decode] key code: the layout test;
# implementation steps 3-4: the plain row write, fp8 pools quantised)
# --------------------------------------------------------------------------
def _e4m3_table() -> np.ndarray:
    """Values of the non-negative finite codes 0x00 .. 0x7E, increasing."""
    return decode_e4m3(np.arange(0x7F, dtype=np.uint8))


def encode_e4m3(x) -> np.ndarray:
    """float32 values -> OCP e4m3 ("fn") codes by the definition: the nearest
    representable value, ties to the code with an even mantissa; magnitudes
    above 448 (and infinities) give +-448; NaN gives 0x7F with x's sign."""
    x = np.asarray(x, dtype=np.float32)
    table = _e4m3_table()
    a = np.abs(x.astype(np.float64))
    sign = np.signbit(x).astype(np.uint8) << np.uint8(7)
    finite = np.isfinite(a)
    a_c = np.where(finite, np.minimum(a, table[-1]), table[-1])
    hi = np.searchsorted(table, a_c, side="left")          # first value >= a
    hi = np.minimum(hi, len(table) - 1)
    lo = np.where(table[hi] == a_c, hi, hi - 1)
    lo = np.maximum(lo, 0)
    d_lo = a_c - table[lo]
    d_hi = table[hi] - a_c
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.isnan(x), np.uint8(0x7F), code)
    return code | sign


def quantize_query(q_bits: np.ndarray, q_scale: float) -> np.ndarray:
    """e4m3 codes of a bf16 query ([DCP decode] 实现拆解 step 3: with an fp8
    KV pool the query is prepared by a fused concat-and-quantise). Each code
    is the nearest e4m3 value to the fp32 quotient q / q_scale, by the same
    rule as the fp8 KV rows (ties to the even code, saturating at 448, NaN
    keeps its sign). ``q_bits`` holds bf16 patterns (uint16), the 512 latent
    dims and the 64 rope dims of each row already side by side."""
    x = decode_bf16(q_bits).astype(np.float32)             # exact
    return encode_e4m3(x / np.float32(q_scale))


def append_kv(kv_pages: np.ndarray, k_nope: np.ndarray, k_rope: np.ndarray, seq_lens: Sequence[int],
              block_table: np.ndarray, shard_id: int, num_shards: int, kv_dtype: str,
              kv_scale: float = 1.0, page_size: int = 64) -> np.ndarray:
    """The pool after shard ``shard_id`` appends the newest n_new tokens of
    every request: token t = L - n_new + i (i < n_new) is written only if
    t >= 0 and t mod S == shard_id, into row block_table[b][t // 64] * 64 +
    t % 64, and only when that page id lies in the pool. ``k_nope`` [B, n, 512]
    and ``k_rope`` [B, n, 64] are bf16 bit patterns (uint16)."""
    out = np.array(kv_pages, copy=True)
    B, n = k_nope.shape[0], k_nope.shape[1]
    max_pages = block_table.shape[1]
    for b in range(B):
        L = int(seq_lens[b])
        for i in range(n):
            t = L - n + i
            if t < 0 or t % num_shards != shard_id or t // page_size >= max_pages:
                continue
            page = int(block_table[b][t // page_size])
            if page < 0 or page >= out.shape[0]:
                continue
            row_bits = np.concatenate([k_nope[b, i], k_rope[b, i]]).astype(np.uint16)
            if kv_dtype == "bf16":
                out[page, t % page_size, :] = row_bits
            elif kv_dtype == "fp8":
                x = decode_bf16(row_bits).astype(np.float32)      # exact
                out[page, t % page_size, :] = encode_e4m3(x / np.float32(kv_scale))
            else:
                raise ValueError(kv_dtype)
    return out
