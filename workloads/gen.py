"""Seeded synthetic inputs for paged MLA decode over a context-sharded KV cache.

This module only *draws and encodes* inputs: request lengths, a shuffled page
pool with its block table, and N(0,1) query / latent-KV values encoded to bf16
or fp8-e4m3 bytes. It holds none of the attention arithmetic. The fp64 oracle
and the HIP path both consume exactly the bytes produced here, each decoding
them with its own code.

Shapes follow the MLA geometry used throughout the pages (the SGLang
``trtllm_mla`` DCP decode page and the symmetric-memory DCP merge page): a
latent KV row of 512 dims plus 64 rope dims (QK dim 576), V = the first 512
latent dims, page size 64.

Recipe (same for every workload):
  * generator: NumPy ``PCG64`` with a fixed seed;
  * draw order: sequence lengths, page permutation, Q, KV (merge partials
    for the merge-only workload);
  * Q and KV values are N(0,1) float32, rounded to bf16 with round-to-nearest
    -even; fp8 KV uses a per-tensor scale amax/448 and RNE with saturation;
    KV values come in chunks of 128 pages, each from its own PCG64 stream
    seeded by (a seed drawn from the main stream, chunk index);
  * the page pool holds exactly sum(ceil(L_b / 64)) pages, randomly permuted
    into the block table; unused block-table entries are -1;
  * KV slots past each request's length (the tail of its last page) hold NaN
    so that any out-of-range read poisons the result.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Optional, Sequence

import numpy as np

PAGE_SIZE = 64
D_QK = 576      # latent 512 + rope 64
D_V = 512       # V is the first 512 latent dims
BF16_NAN = 0x7FC0
E4M3_NAN = 0x7F
E4M3_MAX = 448.0


# --------------------------------------------------------------------------
# encoders (float32 -> storage bytes); inputs only
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16. Inputs are finite by construction.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Encode float32 values to OCP fp8 e4m3 ("fn") bytes.

    Format: 1 sign, 4 exponent (bias 7), 3 mantissa bits; subnormals at
    exponent field 0; no infinities; S.1111.111 is NaN; largest finite 448.
    Rounding is to nearest with ties to even; magnitudes above 448 saturate
    to 448.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    sign = ((u >> np.uint32(24)) & np.uint32(0x80)).astype(np.uint8)
    mag = (u & np.uint32(0x7FFFFFFF)).view(np.int32)
    # normal range (|x| >= 2^-6): round the float32 mantissa to 3 bits (RNE),
    # then rebias the exponent from 127 to 7: code = (bits >> 20) - (120 << 3)
    r = (mag >> 20) & 1
    r += mag
    r += 0x7FFFF
    r >>= 20
    r -= 120 << 3
    np.minimum(r, 0x7E, out=r)                      # saturate to 448
    # subnormal range: value = k * 2^-9 with k = rint(|x| * 512) in 0..8
    k = np.abs(x) * np.float32(512.0)
    np.rint(k, out=k)                               # ties to even
    code = np.where(mag >= 0x3C800000, r, k.astype(np.int32))   # 0x3C800000 = 2^-6
    return code.astype(np.uint8) | sign


# --------------------------------------------------------------------------
# KV value streams: pages are drawn in fixed chunks of CHUNK_PAGES, chunk c
# from its own PCG64 stream seeded by (kv_seed, c); the result does not depend
# on how many threads fill it.
# --------------------------------------------------------------------------
CHUNK_PAGES = 128


def _chunk_rng(kv_seed: int, c: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([kv_seed, c])))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _map_chunks(fn, num_pages: int):
    nchunks = (num_pages + CHUNK_PAGES - 1) // CHUNK_PAGES
    if nchunks <= 1 or _threads() == 1:
        return [fn(c) for c in range(nchunks)]
    with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
        return list(ex.map(fn, range(nchunks)))


def _kv_amax(kv_seed: int, num_pages: int) -> float:
    def one(c):
        n = min(CHUNK_PAGES, num_pages - c * CHUNK_PAGES) * PAGE_SIZE * D_QK
        x = _chunk_rng(kv_seed, c).standard_normal(n, dtype=np.float32)
        return float(np.max(np.abs(x))) if n else 0.0
    vals = _map_chunks(one, num_pages)
    return max(vals) if vals else 1.0


def _fill_kv_chunks(kv_seed: int, kv: np.ndarray, kind: str, scale: float) -> None:
    flat = kv.reshape(kv.shape[0], -1)
    num_pages = kv.shape[0]

    def one(c):
        p0 = c * CHUNK_PAGES
        p1 = min(num_pages, p0 + CHUNK_PAGES)
        x = _chunk_rng(kv_seed, c).standard_normal((p1 - p0) * PAGE_SIZE * D_QK, dtype=np.float32)
        if kind == "bf16":
            flat[p0:p1] = f32_to_bf16_bits(x).reshape(p1 - p0, -1)
        else:
            x /= np.float32(scale)
            flat[p0:p1] = f32_to_e4m3_bits(x).reshape(p1 - p0, -1)
    _map_chunks(one, num_pages)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    heads: int
    q_len: int
    shards: int
    kv_dtype: str                 # "bf16" | "fp8"
    lse_base: str                 # "e" | "2"  (base the partial kernel emits)
    out_dtype: str                # "f32" | "bf16" (partial out dtype)
    softmax_scale: float
    seq_lens: np.ndarray          # [B] int32, global KV length (incl. draft rows)
    block_table: np.ndarray       # [B, max_pages] int32, -1 padded
    kv_pages: np.ndarray          # [num_pages, 64, 576] uint16 (bf16) | uint8 (e4m3)
    kv_scale: float               # per-tensor dequant scale (1.0 for bf16)
    q: np.ndarray                 # [B, q_len, H, 576] uint16 (bf16)
    # per-request decode depth (rows i < q_lens[b] are real, the rest padding
    # up to the step's q_len); None = every request q_len deep
    q_lens: Optional[np.ndarray] = None
    # the query as e4m3 codes [B, q_len, H, 576] uint8 with a per-tensor
    # dequant scale (the fp8-KV path's concat-and-quantise of the query), or
    # None: the query is read as bf16
    q_codes: Optional[np.ndarray] = None
    q_scale: float = 0.0

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def num_pages(self) -> int:
        return int(self.kv_pages.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.batch else 0


# The five workload shapes. Lengths are (kind, a, b): "fixed" lists them,
# "uniform" draws integers in [a, b], "skewed" draws floor(2^U(0,17)) clamped
# to [1, 131072] with eight requests forced to lengths {1,1,2,3,4,5,6,7}.
# The tiny case keeps fp32 partials; the others emit bf16 partial outputs
# (the model dtype, which is what the exchange between shards carries) with
# fp32 LSE.
CONFIGS = {
    1: dict(name="tiny", batch=2, heads=16, q_len=1, shards=4, kv_dtype="bf16",
            lens=("fixed", (37, 130)), lse_base="e", out_dtype="f32"),
    2: dict(name="kimi_like", batch=64, heads=64, q_len=1, shards=4, kv_dtype="bf16",
            lens=("uniform", 4096, 8192), lse_base="e", out_dtype="bf16"),
    3: dict(name="deepseek_like_fp8", batch=32, heads=128, q_len=1, shards=8, kv_dtype="fp8",
            lens=("uniform", 16384, 32768), lse_base="e", out_dtype="bf16"),
    4: dict(name="mtp_q4", batch=32, heads=128, q_len=4, shards=1, kv_dtype="bf16",
            lens=("uniform", 2048, 16384), lse_base="e", out_dtype="bf16"),
    5: dict(name="skewed", batch=128, heads=128, q_len=1, shards=8, kv_dtype="bf16",
            lens=("skewed", 1, 131072), lse_base="2", out_dtype="bf16"),
}
SHORT_LENGTHS = (1, 1, 2, 3, 4, 5, 6, 7)
SOFTMAX_SCALE = 1.0 / math.sqrt(192.0)
MERGE_TOKENS = (1, 8, 16, 32, 64, 128)


def _draw_lengths(rng: np.random.Generator, batch: int, lens) -> np.ndarray:
    kind = lens[0]
    if kind == "fixed":
        vals = np.asarray(lens[1], dtype=np.int64)
        assert vals.shape[0] == batch
        return vals.astype(np.int32)
    if kind == "uniform":
        return rng.integers(lens[1], lens[2] + 1, size=batch).astype(np.int32)
    if kind == "skewed":
        lo, hi = lens[1], lens[2]
        u = rng.uniform(0.0, math.log2(hi), size=batch)
        vals = np.clip(np.floor(np.exp2(u)), lo, hi).astype(np.int64)
        nshort = min(len(SHORT_LENGTHS), batch)
        pos = rng.choice(batch, size=nshort, replace=False)
        vals[pos] = np.asarray(SHORT_LENGTHS[:nshort])
        return vals.astype(np.int32)
    raise ValueError(kind)


def make_workload(name: str, *, batch: int, heads: int, q_len: int, shards: int,
                  kv_dtype: str, lens, seed: int, lse_base: str = "e",
                  out_dtype: str = "f32", softmax_scale: float = SOFTMAX_SCALE,
                  extra_pages: int = 0, var_q: bool = False) -> Workload:
    """Draw one workload. ``lens`` is ("fixed", seq) | ("uniform", a, b) | ("skewed", 1, hi).

    ``extra_pages`` appends NaN-poisoned pages to the pool that no request
    references (a guard against stray page indices). ``var_q`` draws a
    decode depth per request, uniform in [0, q_len] (0: a request with no
    real query row this step), after every other draw, so the rest of the
    workload is the same as without it.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    seq_lens = _draw_lengths(rng, batch, lens)
    pages_per_req = [(int(L) + PAGE_SIZE - 1) // PAGE_SIZE for L in seq_lens]
    num_used = int(sum(pages_per_req))
    max_pages = max(1, max(pages_per_req) if pages_per_req else 1)
    perm = rng.permutation(num_used).astype(np.int32)
    block_table = np.full((batch, max_pages), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages_per_req):
        block_table[b, :n] = perm[off:off + n]
        off += n

    q_f32 = rng.standard_normal((batch, q_len, heads, D_QK), dtype=np.float32)
    q_bits = f32_to_bf16_bits(q_f32)
    del q_f32

    num_pages = num_used + extra_pages
    kv_seed = int(rng.integers(0, 2**63 - 1))
    if kv_dtype == "bf16":
        kv = np.empty((num_pages, PAGE_SIZE, D_QK), dtype=np.uint16)
        _fill_kv_chunks(kv_seed, kv, "bf16", 1.0)
        kv_scale = 1.0
        nan_code = BF16_NAN
    elif kv_dtype == "fp8":
        # per-tensor scale = amax / 448 over the drawn values (first pass),
        # then the same chunk streams are drawn again and encoded
        amax = _kv_amax(kv_seed, num_pages)
        kv_scale = amax / E4M3_MAX if amax > 0 else 1.0
        kv = np.empty((num_pages, PAGE_SIZE, D_QK), dtype=np.uint8)
        _fill_kv_chunks(kv_seed, kv, "fp8", kv_scale)
        nan_code = E4M3_NAN
    else:
        raise ValueError(kv_dtype)

    # poison the unused tail slots of every request's last page, and extra pages
    for b, L in enumerate(seq_lens):
        L = int(L)
        if L % PAGE_SIZE:
            last = block_table[b, L // PAGE_SIZE]
            kv[last, L % PAGE_SIZE:, :] = nan_code
    if extra_pages:
        kv[num_used:] = nan_code

    q_lens = rng.integers(0, q_len + 1, size=batch).astype(np.int32) if var_q else None

    return Workload(name=name, batch=batch, heads=heads, q_len=q_len, shards=shards,
                    kv_dtype=kv_dtype, lse_base=lse_base, out_dtype=out_dtype,
                    softmax_scale=softmax_scale, seq_lens=seq_lens,
                    block_table=block_table, kv_pages=kv, kv_scale=float(kv_scale),
                    q=q_bits, q_lens=q_lens)


def make_config(index: int, seed: Optional[int] = None, **overrides) -> Workload:
    """One of the five named workloads, seed 1000 + index unless given.

    ``overrides`` replace any field (e.g. ``batch``, ``lens``) to build a
    scaled-down instance with the same structure for parity tests.
    """
    spec = dict(CONFIGS[index])
    spec.update(overrides)
    return make_workload(spec.pop("name"), seed=1000 + index if seed is None else seed, **spec)


def _decode_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns to float32 (exact widening), for building inputs."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def plant_rising_keys(wl: Workload, tiles=(2, 5), magnitudes=(1.5, 2.5), group: int = 16) -> Workload:
    """Overwrite the latent rows of chosen token ranges with keys aligned to
    the request's queries, so that the scores of later tiles rise far above
    those of the first tile (inputs that make an online softmax move its
    running maximum several times per row).

    For each request and each entry k of ``tiles``, every token of the
    global range [32 S tiles[k], 32 S (tiles[k] + 1)) (owned-token tile
    ``tiles[k]`` of every one of the S shards) gets the row
    ``magnitudes[k] * sign(sum of the query rows of one group)``, all 576
    dims. The query rows (draft row i, head h; row = i H + h) are dealt to
    groups of ``group`` consecutive rows, and a planted token t goes to group
    (t // S) mod (number of groups), its index within the shard that owns
    it, so that every shard's planted tile holds keys of every group. Values
    are encoded like the rest of the pool (bf16 RNE, or e4m3 with the pool's
    scale). Only tokens below the request's length are
    touched. Returns ``wl`` (modified in place).
    """
    S, H, q = wl.shards, wl.heads, wl.q_len
    rows = q * H
    ngroups = (rows + group - 1) // group
    for b in range(wl.batch):
        L = int(wl.seq_lens[b])
        qf = _decode_bf16_bits(wl.q[b]).reshape(rows, D_QK).astype(np.float64)
        gsign = np.stack([np.sign(qf[g * group:(g + 1) * group].sum(axis=0)) for g in range(ngroups)])
        gsign[gsign == 0] = 1.0
        for tile, mag in zip(tiles, magnitudes):
            t0, t1 = 32 * S * tile, min(32 * S * (tile + 1), L)
            for t in range(t0, t1):
                row = (mag * gsign[(t // S) % ngroups]).astype(np.float32)
                page = int(wl.block_table[b, t // PAGE_SIZE])
                if wl.kv_dtype == "bf16":
                    wl.kv_pages[page, t % PAGE_SIZE] = f32_to_bf16_bits(row)
                else:
                    wl.kv_pages[page, t % PAGE_SIZE] = f32_to_e4m3_bits(row / np.float32(wl.kv_scale))
    return wl


@dataclasses.dataclass
class MergeInputs:
    outs: np.ndarray      # [S, N, H, Dv] uint16 (bf16) or float32
    lses: np.ndarray      # [S, N, H] float32 (natural log unless bases say otherwise)
    bases: Sequence[str]  # per shard "e" | "2"


def make_merge_inputs(tokens: int, *, shards: int = 4, heads: int = 64, dv: int = D_V,
                      seed: int = 2002, dtype: str = "bf16", bases: Optional[Sequence[str]] = None,
                      neutral_frac: float = 0.0) -> MergeInputs:
    """Partial outputs and LSEs shaped like the DCP merge's inputs.

    Partial out ~ N(0,1) (bf16 or fp32), LSE ~ 8 + 2*N(0,1); ``bases`` only
    labels which logarithm base each shard's LSE values are read in.
    ``neutral_frac`` of the (shard, row, head) entries are set to the neutral
    state (out 0, LSE -inf), as an empty shard emits.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    o = rng.standard_normal((shards, tokens, heads, dv), dtype=np.float32)
    lse = (8.0 + 2.0 * rng.standard_normal((shards, tokens, heads))).astype(np.float32)
    if neutral_frac > 0:
        mask = rng.uniform(size=(shards, tokens, heads)) < neutral_frac
        lse[mask] = -np.inf
        o[mask] = 0.0
    bases = list(bases) if bases is not None else ["e"] * shards
    outs = f32_to_bf16_bits(o) if dtype == "bf16" else o
    return MergeInputs(outs=outs, lses=lse, bases=bases)


@dataclasses.dataclass
class AppendInputs:
    k_nope: np.ndarray        # [B, n_new, 512] uint16 (bf16 bits)
    k_rope: np.ndarray        # [B, n_new, 64] uint16 (bf16 bits)
    seq_lens: np.ndarray      # [B] int32, new global lengths
    block_table: np.ndarray   # [B, max_pages] int32 (some entries -1 or past the pool)
    kv_pages: np.ndarray      # [num_pages, 64, 576] uint16 (bf16) | uint8 (e4m3), the pool before
    kv_dtype: str
    kv_scale: float


def make_append_inputs(*, batch: int = 40, n_new: int = 1, max_pages: int = 6, num_pages: int = 256,
                       kv_dtype: str = "bf16", kv_scale: float = 0.75, seed: int = 3003,
                       special: Sequence[float] = ()) -> AppendInputs:
    """New-token KV rows and a paged pool for the append step.

    Lengths cover the edge cases of the owner and page arithmetic: 1 .. n_new
    (tokens before the request start), page boundaries (63, 64, 65, 128),
    the last slot of the table (max_pages * 64) and one past it, then uniform
    draws. Block tables hold distinct pages of the pool (no two requests
    share one), with a few entries
    set to -1 and to num_pages (outside the pool). Row values are N(0, 4)
    bf16; ``special`` values (bf16-representable, e.g. NaN, +-inf, format
    midpoints) are planted at seeded positions. The pool starts as random
    bytes so that every write and every untouched row is visible.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    fixed = [1, 2, 3, n_new, 63, 64, 65, 128, max_pages * 64, max_pages * 64 + 1]
    lens = list(fixed) + list(rng.integers(1, max_pages * 64 + 1, size=max(batch - len(fixed), 0)))
    lens = np.asarray(lens[:batch], dtype=np.int32)
    if num_pages < batch * max_pages:
        raise ValueError("the pool must hold batch * max_pages distinct pages")
    bt = rng.permutation(num_pages)[:batch * max_pages].reshape(batch, max_pages).astype(np.int32)
    holes = rng.uniform(size=bt.shape)
    bt[holes < 0.04] = -1
    bt[(holes >= 0.04) & (holes < 0.08)] = num_pages
    x = (2.0 * rng.standard_normal((batch, n_new, D_QK))).astype(np.float32)
    if len(special):
        flat = x.reshape(-1)
        pos = rng.choice(flat.size, size=min(len(special) * 8, flat.size), replace=False)
        flat[pos] = np.resize(np.asarray(special, dtype=np.float32), pos.size)
    bits = f32_to_bf16_bits(x)
    if kv_dtype == "bf16":
        pool = rng.integers(0, 1 << 16, size=(num_pages, PAGE_SIZE, D_QK), dtype=np.uint16)
    elif kv_dtype == "fp8":
        pool = rng.integers(0, 1 << 8, size=(num_pages, PAGE_SIZE, D_QK), dtype=np.uint8)
    else:
        raise ValueError(kv_dtype)
    return AppendInputs(k_nope=np.ascontiguousarray(bits[..., :512]), k_rope=np.ascontiguousarray(bits[..., 512:]),
                        seq_lens=lens, block_table=bt, kv_pages=pool, kv_dtype=kv_dtype, kv_scale=float(kv_scale))
