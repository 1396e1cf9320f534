// Rank-local paged MLA decode: a persistent, warp-specialised kernel.
//
// One shard r of S owns the tokens t = j S + r of every request (prhub.com.cn
// digest of sgl-project/sglang PR 33926, sections 功能与动机 and 实现拆解
// step 3); this file computes, for each query row, softmax attention over
// those tokens and emits the rank-local (out, lse), (0, -inf) where a row
// sees no owned token.
//
// Schedule. The shard's work is a sequence of units (request b, block of 64
// query rows rb, 32-token tile), ordered by segment s = b * row_blocks + rb
// and tile. A launch may also run every shard at once (the single-launch
// decode of all shards): a segment is then (b, rb, shard r), the S segments
// of (b, rb) are neighbours, and the pieces of all of them are merged by
// the combine with the same LSE-weighted reduction as the cross-shard merge
// (github.com sgl-project/sglang PR 33364, Modifications, the fourth
// kernel), so the shards' partials never leave the workspace. stream_plan_kernel lays the segments out on device (no host
// synchronisation) and each persistent workgroup takes a contiguous share of
// the units of about equal cost. A segment that a workgroup holds entirely
// is finalised in place; a segment cut at workgroup boundaries leaves one
// bf16 partial per piece, combined by stream_combine_kernel (mla_combine.hip).
//
// Workgroup (attn_ws_kernel). Eight waves, two per SIMD: four score waves
// (S^T = K Q^T on v_mfma_f32_32x32x16_bf16, two per row group of 32 rows,
// each over half the 576 QK dims, and the online softmax) and four output
// waves (O^T += V^T P^T for all 64 rows, 128 dims each). Tiles move HBM ->
// LDS with global_load_lds_dwordx4 (no register staging) through four
// stages, as stored: bf16 (36 KB) or fp8 e4m3 (18 KB, converted to bf16 in
// registers, exactly); the row of every token comes from the block table or
// the local KV indices by scalar loads, and out-of-pool pages point the copy
// at a constant NaN row.
#include "mla_device.h"

#include <hip/hip_ext.h>


namespace mla {
namespace {

constexpr int kStageBytes = kTile * kDqk * 2;      // 36864: one bf16 tile
constexpr int kRopeBase = kTile * 1024;             // rope part of a bf16 stage (dims 512..575)
// A row's exponent reference moves up (rescaling its accumulator) only when a
// tile's max exceeds it by more than this (log2 units), so rescaling is rare
// and unnormalised probabilities stay below 2^kRescaleSlack.
constexpr float kRescaleSlack = 8.0f;




// ---------------------------------------------------------------------------
// plan
// ---------------------------------------------------------------------------
// Exclusive scan of a pair of ints per thread over the 1024-thread block
// (wave scans with shuffles, then the 16 wave totals); `total` gets the sums.
__device__ __forceinline__ int2 block_excl_scan2(int a, int b, int2* s_wave, int2& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int ia = a, ib = b;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int xa = __shfl_up(ia, off), xb = __shfl_up(ib, off);
    if (lane >= off) {
      ia += xa;
      ib += xb;
    }
  }
  if (lane == 63) s_wave[wave] = make_int2(ia, ib);
  __syncthreads();
  int pa = 0, pb = 0, ta = 0, tb = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const int2 v = s_wave[w];
    if (w < wave) {
      pa += v.x;
      pb += v.y;
    }
    ta += v.x;
    tb += v.y;
  }
  __syncthreads();
  total = make_int2(ta, tb);
  return make_int2(pa + ia - a, pb + ib - b);
}

// Last index i in [0, n) with a[i] <= x (a nondecreasing, a[0] <= x).
__device__ __forceinline__ int last_le(const int32_t* a, int n, long long x) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid;
    else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ int seg_count(const DecodeParams& p, int s) {
  const SegId id = seg_id(p, s);
  return owned_count(p, id.b, id.r);
}
__device__ __forceinline__ int seg_tiles(const DecodeParams& p, int s) {
  return (seg_count(p, s) + kTile - 1) / kTile;
}

// One workgroup of 1024 threads; thread i handles a contiguous block of
// segments. The segment offsets stay in LDS when they fit (the binary
// searches then cost LDS latency only), else in the workspace.
//
// Row-block groups (p.rgroup = R > 1, a request with R row blocks): the
// schedule is made over super-segments (request, shard), whose units are
// their tiles, and over groups of R consecutive workgroups; workgroup
// g = R gamma + j of group gamma takes row block j of the units its group
// holds. The R workgroups of a group walk the same tiles of the same request
// at the same time on one XCD (groups never straddle XCDs when the grid
// divides into 8 x R), so each tile comes from HBM once for all row blocks
// instead of once per row block. R = 1 is the plain schedule, where a
// super-segment is a segment.
constexpr int kPlanLdsSegs = 6144;

// segment of super-segment `sup` for row block j
__device__ __forceinline__ int seg_of_sup(const DecodeParams& p, int sup, int j) {
  if (p.rgroup == 1) return sup;
  const int b = sup / p.fold, ri = sup - b * p.fold;
  return (b * p.row_blocks + j) * p.fold + ri;
}
// owned-token count of super-segment `sup`
__device__ __forceinline__ int sup_count(const DecodeParams& p, int sup) {
  if (p.rgroup == 1) return seg_count(p, sup);
  const int b = sup / p.fold, ri = sup - b * p.fold;
  return owned_count(p, b, p.fold > 1 ? ri : p.shard);
}

__global__ __launch_bounds__(1024) void stream_plan_kernel(DecodeParams p) {
  __shared__ int32_t s_arr[2 * (kPlanLdsSegs + 1)];
  __shared__ int32_t s_cnt[kPlanLdsSegs];           // owned tokens of each super-segment
  __shared__ int32_t s_wgu[kMaxGrid + 1];           // first unit of each group
  __shared__ int2 s_wave[16];
  const int tid = threadIdx.x;
  const int RB = p.row_blocks, GR = p.rgroup;
  const int nseg = p.batch * RB * p.fold;
  const int nsup = GR == 1 ? nseg : p.batch * p.fold;
  const bool in_lds = nsup <= kPlanLdsSegs;
  int32_t* const off = in_lds ? s_arr : p.seg_off;              // unit offset of each super-segment
  int32_t* const coff = in_lds ? s_arr + kPlanLdsSegs + 1 : p.seg_coff;   // cost offset
  const int per = (nsup + 1023) / 1024;
  const int s0 = min(tid * per, nsup), s1 = min(s0 + per, nsup);

  // the row-block groups' rendezvous counters start at zero
  for (int q = tid; q < kMaxGrid; q += 1024) p.grp_sync[q] = 0;
  // owned-token counts per request and shard
  for (int q = tid; q < p.batch * p.fold; q += 1024) {
    const int b = q / p.fold, ri = q - b * p.fold;
    p.req_cnt[q] = owned_count(p, b, p.fold > 1 ? ri : p.shard);
  }
  // tiles and costs (a super-segment costs its tiles plus kPieceCost for
  // loading its queries) of this thread's super-segments, scanned over the
  // block. When the launch runs every shard, a piece continues across the
  // shards of its row block (their super-segments are neighbours), so only a
  // row block's first shard pays the query cost; shard 0 owns token 0, so it
  // has tiles whenever any shard of the request has
  const int kPieceCost = p.kv_fp8 ? kPieceCostFp8 : kPieceCostBf16;
  auto piece_cost = [&](int s) { return p.fold > 1 && s % p.fold != 0 ? 0 : kPieceCost; };
  int su = 0, sc = 0;
  for (int s = s0; s < s1; ++s) {
    const int cnt = sup_count(p, s);
    if (in_lds) s_cnt[s] = cnt;
    const int n = (cnt + kTile - 1) / kTile;
    su += n;
    sc += n > 0 ? n + piece_cost(s) : 0;
  }
  int2 tot;
  const int2 ex = block_excl_scan2(su, sc, s_wave, tot);
  {
    int u = ex.x, c = ex.y;
    for (int s = s0; s < s1; ++s) {
      const int n = ((in_lds ? s_cnt[s] : sup_count(p, s)) + kTile - 1) / kTile;
      off[s] = u;
      coff[s] = c;
      u += n;
      c += n > 0 ? n + piece_cost(s) : 0;
    }
  }
  const int U = tot.x, C = tot.y;
  // groups in use: at most one per cost unit, so consecutive group
  // boundaries differ and only a piece's first group can start inside its
  // query-load cost
  const int NG = min(p.grid / GR, C);
  if (tid == 0) {
    off[nsup] = U;
    coff[nsup] = C;
    p.plan[0] = U;
    p.plan[1] = NG * GR;
    s_wgu[NG] = U;
    p.wg_ustart[NG] = U;
  }
  __syncthreads();

  // first unit of each group: cost boundary gamma C / NG mapped to the unit
  // sequence (a boundary inside a super-segment's query cost maps to its
  // first tile)
  for (int g = tid; g < NG; g += 1024) {
    const long long x = (long long)g * C / NG;
    const int s = last_le(coff, nsup + 1, x);
    const int n = off[s + 1] - off[s];
    long long k = x - coff[s] - piece_cost(s);
    k = k < 0 ? 0 : (k > n - 1 ? n - 1 : k);
    s_wgu[g] = off[s] + (int)k;
    p.wg_ustart[g] = off[s] + (int)k;
    p.wg_start[g] = make_int2(s, (int)k);
  }
  __syncthreads();

  // start record of each workgroup (group w / GR, row block w % GR): its
  // range, its first unit with the owned-token count of that request, and
  // the segment (with its count) of the unit after its first super-segment,
  // so that the decode kernel resolves the rows of its first two tiles after
  // a single round of loads
  for (int w = tid; w < p.grid; w += 1024) {
    int32_t* rec = p.wg_rec + (long long)w * kRecInts;
    const int grp = w / GR, j = w - grp * GR;
    const int u0 = grp < NG ? s_wgu[grp] : 0, u1 = grp < NG ? s_wgu[grp + 1] : 0;
    int seg = 0, tile = 0, cnt = 0, seg1 = 0, cnt1 = 0;
    if (u1 > u0) {
      const int sp = last_le(off, nsup + 1, u0);
      tile = u0 - off[sp];
      seg = seg_of_sup(p, sp, j);
      cnt = in_lds ? s_cnt[sp] : sup_count(p, sp);
      const int un = off[sp + 1];          // first unit past the first super-segment
      if (un < u1) {
        const int sp1 = last_le(off, nsup + 1, un);
        seg1 = seg_of_sup(p, sp1, j);
        cnt1 = in_lds ? s_cnt[sp1] : sup_count(p, sp1);
      }
    }
    rec[0] = u1 - u0;
    rec[1] = seg;
    rec[2] = tile;
    rec[3] = cnt;
    rec[4] = seg1;
    rec[5] = cnt1;
  }

  // pieces of each segment (one per non-empty group its super-segment
  // meets) and partial slots (only for segments cut into several pieces),
  // allocated in segment order. When the launch runs every shard, the
  // pieces are those of the row block's run of S segments (one per group
  // the run meets: a group's piece spans the run's shards it holds), every
  // piece leaves a partial, and each segment of the run records the run's
  // slots (thread ranges are whole runs)
  const bool runs = p.fold > 1;
  const int np_slot = runs ? 1 : 2;
  int sper = (nseg + 1023) / 1024;
  if (runs) sper = (sper + p.fold - 1) / p.fold * p.fold;
  const int q0 = min(tid * sper, nseg), q1 = min(q0 + sper, nseg);
  auto seg_pieces = [&](int s, int& first) {
    int o, e;
    if (GR > 1) {
      const int q = s / p.fold, ri = s - q * p.fold;
      const int sp = (q / RB) * p.fold + ri;
      o = off[runs ? sp - ri : sp];
      e = off[runs ? sp - ri + p.fold : sp + 1];
    } else {
      const int r0 = runs ? s % p.fold : 0;
      o = off[s - r0];
      e = off[runs ? s - r0 + p.fold : s + 1];
    }
    first = 0;
    if (e <= o) return 0;
    first = last_le(s_wgu, NG, o);
    return last_le(s_wgu, NG, e - 1) - first + 1;
  };
  int ms = 0;
  for (int s = q0; s < q1; ++s) {
    if (runs && s % p.fold != 0) continue;
    int first;
    const int np = seg_pieces(s, first);
    ms += np >= np_slot ? np : 0;
  }
  const int2 ex2 = block_excl_scan2(ms, 0, s_wave, tot);
  int slot = ex2.x, run_slot = slot;
  for (int s = q0; s < q1; ++s) {
    int first;
    const int np = seg_pieces(s, first);
    if (!runs || s % p.fold == 0) {
      run_slot = slot;
      slot += np >= np_slot ? np : 0;
    }
    p.seg_info[s] = make_int4(run_slot, np, first, 0);
  }
}

// ---------------------------------------------------------------------------
// streaming attention
// ---------------------------------------------------------------------------
// Position in the unit sequence: segment, its request, row block and shard,
// tile, and the segment's tile count and owned-token count. Wave-uniform.
struct Cursor {
  int seg, b, rb, r, tile, ntiles, cnt;

  __device__ __forceinline__ void start_known(const DecodeParams& p, int s, int t, int count) {
    const SegId id = seg_id(p, s);
    seg = s;
    b = id.b;
    rb = id.rb;
    r = id.r;
    tile = t;
    cnt = count;
    ntiles = (cnt + kTile - 1) / kTile;
  }
  // move to the next unit; only called when one exists (kFold: the launch
  // runs every shard, p.fold > 1)
  template <bool kFold>
  __device__ __forceinline__ void advance(const DecodeParams& p) {
    if (++tile < ntiles) return;
    tile = 0;
    if (p.rgroup > 1) {
      // row-block groups: the same row block of the next (request, shard)
      for (;;) {
        if (kFold && ++r < p.fold) {
        } else {
          ++b;
          r = kFold ? 0 : r;
        }
        seg = (b * p.row_blocks + rb) * p.fold + (kFold ? r : 0);
        cnt = ld_const(p.req_cnt + b * p.fold + (kFold ? r : 0));
        ntiles = (cnt + kTile - 1) / kTile;
        if (ntiles > 0) return;
      }
    }
    for (;;) {
      ++seg;
      if (kFold && ++r < p.fold) {
        cnt = ld_const(p.req_cnt + b * p.fold + r);
      } else {
        const bool next_b = ++rb == p.row_blocks;
        if (next_b) {
          rb = 0;
          ++b;
        }
        if (kFold) {
          r = 0;
          cnt = ld_const(p.req_cnt + b * p.fold);
        } else if (next_b) {
          cnt = ld_const(p.req_cnt + b);
        }
      }
      ntiles = (cnt + kTile - 1) / kTile;
      if (ntiles > 0) break;
    }
  }
  // move n >= 1 units forward (they exist)
  template <bool kFold>
  __device__ __forceinline__ void advance_by(const DecodeParams& p, int n) {
    for (;;) {
      const int left = ntiles - 1 - tile;
      if (n <= left) {
        tile += n;
        return;
      }
      n -= left + 1;
      tile = ntiles - 1;
      advance<kFold>(p);
      if (n == 0) return;
    }
  }
  // units from here to the end of the row block's run when the launch runs
  // every shard (this segment's and the later shards' of the same request
  // and row block)
  __device__ __forceinline__ int run_units(const DecodeParams& p) const {
    int n = ntiles - tile;
    for (int q = r + 1; q < p.fold; ++q) n += (ld_const(p.req_cnt + b * p.fold + q) + kTile - 1) / kTile;
    return n;
  }
};

// bf16 stage layout (one 32-token tile, 36 KB, token-major, swizzled):
//   chunk c < 64 (dims 8c .. 8c + 7) of token t at byte 1024 t + 16 (c ^ swz(t)),
//   chunk c >= 64 (rope) at kRopeBase + 128 t + 16 ((c - 64) ^ rswz(t)).
// The LDS serves 64 banks of 4 bytes a cycle: 16 lanes of a 16-byte read,
// 32 lanes of an 8-byte read. swz permutes the 16 chunks of each 256-byte
// group so that 16 consecutive tokens put one chunk in 16 different places
// (the score reads), and the four tokens of a transposed V read land in four
// different 64-byte quarters; rswz does the same for the rope tails, two
// tokens to 256 bytes.
__host__ __device__ constexpr int chunk_swz(int t) { return 4 * (t & 3) + ((t >> 2) & 3); }
__host__ __device__ constexpr int rope_swz(int t) { return (t >> 1) & 7; }

// QK A operand of this wave's i-th k-step (see the kernel for the layout).
template <int kG>
__device__ __forceinline__ bf16x8_t qk_operand(const uint8_t* ks, uint32_t qk0, uint32_t rope0, int i) {
  return i / kG < 8 ? *(const bf16x8_t*)(ks + (qk0 ^ (32u * (i % kG) + 128u * (i / kG))))
                    : *(const bf16x8_t*)(ks + (rope0 ^ (32u * (i % kG))));
}

// PV operand of step st = 2 db + m (db local to the wave's slice): dims
// 32 db .. + 31 of tokens 16 m .. 16 m + 15 in the order of the P values,
// from two transposing loads of four tokens each (the second 8 tokens on,
// whose swizzle differs from the first's by 2: swz(t + 8) = swz(t) ^ 2,
// swz(t + 16) = swz(t)).
__device__ __forceinline__ bf16x8_t pv_operand(const uint8_t* ks, uint32_t pv0, int st) {
  const int db = st >> 1, m = st & 1;
  const uint32_t a = pv0 ^ (64u * db);
  const i16x4_t lo = lds_read_tr16(ks + a + 16384 * m);
  const i16x4_t hi = lds_read_tr16(ks + (a ^ 32u) + 8192 + 16384 * m);
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// max over lanes l and l ^ 32 (the two halves of a wave hold the two token
// halves of one query row)
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// tile rows and copies
// ---------------------------------------------------------------------------
// Rows that tokens read instead of the pool: zeros for tokens past a
// request's owned range (finite, and masked by the visibility limit) and NaN
// for a page id or row outside the pool (poisons the request's result rather
// than reading out of bounds).
struct ConstRows {
  uint32_t zero[kDqk / 2];       // 1152 bytes
  uint32_t nan_bf16[kDqk / 2];   // bf16 NaN 0x7FC0
  uint32_t nan_fp8[kDqk / 4];    // e4m3 NaN 0x7F
  constexpr ConstRows() : zero(), nan_bf16(), nan_fp8() {
    for (int i = 0; i < kDqk / 2; ++i) nan_bf16[i] = 0x7FC07FC0u;
    for (int i = 0; i < kDqk / 4; ++i) nan_fp8[i] = 0x7F7F7F7Fu;
  }
};
__device__ __attribute__((aligned(256))) const ConstRows g_const_rows;

// Table entries for the eight tokens 8 w .. 8 w + 7 a wave copies of a tile,
// read with scalar loads: the pages they fall in (block table; at most three
// for up to 16 shards) or their rows (local indices). Indices are clamped to
// the table row; entries of tokens past the owned range are never used.
struct TileEntries {
  int p0;
  int e0, e1, e2, e3, e4, e5, e6, e7;
};
template <bool kLocal>
__device__ __forceinline__ void load_entries(const DecodeParams& p, const Cursor& c, int wave, TileEntries& te) {
  const int j0 = c.tile * kTile + 8 * wave;
  if constexpr (kLocal) {
    const int32_t* base = p.local_kv_indices + (long long)c.b * p.local_kv_stride;
    const int last = p.local_kv_stride - 1;
    te.e0 = ld_const(base + min(j0 + 0, last));
    te.e1 = ld_const(base + min(j0 + 1, last));
    te.e2 = ld_const(base + min(j0 + 2, last));
    te.e3 = ld_const(base + min(j0 + 3, last));
    te.e4 = ld_const(base + min(j0 + 4, last));
    te.e5 = ld_const(base + min(j0 + 5, last));
    te.e6 = ld_const(base + min(j0 + 6, last));
    te.e7 = ld_const(base + min(j0 + 7, last));
    te.p0 = 0;
  } else {
    te.p0 = (j0 * p.num_shards + c.r) >> 6;
    const int32_t* base = p.block_table + (long long)c.b * p.max_pages;
    const int last = p.max_pages - 1;
    te.e0 = ld_const(base + min(te.p0 + 0, last));
    te.e1 = ld_const(base + min(te.p0 + 1, last));
    te.e2 = ld_const(base + min(te.p0 + 2, last));
    te.e3 = te.e4 = te.e5 = te.e6 = te.e7 = 0;
  }
}

// Source row of token 8 w + (lane >> 3) of the cursor's tile for copying
// wave w (valid: the tile exists in this workgroup's range).
template <bool kLocal, bool kFp8 = false>
__device__ __forceinline__ const uint8_t* token_src(const DecodeParams& p, const Cursor& c, bool valid,
                                                    const TileEntries& te, int wave) {
  constexpr long long kRowBytes = kFp8 ? kDqk : 2 * kDqk;
  const int lane = threadIdx.x & 63;
  const int tk = lane >> 3;
  const int j = c.tile * kTile + 8 * wave + tk;
  const uint8_t* zero = reinterpret_cast<const uint8_t*>(g_const_rows.zero);
  const uint8_t* nan = kFp8 ? reinterpret_cast<const uint8_t*>(g_const_rows.nan_fp8)
                            : reinterpret_cast<const uint8_t*>(g_const_rows.nan_bf16);
  if (!valid || j >= c.cnt) return zero;
  if constexpr (kLocal) {
    // e = entry tk, as a sum of differences (a select chain here is turned
    // into an indexed load from a stack copy)
    unsigned e = (unsigned)te.e0;
    e += tk >= 1 ? (unsigned)te.e1 - (unsigned)te.e0 : 0u;
    e += tk >= 2 ? (unsigned)te.e2 - (unsigned)te.e1 : 0u;
    e += tk >= 3 ? (unsigned)te.e3 - (unsigned)te.e2 : 0u;
    e += tk >= 4 ? (unsigned)te.e4 - (unsigned)te.e3 : 0u;
    e += tk >= 5 ? (unsigned)te.e5 - (unsigned)te.e4 : 0u;
    e += tk >= 6 ? (unsigned)te.e6 - (unsigned)te.e5 : 0u;
    e += tk >= 7 ? (unsigned)te.e7 - (unsigned)te.e6 : 0u;
    const int ei = (int)e;
    const bool ok = ei >= 0 && (long long)ei < (long long)p.num_pages * kPage;
    return ok ? p.kv + (long long)ei * kRowBytes : nan;
  } else {
    const int t = j * p.num_shards + c.r;
    const int d = (t >> 6) - te.p0;
    unsigned eu = (unsigned)te.e0;
    eu += d >= 1 ? (unsigned)te.e1 - (unsigned)te.e0 : 0u;
    eu += d >= 2 ? (unsigned)te.e2 - (unsigned)te.e1 : 0u;
    const int e = (int)eu;
    const bool ok = e >= 0 && e < p.num_pages;
    return ok ? p.kv + ((long long)e * kPage + (t & 63)) * kRowBytes : nan;
  }
}

// Copy j of a bf16 tile into a stage (the layout above):
// j = 0 moves the eight rope tails of the wave's tokens, j = 1 + i the 1 KB
// main part of token 8 w + i (one row per copy, as a scalar base).
template <int kJ, bool kNT>
__device__ __forceinline__ void copy_tile_part(const uint8_t* src, uint32_t stage_lds, int wave) {
  const int lane = threadIdx.x & 63;
  if constexpr (kJ == 0) {
    lds_dma16<kNT>(src + 16 * (64 + ((lane & 7) ^ rope_swz(8 * wave + (lane >> 3)))),
              __builtin_amdgcn_readfirstlane(stage_lds + kRopeBase + 1024 * wave));
  } else {
    constexpr int i = kJ - 1;
    const uint64_t a = reinterpret_cast<uint64_t>(src);
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)a, 8 * i);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(a >> 32), 8 * i);
    const uint8_t* base = reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
    lds_dma16_sbase<kNT>(base, (uint32_t)(16 * (lane ^ chunk_swz(8 * wave + i))),
                         __builtin_amdgcn_readfirstlane(stage_lds + 1024 * (8 * wave + i)));
  }
}
template <bool kNT>
__device__ __forceinline__ void copy_tile_part_rt(int j, const uint8_t* src, uint32_t stage_lds, int wave) {
  switch (j) {
    case 0: copy_tile_part<0, kNT>(src, stage_lds, wave); break;
    case 1: copy_tile_part<1, kNT>(src, stage_lds, wave); break;
    case 2: copy_tile_part<2, kNT>(src, stage_lds, wave); break;
    case 3: copy_tile_part<3, kNT>(src, stage_lds, wave); break;
    case 4: copy_tile_part<4, kNT>(src, stage_lds, wave); break;
    case 5: copy_tile_part<5, kNT>(src, stage_lds, wave); break;
    case 6: copy_tile_part<6, kNT>(src, stage_lds, wave); break;
    case 7: copy_tile_part<7, kNT>(src, stage_lds, wave); break;
    default: copy_tile_part<8, kNT>(src, stage_lds, wave); break;
  }
}

// ---------------------------------------------------------------------------
// fp8 tiles for the warp-specialised kernel: staged as stored, converted to
// bf16 in registers (exact: every e4m3 value is a bf16 value)
// ---------------------------------------------------------------------------
// Stage layout (18 KB): main chunk c (16 dims) of token t at
// 512 t + 16 (c ^ fp8_swz(t, c)), rope chunk r at kRope8 + 64 t +
// 16 (r ^ ((t >> 2) & 3)). The swizzle makes the 16-byte K reads of 16
// tokens and the transposing V reads of each half wave conflict free.
constexpr int kStage8 = kTile * kDqk;        // 18432
constexpr int kRope8 = kTile * 512;          // rope part of an fp8 stage
__host__ __device__ constexpr int fp8_swz(int t, int c) { return (t & 15) ^ (4 * (c & 1)); }

__device__ __forceinline__ bf16x8_t cvt_fp8x8(uint32_t w0, uint32_t w1) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t y0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2_t y1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2_t y2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2_t y3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8_t{y0[0], y0[1], y1[0], y1[1], y2[0], y2[1], y3[0], y3[1]};
}

// Copy j of an fp8 tile for copying wave w (tokens 8 w .. 8 w + 7; srcw:
// per lane the row of token 8 w + (lane >> 3)): j < 4 moves the 512-byte
// main parts of tokens 8 w + 2 j and + 1 (one per half wave), j = 4 the
// eight 64-byte rope tails (a half copy, 32 lanes).
template <int kJ, bool kNT>
__device__ __forceinline__ void copy8_tile_part(const uint8_t* srcw, uint32_t stage_lds, int wave) {
  const int lane = threadIdx.x & 63;
  const uint64_t a = reinterpret_cast<uint64_t>(srcw);
  if constexpr (kJ < 4) {
    const uint32_t lo0 = __builtin_amdgcn_readlane((uint32_t)a, 16 * kJ);
    const uint32_t hi0 = __builtin_amdgcn_readlane((uint32_t)(a >> 32), 16 * kJ);
    const uint32_t lo1 = __builtin_amdgcn_readlane((uint32_t)a, 16 * kJ + 8);
    const uint32_t hi1 = __builtin_amdgcn_readlane((uint32_t)(a >> 32), 16 * kJ + 8);
    const bool second = lane >= 32;
    const uint64_t row = second ? (((uint64_t)hi1 << 32) | lo1) : (((uint64_t)hi0 << 32) | lo0);
    const int t = 8 * wave + 2 * kJ + (second ? 1 : 0);
    const int pos = lane & 31, x = (pos ^ t) & 15;
    const int c = pos ^ (t & 15) ^ (4 * (x & 1));
    lds_dma16<kNT>(reinterpret_cast<const uint8_t*>(row) + 16 * c,
              __builtin_amdgcn_readfirstlane(stage_lds + 512 * (8 * wave + 2 * kJ)));
  } else {
    const int tl = (lane >> 2) & 7;
    const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)a, 8 * tl);
    const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(a >> 32), 8 * tl);
    const uint8_t* row = reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
    const int t = 8 * wave + tl;
    const int r = (lane & 3) ^ ((t >> 2) & 3);
    if (lane < 32) lds_dma16<kNT>(row + 512 + 16 * r, __builtin_amdgcn_readfirstlane(stage_lds + kRope8 + 512 * wave));
  }
}
template <bool kNT>
__device__ __forceinline__ void copy8_tile_part_rt(int j, const uint8_t* srcw, uint32_t stage_lds, int wave) {
  switch (j) {
    case 0: copy8_tile_part<0, kNT>(srcw, stage_lds, wave); break;
    case 1: copy8_tile_part<1, kNT>(srcw, stage_lds, wave); break;
    case 2: copy8_tile_part<2, kNT>(srcw, stage_lds, wave); break;
    case 3: copy8_tile_part<3, kNT>(srcw, stage_lds, wave); break;
    default: copy8_tile_part<4, kNT>(srcw, stage_lds, wave); break;
  }
}

// ---------------------------------------------------------------------------
// warp-specialised attention (64-row blocks)
// ---------------------------------------------------------------------------
// Eight waves, two per SIMD, in two roles (a second wave per SIMD to issue
// from while one waits on LDS; the register file holds both):
//  * waves 0..3 compute scores: wave (rg, ds) forms the partial S^T of row
//    group rg over half ds of the 576 QK dims; the ds = 1 wave hands its
//    partial to its partner through LDS, and the ds = 0 wave adds the two,
//    runs the online softmax (split into chunks between the next tile's
//    score MFMAs) and writes P (bf16, in the B-operand order of the PV
//    MFMAs) into the rope part of that tile's stage, which no wave reads
//    any more, with each row's rescale factor;
//  * waves 4..7 hold the output: wave 4 + q accumulates O^T for dims
//    128 q .. 128 q + 127 of all 64 rows (each V element is read from LDS
//    once per workgroup) and issues the tile copies (nine per barrier, so
//    the wait before each barrier is a constant vmcnt(9)).
// Tile i: barrier (tile i landed; copies of tile i + 2 go out) -> scores of
// tile i with the softmax of tile i - 1 | barrier | P V of tile i - 1.
// fp8 KV (kFp8): tiles stay fp8 in LDS (18 KB stages, five copies per wave
// and tile) and are converted in registers; K is read 16 bytes (two k-steps)
// per lane, V with ds_read_b64_tr_b8; P goes to a buffer of its own (the
// fp8 rope part is too small) and the output is staged in a region of its
// own.
constexpr int kWsRows = 64;
constexpr int kWsStagePitch = 272;     // output staging row: 128 bf16 + 16 bytes

template <bool kLocal, bool kFp8, bool kFold, bool kQ8, bool kNT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_ws_kernel(DecodeParams p) {
  static_assert(!kQ8 || kFp8, "an e4m3 query goes with an e4m3 KV pool");
  constexpr int kNS = 4;
  constexpr int kStageB = kFp8 ? kStage8 : kStageBytes;
  constexpr int kCopies = kFp8 ? 5 : 9;
  constexpr int kG = 2;                 // k-steps per 32-dim group of a score wave
  constexpr int kKS = 18;               // score MFMAs per wave and tile
  constexpr int kAhead = 4;
  constexpr int kChunks = 9;            // softmax chunks between score MFMAs
  constexpr int kPBytes = kWsRows * 32 * 2;                      // P of one tile (bf16)
  constexpr int kStgBytes = 4 * kWsRows * kWsStagePitch;         // output staging (fp8)
  constexpr int kSmem = kNS * kStageB + (kFp8 ? 2 * kPBytes + kStgBytes : 0);

  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmem];
  __shared__ __attribute__((aligned(16))) f32x4_t xbuf[2 * 4 * 64];   // [rg][4][lane]
  __shared__ float fbuf[2 * kWsRows];   // [tile parity][row]: rescale factor of the tile's P
  __shared__ float lbuf[kWsRows];       // row sums at the end of a piece

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tok = lane & 31, hi = lane >> 5;

  int g = blockIdx.x;
  if ((p.grid & 7) == 0) g = (blockIdx.x & 7) * (p.grid >> 3) + (blockIdx.x >> 3);
  const int32_t* rec = p.wg_rec + (long long)g * kRecInts;
  const int Uw = ld_const(rec);
  const int rec_seg = ld_const(rec + 1), rec_tile = ld_const(rec + 2), rec_cnt = ld_const(rec + 3);
  const int rec_seg1 = ld_const(rec + 4), rec_cnt1 = ld_const(rec + 5);
  if (Uw <= 0) return;
  const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(lds_address(smem));
  // P^T of tile u, row group r, token half m: 16 bytes per lane at
  // p_area(u) + 2048 r + 64 row + 16 ((2 m + hi) ^ ((row >> 2) & 3)), in the
  // rope part of the tile's stage (bf16) or a buffer per tile parity (fp8)
  auto p_area = [&](int u) -> uint8_t* {
    if constexpr (kFp8) return smem + kNS * kStageB + (u & 1) * kPBytes;
    else return smem + kStageB * (u & (kNS - 1)) + kRopeBase;
  };
  const uint32_t poff = (uint32_t)(64 * tok);
  const int pswz = (tok >> 2) & 3;

  if (wave < 4) {
    // ------------------------------------------------------------ scores
    const int rg = wave & 1, ds = wave >> 1;
    const uint32_t qk0 = (uint32_t)(1024 * tok + 16 * ((2 * kG * ds + hi) ^ chunk_swz(tok)));
    const uint32_t rope0 = (uint32_t)(kRopeBase + 128 * tok + 16 * ((2 * kG * ds + hi) ^ rope_swz(tok)));
    // fp8: score step i = 2 j + u uses 16-dim chunk 2 m + hi of the lane's
    // token, m = 2 j + ds (m = 16, 17: rope), its 8-byte half u; the query
    // registers follow the same order of the dims
    const uint32_t qk8 = (uint32_t)(512 * tok + 16 * (hi ^ (tok & 15) ^ (4 * hi)));
    const uint32_t rope8 = (uint32_t)(kRope8 + 64 * tok + 16 * ((2 * ds + hi) ^ ((tok >> 2) & 3)));
    Cursor cc;
    cc.start_known(p, rec_seg, rec_tile, rec_cnt);
    bf16x8_t qreg[kKS];
    // e4m3 query (kQ8): the B operands of this wave's five fp8 MFMAs, each
    // 32 codes a lane: dims 32 m0 + 16 hi .. + 15 and 32 m1 + 16 hi .. + 15
    // with (m0, m1) = (4 j + ds, 4 j + 2 + ds) for j < 4, and the rope group
    // m0 = 16 + ds with a zero second half for j = 4; the A operand of MFMA
    // j holds the same dims of the lane's token (k8_load of 2 j and 2 j + 1)
    typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
    i32x8_t q8reg[5];
    bf16x8_t ka[kAhead];
    u32x4_t kraw[2];
    f32x16_t acc;
    auto k8_load = [&](const uint8_t* ks, int j) -> u32x4_t {
      const int m = 2 * j + ds;
      return m < 16 ? *(const u32x4_t*)(ks + (qk8 ^ (32u * (uint32_t)m))) : *(const u32x4_t*)(ks + rope8);
    };
    auto qk_start = [&](const uint8_t* ks) {
      if constexpr (kFp8) {
        kraw[0] = k8_load(ks, 0);
        kraw[1] = k8_load(ks, 1);
      } else {
#pragma unroll
        for (int u = 0; u < kAhead; ++u) ka[u] = qk_operand<kG>(ks, qk0, rope0, u);
      }
      acc = f32x16_t{};
    };
    auto qk_step = [&](const uint8_t* ks, int i) {
      if constexpr (kQ8) {
        // fp8 MFMA j after step 4 j + 1 (and the last after step 17); the
        // next MFMA's K bytes are read right after it is issued
        if (i % 4 == 1 || i == kKS - 1) {
          const int j = i / 4;
          const i32x8_t a = {(int32_t)kraw[0][0], (int32_t)kraw[0][1], (int32_t)kraw[0][2], (int32_t)kraw[0][3],
                             (int32_t)kraw[1][0], (int32_t)kraw[1][1], (int32_t)kraw[1][2], (int32_t)kraw[1][3]};
          acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, q8reg[j], acc, 0, 0, 0, 127, 0, 127);
          if (j < 4) {
            kraw[0] = k8_load(ks, 2 * j + 2);
            kraw[1] = k8_load(ks, 2 * j + 3);
          }
        }
      } else if constexpr (kFp8) {
        const int j = i >> 1, u = i & 1;
        const bf16x8_t a = cvt_fp8x8(kraw[j & 1][2 * u], kraw[j & 1][2 * u + 1]);
        if (u == 1 && j + 2 < kKS / 2) kraw[j & 1] = k8_load(ks, j + 2);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[i], acc, 0, 0, 0);
      } else {
        const bf16x8_t a = ka[i % kAhead];
        if (i + kAhead < kKS) ka[i % kAhead] = qk_operand<kG>(ks, qk0, rope0, i + kAhead);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[i], acc, 0, 0, 0);
      }
    };
    f32x4_t* xmine = xbuf + (rg * 4) * 64 + lane;
    // launch of every shard, row-block groups: the workgroups of a group walk
    // the same tiles for their row blocks, and each tile comes from HBM once
    // only while they stay close (the later one reads it from L2). Over long
    // walks their clocks drift them apart, so every kSyncTiles tiles one
    // partner score wave of each adds to the group's counter and waits, a
    // bounded number of polls, for the others to arrive; the barrier after
    // it holds the whole workgroup. It paces only: the results do not
    // depend on it, and a partner that never comes costs kSyncPolls polls.
    constexpr int kSyncTiles = 64;
    constexpr int kSyncPolls = 8;
    auto rendezvous = [&](int tile) {
      if (p.rgroup > 1 && wave == 2 && tile > 0 && tile % kSyncTiles == 0) {
        if (lane == 0) {
          int32_t* ctr = p.grp_sync + g / p.rgroup;
          const int target = (tile / kSyncTiles) * p.rgroup;
          __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          for (int i = 0; i < kSyncPolls; ++i) {
            if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) break;
            __builtin_amdgcn_s_sleep(16);
          }
        }
      }
    };

    int t = 0;
    while (t < Uw) {
      const int b = cc.b, rb = cc.rb, tile0 = cc.tile, ntiles = cc.ntiles, cnt = cc.cnt, sh = cc.r, seg = cc.seg;
      // a piece: the rest of the segment, or, when the launch runs every
      // shard, the rest of the row block's run over its shards (the online
      // softmax simply continues over the next shard's tokens)
      const int n = min(kFold ? cc.run_units(p) : ntiles - tile0, Uw - t);
      const int row = rb * kWsRows + rg * 32 + tok;
      const bool row_ok = row < p.rows;
      if constexpr (kQ8) {
        const long long qn = (long long)b * p.rows + (row_ok ? row : 0);
        const uint8_t* qrow8 = p.q8 + qn * p.q8_stride + 16 * hi;
#pragma unroll
        for (int j = 0; j < 5; ++j) {
          const u32x4_t x0 = *(const u32x4_t*)(qrow8 + 32 * (j < 4 ? 4 * j + ds : 16 + ds));
          const u32x4_t x1 = j < 4 ? *(const u32x4_t*)(qrow8 + 32 * (4 * j + 2 + ds)) : u32x4_t{};
          const i32x8_t x = {(int32_t)x0[0], (int32_t)x0[1], (int32_t)x0[2], (int32_t)x0[3],
                             (int32_t)x1[0], (int32_t)x1[1], (int32_t)x1[2], (int32_t)x1[3]};
          q8reg[j] = row_ok ? x : i32x8_t{};
        }
      } else {
        const long long qn = (long long)b * p.rows + (row_ok ? row : 0);
        const uint16_t* qrow = p.q + qn * p.q_stride;
        const uint16_t* rrow = p.q_rope + qn * p.q_rope_stride - 512;
#pragma unroll
        for (int i = 0; i < kKS; ++i) {
          int d0;
          if constexpr (kFp8) d0 = 32 * (2 * (i >> 1) + ds) + 16 * hi + 8 * (i & 1);
          else d0 = 16 * (4 * (i / kG) + kG * ds + i % kG) + 8 * hi;
          // steps 0..15 read latent dims (< 512), steps 16, 17 rope dims
          const bf16x8_t x = *(const bf16x8_t*)((i < 16 ? qrow : rrow) + d0);
          qreg[i] = row_ok ? x : bf16x8_t{};
        }
      }
      wait_vmcnt<0>();
      // owned tokens row (draft i) may see: t = j S + r <= L - q_b + i, with
      // q_b the request's decode depth (rows i >= q_b are padding: none)
      int L = ld_const(p.seq_lens + b);
      L = L < 0 ? 0 : min(L, p.max_pages * kPage);
      int qb = p.q_len;
      if (p.q_lens != nullptr) {
        qb = ld_const(p.q_lens + b);
        qb = qb < 0 ? 0 : (qb > p.q_len ? p.q_len : qb);
      }
      const int di = (row >= p.heads) + (row >= 2 * p.heads) + (row >= 3 * p.heads);
      auto jvis_of = [&](int shv, int cntv) {
        int jv = 0;
        for (int k = 0; k < p.q_len; ++k) {
          const int lim = L - qb + k - shv;
          const int jl = lim >= 0 ? min(cntv, lim / p.num_shards + 1) : 0;
          jv = di == k && k < qb ? jl : jv;
        }
        return jv;
      };
      const int jvis = jvis_of(sh, cnt);
      // kFold: the visibility limit of each tile of the piece, from a cursor
      // over its tiles (the shard changes within a piece)
      Cursor cs = cc;
      int jv_sh = sh, jv_cur = jvis, limk = 0;
      auto next_lim = [&](int k) {
        if (cs.r != jv_sh) {
          jv_sh = cs.r;
          jv_cur = jvis_of(cs.r, cs.cnt);
        }
        limk = jv_cur - cs.tile * kTile;
        if (k + 1 < n) cs.template advance<kFold>(p);
      };
      float m_ref = kNegInf, l_sum = 0.f;
      // online softmax of a tile in base 2 (lane: one row, 16 tokens; value
      // v is token 8 (v >> 2) + 4 hi + (v & 3)); tokens at or past the row's
      // visibility limit are masked; the max is taken on the raw scores and
      // the scale folded into the exponent's FMA. Chunks 0 and 1 mask and
      // take the max (and move the reference), the rest exponentiate.
      float f = 1.f, tmax = kNegInf, neg_m = 0.f;
      int lim = 0;
      auto softmax_chunk = [&](int c, int k, f32x16_t& sc, bf16x8_t (&pb)[2]) {
        if (c == 0) {
          lim = (kFold ? limk : jvis - (tile0 + k) * kTile) - 4 * hi;
          tmax = kNegInf;
        }
        if (c < 2) {
#pragma unroll
          for (int v = 8 * c; v < 8 * c + 8; ++v) {
            const int cc_ = 8 * (v >> 2) + (v & 3);
            sc[v] = cc_ < lim ? sc[v] : kNegInf;
            tmax = fmaxf(tmax, sc[v]);
          }
        }
        if (c == 1) {
          const float tm = xor32_max(tmax) * p.scale_log2;
          const bool grow = m_ref != kNegInf && tm > m_ref + kRescaleSlack;
          f = grow ? exp2_fast(m_ref - tm) : 1.f;
          l_sum *= f;
          m_ref = grow || m_ref == kNegInf ? tm : m_ref;
          neg_m = m_ref == kNegInf ? 0.f : -m_ref;
        }
        if (c >= 2) {
          // pairs of probabilities rounded to bf16 together; the row sum
          // adds the rounded pair (v_dot2c_f32_bf16 with {1, 1}), i.e. the
          // values the P V product takes, so the output is an exact weighted
          // mean of V rows. Against the unrounded sum this halves the largest
          // error on short contexts, where outputs are as large as single V
          // rows (a CPU model of this arithmetic on the skewed workload's
          // shortest requests: ~0.019 -> ~0.011), and it is one instruction
          // per pair instead of two additions
          constexpr int kE = kChunks - 2;
          typedef float f32x2_t __attribute__((ext_vector_type(2)));
          typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
          const int v0 = 2 * ((c - 2) * 8 / kE), v1 = 2 * ((c - 1) * 8 / kE);
#pragma unroll
          for (int v = 0; v < 16; v += 2) {
            if (v >= v0 && v < v1) {
              const f32x2_t pr = {exp2_fast(__builtin_fmaf(sc[v], p.scale_log2, neg_m)),
                                  exp2_fast(__builtin_fmaf(sc[v + 1], p.scale_log2, neg_m))};
              const bf16x2v_t pk = __builtin_convertvector(pr, bf16x2v_t);
              l_sum = __builtin_amdgcn_fdot2_f32_bf16(pk, bf16x2v_t{(__bf16)1.f, (__bf16)1.f}, l_sum, false);
              pb[v >> 3][v & 7] = pk[0];
              pb[v >> 3][(v & 7) + 1] = pk[1];
            }
          }
        }
      };
      // P of tile u into the rope part of its stage, and the row's factor
      auto write_p = [&](int u, const bf16x8_t (&pb)[2]) {
        uint8_t* st = p_area(u) + poff + 2048 * rg;
#pragma unroll
        for (int m = 0; m < 2; ++m) *(bf16x8_t*)(st + 16 * ((2 * m + hi) ^ pswz)) = pb[m];
        if (hi == 0) fbuf[(u & 1) * kWsRows + rg * 32 + tok] = f;
      };
      auto partner_sum = [&]() {
        f32x16_t r;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4_t v = xmine[64 * q];
#pragma unroll
          for (int e = 0; e < 4; ++e) r[4 * q + e] = acc[4 * q + e] + v[e];
        }
        return r;
      };

      f32x16_t s_cur;
      // tile 0: its scores
      if constexpr (kFold) rendezvous(t);
      __syncthreads();   // tile t landed
      {
        const uint8_t* ksq = smem + kStageB * (t & (kNS - 1));
        qk_start(ksq);
#pragma unroll
        for (int i = 0; i < kKS; ++i) qk_step(ksq, i);
        if (ds == 1) {
#pragma unroll
          for (int q = 0; q < 4; ++q) xmine[64 * q] = f32x4_t{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
        }
      }
      __syncthreads();   // partials exchanged
      if (ds == 0) s_cur = partner_sum();
      for (int k = 0; k + 1 < n; ++k) {
        if constexpr (kFold) rendezvous(t + k + 1);
        __syncthreads();   // tile t + k + 1 landed
        const uint8_t* ksq = smem + kStageB * ((t + k + 1) & (kNS - 1));
        qk_start(ksq);
        if (ds == 0) {
          if constexpr (kFold) next_lim(k);
          bf16x8_t pb[2];
#pragma unroll
          for (int i = 0; i < kKS; ++i) {
            qk_step(ksq, i);
            if (i % 2 == 1) softmax_chunk(i / 2, k, s_cur, pb);
            __builtin_amdgcn_sched_barrier(0);
          }
          write_p(t + k, pb);
        } else {
#pragma unroll
          for (int i = 0; i < kKS; ++i) qk_step(ksq, i);
#pragma unroll
          for (int q = 0; q < 4; ++q) xmine[64 * q] = f32x4_t{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
        }
        __syncthreads();   // P of tile t + k and the partials exchanged
        if (ds == 0) s_cur = partner_sum();
      }
      // the last tile's softmax; row sums and LSE of the piece (finalised in
      // place when this workgroup holds the whole segment of a one-shard launch)
      const bool single = !kFold && tile0 == 0 && n == ntiles;
      if (ds == 0) {
        if constexpr (kFold) next_lim(n - 1);
        bf16x8_t pb[2];
#pragma unroll
        for (int c = 0; c < kChunks; ++c) softmax_chunk(c, n - 1, s_cur, pb);
        write_p(t + n - 1, pb);
        const float l_tot = xor32_sum(l_sum);
        if (hi == 0) lbuf[rg * 32 + tok] = l_tot;
        const bool any = l_tot > 0.f || l_tot != l_tot;
        const float lse2 = any ? m_ref + log2_fast(l_tot) : kNegInf;
        if (row_ok && hi == 0) {
          if (single) {
            p.lse[(long long)b * p.rows + row] = p.lse_base2 ? lse2 : lse2 * kLn2;
          } else {
            const int4 si = ld_const(p.seg_info + seg);
            p.spart_lse[(long long)(si.x + g / p.rgroup - si.z) * kWsRows + (row - rb * kWsRows)] = lse2;
          }
        }
      }
      __syncthreads();   // P of the last tile and the row sums written
      __syncthreads();   // every output wave is done with the stages
      t += n;
      if (t < Uw) {
        if constexpr (kFold) {
          cc.template advance_by<kFold>(p, n);
        } else {
          cc.tile = ntiles - 1;
          cc.template advance<kFold>(p);
        }
      }
    }
    wait_vmcnt<0>();
  } else {
    // ------------------------------------------------------------ output
    const int wq = wave - 4;
    uint32_t pv0;
    {
      const int g16 = lane >> 4, r4 = (lane >> 2) & 3, q4 = lane & 3;
      const int tl = 4 * (g16 >> 1) + r4;
      const int y = 2 * (g16 & 1) + (q4 >> 1);
      pv0 = (uint32_t)(1024 * tl + 16 * (y ^ chunk_swz(tl)) + 8 * (q4 & 1) + 256 * wq);
    }
    // fp8 V^T operands (ds_read_b64_tr_b8): lane i of each 16-lane group G
    // points at the 8 dims 32 db + 16 (G & 1) + 8 (i & 1) (of the wave's
    // slice) of token 8 (e >> 2) + 4 (G >> 1) + (e & 3), e = i >> 1 (+ 16 for
    // the second token half), so that lane l receives 8 tokens of dim l & 31
    // in the order of the P values
    uint32_t pv8[4];
    {
      const int G = lane >> 4, i = lane & 15, e = i >> 1;
      const int tl = 8 * (e >> 2) + 4 * (G >> 1) + (e & 3);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int c = 8 * wq + 2 * db + (G & 1);
        pv8[db] = (uint32_t)(512 * tl + 16 * (c ^ fp8_swz(tl, c)) + 8 * (i & 1));
      }
    }
    auto copy_part = [&](int j, const uint8_t* src, uint32_t st) {
      if constexpr (kFp8) copy8_tile_part_rt<kNT>(j, src, st, wq);
      else copy_tile_part_rt<kNT>(j, src, st, wq);
    };
    Cursor cc, cl;
    cc.start_known(p, rec_seg, rec_tile, rec_cnt);
    cl = cc;
    if (1 < Uw) {
      if (cl.tile + 1 < cl.ntiles) ++cl.tile;
      else cl.start_known(p, rec_seg1, 0, rec_cnt1);
    }
    {
      TileEntries te0, te1;
      load_entries<kLocal>(p, cc, wq, te0);
      if (1 < Uw) load_entries<kLocal>(p, cl, wq, te1);
      const uint8_t* src0 = token_src<kLocal, kFp8>(p, cc, true, te0, wq);
#pragma unroll
      for (int j = 0; j < kCopies; ++j) copy_part(j, src0, smem_lds);
      const uint8_t* src1 = token_src<kLocal, kFp8>(p, cl, 1 < Uw, te1, wq);
#pragma unroll
      for (int j = 0; j < kCopies; ++j) copy_part(j, src1, smem_lds + kStageB);
    }
    int ncopied = 2;
    TileEntries te;
    if (2 < Uw) {
      cl.template advance<kFold>(p);
      load_entries<kLocal>(p, cl, wq, te);
    }
    // tile barrier: the next scores' tile has landed in every wave and the
    // stage of the tile two back is free: the copies of tile ncopied go out
    auto tile_barrier = [&]() {
      wait_vmcnt<kCopies>();
      __syncthreads();
      const uint8_t* csrc = token_src<kLocal, kFp8>(p, cl, ncopied < Uw, te, wq);
      const uint32_t cst = __builtin_amdgcn_readfirstlane(smem_lds + kStageB * (ncopied & (kNS - 1)));
#pragma unroll
      for (int j = 0; j < kCopies; ++j) copy_part(j, csrc, cst);
      ++ncopied;
      if (ncopied < Uw) {
        cl.template advance<kFold>(p);
        load_entries<kLocal>(p, cl, wq, te);
      }
    };
    f32x16_t o[4][2];
    bf16x8_t va[8];
    auto load_v = [&](const uint8_t* ks) {
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        if constexpr (kFp8) {
          typedef int32_t i32x2_t __attribute__((ext_vector_type(2)));
          const i32x2_t x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) i32x2_t*)(ks + pv8[st >> 1] + 8192 * (st & 1)));
          va[st] = cvt_fp8x8((uint32_t)x[0], (uint32_t)x[1]);
        } else {
          va[st] = pv_operand(ks, pv0, st);
        }
      }
    };
    // O^T[dim][row] += V^T[dim][token] P^T[token][row] for both row groups,
    // after the rows' rescale (f = 1 unless the reference moved)
    auto pv_tile = [&](int u) {
      const float f0 = fbuf[(u & 1) * kWsRows + tok];
      const float f1 = fbuf[(u & 1) * kWsRows + 32 + tok];
      const uint8_t* pa = p_area(u) + poff;
      bf16x8_t pp[2][2];
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int m = 0; m < 2; ++m)
          pp[r][m] = *(const bf16x8_t*)(pa + 2048 * r + 16 * ((2 * m + hi) ^ pswz));
      if (__builtin_expect(__ballot(f0 != 1.f) != 0, 0)) {
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db][0] *= f0;
      }
      if (__builtin_expect(__ballot(f1 != 1.f) != 0, 0)) {
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db][1] *= f1;
      }
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 2; ++r)
            o[db][r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[2 * db + m], pp[r][m], o[db][r], 0, 0, 0);
    };

    int t = 0;
    while (t < Uw) {
      const int b = cc.b, rb = cc.rb, tile0 = cc.tile, ntiles = cc.ntiles, seg = cc.seg;
      const int n = min(kFold ? cc.run_units(p) : ntiles - tile0, Uw - t);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 2; ++r) o[db][r] = f32x16_t{};
      tile_barrier();    // tile t landed
      __syncthreads();   // partials exchanged
      for (int k = 0; k + 1 < n; ++k) {
        tile_barrier();  // tile t + k + 1 landed
        const uint8_t* ksv = smem + kStageB * ((t + k) & (kNS - 1));
        load_v(ksv);
        __syncthreads();   // P of tile t + k written
        pv_tile(t + k);
      }
      {
        const uint8_t* ksv = smem + kStageB * ((t + n - 1) & (kNS - 1));
        load_v(ksv);
        __syncthreads();   // P of the last tile and the row sums written
        pv_tile(t + n - 1);
      }
      const float l0 = lbuf[tok], l1 = lbuf[32 + tok];
      __syncthreads();   // every output wave is done with the stages
      // epilogue: lane l holds rows r * 32 + (l & 31); o[db][r][v] is dim
      // 128 wq + 32 db + 8 (v >> 2) + 4 hi + (v & 3). The rows are stored
      // non-temporally: nothing in this launch reads them again, and rows
      // left dirty in the XCDs' L2 caches would all be written back when the
      // launch ends (kimi-like shard 34.8 -> 32.3 µs, fp8 52 -> 50 µs)
      float inv[2];
      {
        const bool a0 = l0 > 0.f || l0 != l0, a1 = l1 > 0.f || l1 != l1;
        inv[0] = a0 ? p.out_scale / l0 : 0.f;
        inv[1] = a1 ? p.out_scale / l1 : 0.f;
      }
      const bool single = !kFold && tile0 == 0 && n == ntiles;
      const int row0 = rb * kWsRows;
      if (single && !p.out_bf16) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int row = row0 + r * 32 + tok;
          if (row < p.rows) {
            float* dst = (float*)p.out + ((long long)b * p.rows + row) * kDv + 128 * wq + 4 * hi;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const f32x4_t x = {o[db][r][4 * q] * inv[r], o[db][r][4 * q + 1] * inv[r],
                                   o[db][r][4 * q + 2] * inv[r], o[db][r][4 * q + 3] * inv[r]};
                __builtin_nontemporal_store(x, (f32x4_t*)(dst + 32 * db + 8 * q));
              }
          }
        }
      } else {
        // bf16 rows through LDS (bf16: the stages of the piece's last two
        // tiles, which are free; fp8: a region of its own): 64 rows x 128
        // dims per wave, stored 16 bytes a lane
        uint8_t* sb;
        if constexpr (kFp8) sb = smem + kNS * kStageB + 2 * kPBytes + wq * (kWsRows * kWsStagePitch);
        else sb = smem + kStageB * ((t + n - 1 - (wq >> 1)) & (kNS - 1)) + (wq & 1) * (kWsRows * kWsStagePitch);
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const bf16x4_t x = {(__bf16)(o[db][r][4 * q] * inv[r]), (__bf16)(o[db][r][4 * q + 1] * inv[r]),
                                  (__bf16)(o[db][r][4 * q + 2] * inv[r]), (__bf16)(o[db][r][4 * q + 3] * inv[r])};
              *(bf16x4_t*)(sb + kWsStagePitch * (r * 32 + tok) + 2 * (32 * db + 8 * q + 4 * hi)) = x;
            }
        __bf16* obase;
        if (single) {
          obase = (__bf16*)p.out + ((long long)b * p.rows + row0) * kDv;
        } else {
          const int4 si = ld_const(p.seg_info + seg);
          obase = (__bf16*)p.spart_o + ((long long)(si.x + g / p.rgroup - si.z) * kWsRows) * kDv;
        }
        const int rr0 = lane >> 4, c16 = lane & 15;
#pragma unroll
        for (int i = 0; i < kWsRows / 4; ++i) {
          const int rr = 4 * i + rr0;
          const bf16x8_t x = *(const bf16x8_t*)(sb + kWsStagePitch * rr + 16 * c16);
          if (row0 + rr < p.rows) __builtin_nontemporal_store(x, (bf16x8_t*)(obase + (long long)rr * kDv + 128 * wq + 8 * c16));
        }
        // the staging writes are complete before the next barrier on every
        // control path (the reads above wait for them only where a row's
        // store runs; row 0 always does, but the compiler cannot know it)
        wait_lgkmcnt0();
      }
      t += n;
      if (t < Uw) {
        if constexpr (kFold) {
          cc.template advance_by<kFold>(p, n);
        } else {
          cc.tile = ntiles - 1;
          cc.template advance<kFold>(p);
        }
      }
    }
    // no copy may still be writing this workgroup's LDS when it exits
    wait_vmcnt<0>();
  }
}

template <bool kNT>
const void* pick_ws_kernel(bool fp8, bool q8, bool fold, bool local) {
  if (fp8 && q8)
    return fold    ? reinterpret_cast<const void*>(&attn_ws_kernel<false, true, true, true, kNT>)
           : local ? reinterpret_cast<const void*>(&attn_ws_kernel<true, true, false, true, kNT>)
                   : reinterpret_cast<const void*>(&attn_ws_kernel<false, true, false, true, kNT>);
  if (fp8)
    return fold    ? reinterpret_cast<const void*>(&attn_ws_kernel<false, true, true, false, kNT>)
           : local ? reinterpret_cast<const void*>(&attn_ws_kernel<true, true, false, false, kNT>)
                   : reinterpret_cast<const void*>(&attn_ws_kernel<false, true, false, false, kNT>);
  return fold    ? reinterpret_cast<const void*>(&attn_ws_kernel<false, false, true, false, kNT>)
         : local ? reinterpret_cast<const void*>(&attn_ws_kernel<true, false, false, false, kNT>)
                 : reinterpret_cast<const void*>(&attn_ws_kernel<false, false, false, false, kNT>);
}

}  // namespace

hipError_t launch_decode_plan(const DecodeParams& p, hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(stream_plan_kernel, dim3(1), dim3(1024), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_stream(const DecodeParams& p, bool run_plan, hipEvent_t ev_begin, hipEvent_t ev_end,
                                hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  hipError_t err = run_plan ? launch_decode_plan(p, stream) : hipSuccess;
  if (err != hipSuccess) return err;
  // the events, when given, take the attention kernel's own start and end
  // times (recorded with the dispatch, no separate marker packets)
  void* args[] = {const_cast<DecodeParams*>(&p)};
  const void* fn;
  // the launch of every shard reads the global block table (no shard
  // metadata) and is an instantiation of its own
  const bool local = p.local_kv_indices != nullptr;
  const bool fold = p.fold > 1;
  if (fold && local) return hipErrorInvalidValue;
  // streaming (non-temporal) tile copies when no other workgroup reads the
  // same tiles (one row block per request): the KV stream then does not
  // evict the lines that are read again (block table, queries) from the
  // caches (kimi-like per-shard kernel ~+5%, single launch ~-10%); row-block
  // groups read each tile from L2 after their first member, so they keep the
  // default policy (streaming there: MTP +3-6%, skewed +1.5-3%)
  fn = p.rgroup == 1 ? pick_ws_kernel<true>(p.kv_fp8, p.q8 != nullptr, fold, local)
                     : pick_ws_kernel<false>(p.kv_fp8, p.q8 != nullptr, fold, local);
  err = hipExtLaunchKernel(fn, dim3(p.grid), dim3(512), args, 0, stream, ev_begin, ev_end, 0);
  if (err != hipSuccess) return err;
  return launch_combine(p, stream);
}

}  // namespace mla
