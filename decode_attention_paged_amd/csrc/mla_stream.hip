// Rank-local paged MLA decode: persistent streaming kernels.
//
// One shard r of S owns the tokens t = j S + r of every request (prhub.com.cn
// digest of sgl-project/sglang PR 33926, sections 功能与动机 and 实现拆解
// step 3); this file computes, for each query row, softmax attention over
// those tokens and emits the rank-local (out, lse), (0, -inf) where a row
// sees no owned token.
//
// Schedule. The shard's work is a sequence of units (request b, block of
// query rows rb, 32-token tile), ordered by segment s = b * row_blocks + rb
// and tile. stream_plan_kernel lays the segments out on device (no host
// synchronisation) and one workgroup per CU takes a contiguous share of the
// units of about equal cost. A segment that a workgroup holds entirely is
// finalised in place; a segment cut at workgroup boundaries leaves one bf16
// partial per piece, combined by stream_combine_kernel.
//
// Workgroup. Four waves: rows_blk / 32 row groups of 32 query rows times
// 4 / (rows_blk / 32) slices of the 512 V dims. The waves of a row group
// split the 576 QK dims and exchange their partial scores through LDS
// (S^T = K Q^T, v_mfma_f32_32x32x16_bf16); each wave then accumulates the
// output of its dims slice.
//
// bf16 KV (attn_pipe_kernel). Tiles move HBM -> LDS with
// global_load_lds_dwordx4 (no register staging) through four 36 KB stages;
// the row of every token comes from the block table by scalar loads, and
// out-of-pool pages point the copy at a constant NaN row. The loop overlaps
// two tiles: the scores of tile k + 1 run with tile k's softmax on the VALU
// and then with tile k's accumulation (O^T += V^T P^T) on the MFMAs.
//
// fp8 KV (attn_stream_kernel<.., true>). Tiles are staged as stored (five
// 18 KB stages), converted to a bf16 compute stage, and the row indices move
// into an LDS ring 2 * 5 - 2 tiles ahead; every vector-memory operation in
// the tile loop is an asynchronous copy and the loop waits on exactly the
// tile it needs (s_waitcnt vmcnt(n) with n counted by the wave).
#include "mla_device.h"

#include <hip/hip_ext.h>

#include <limits.h>
#include <type_traits>

namespace mla {
namespace {

constexpr int kStageBytes = kTile * kDqk * 2;      // 36864: one tile
constexpr int kRopeBase = kTile * 1024;             // rope part of a stage (dims 512..575)
constexpr int kStageBytes8 = kTile * kDqk;          // 18432: one fp8 tile as stored
constexpr int kRing = 16;                          // row-index ring, in tiles
// A row's exponent reference moves up (rescaling its accumulator) only when a
// tile's max exceeds it by more than this (log2 units), so rescaling is rare
// and unnormalised probabilities stay below 2^kRescaleSlack.
constexpr float kRescaleSlack = 8.0f;

constexpr int kPieceCost = 3;     // query load + epilogue of a piece, in tiles

constexpr int kRowPastEnd = -2;   // token past the request's owned range
constexpr int kRowBad = -1;       // page id or row outside the pool


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

__device__ __forceinline__ int seg_tiles(const DecodeParams& p, int s) {
  const int b = s / p.row_blocks;
  return (local_count(p, b) + kTile - 1) / kTile;
}

// One workgroup of 1024 threads; thread i handles a contiguous block of
// segments. The segment offsets stay in LDS when they fit (the binary
// searches then cost LDS latency only), else in the workspace.
constexpr int kPlanLdsSegs = 6144;

__global__ __launch_bounds__(1024) void stream_plan_kernel(DecodeParams p) {
  __shared__ int32_t s_arr[2 * (kPlanLdsSegs + 1)];
  __shared__ int32_t s_cnt[kPlanLdsSegs];           // owned tokens per segment's request
  __shared__ int32_t s_wgu[kMaxGrid + 1];
  __shared__ int2 s_wave[16];
  const int tid = threadIdx.x;
  const int RB = p.row_blocks;
  const int nseg = p.batch * RB;
  const bool in_lds = nseg <= kPlanLdsSegs;
  int32_t* const off = in_lds ? s_arr : p.seg_off;              // unit offset of each segment
  int32_t* const coff = in_lds ? s_arr + kPlanLdsSegs + 1 : p.seg_coff;   // cost offset
  const int per = (nseg + 1023) / 1024;
  const int s0 = min(tid * per, nseg), s1 = min(s0 + per, nseg);

  // tiles and costs (a segment costs its tiles plus kPieceCost for loading
  // its queries) of this thread's segments, scanned over the block
  int su = 0, sc = 0;
  for (int s = s0; s < s1; ++s) {
    const int b = s / RB;
    const int cnt = local_count(p, b);
    if (s - b * RB == 0) p.req_cnt[b] = cnt;
    if (in_lds) s_cnt[s] = cnt;
    const int n = (cnt + kTile - 1) / kTile;
    su += n;
    sc += n > 0 ? n + kPieceCost : 0;
  }
  int2 tot;
  const int2 ex = block_excl_scan2(su, sc, s_wave, tot);
  {
    int u = ex.x, c = ex.y;
    for (int s = s0; s < s1; ++s) {
      const int n = seg_tiles(p, s);
      off[s] = u;
      coff[s] = c;
      u += n;
      c += n > 0 ? n + kPieceCost : 0;
    }
  }
  const int U = tot.x, C = tot.y;
  // workgroups in use: at most one per cost unit, so consecutive workgroup
  // boundaries differ and only a piece's first workgroup can start inside
  // its query-load cost
  const int G = min(p.grid, C);
  if (tid == 0) {
    off[nseg] = U;
    coff[nseg] = C;
    p.plan[0] = U;
    p.plan[1] = G;
    s_wgu[G] = U;
    p.wg_ustart[G] = U;
  }
  __syncthreads();

  // first unit of each workgroup: cost boundary g C / G mapped to the unit
  // sequence (a boundary inside a segment's query cost maps to its first tile)
  for (int g = tid; g < G; g += 1024) {
    const long long x = (long long)g * C / G;
    const int s = last_le(coff, nseg + 1, x);
    const int n = off[s + 1] - off[s];
    long long k = x - coff[s] - kPieceCost;
    k = k < 0 ? 0 : (k > n - 1 ? n - 1 : k);
    s_wgu[g] = off[s] + (int)k;
    p.wg_ustart[g] = off[s] + (int)k;
    p.wg_start[g] = make_int2(s, (int)k);
  }
  __syncthreads();

  // start record of each workgroup: its range, its first unit with the
  // owned-token count of that request, and the segment (with its count) of
  // the unit after its first segment, so that the decode kernel resolves
  // the rows of its first two tiles after a single round of loads
  for (int w = tid; w < p.grid; w += 1024) {
    int32_t* rec = p.wg_rec + (long long)w * kRecInts;
    const int u0 = w < G ? s_wgu[w] : 0, u1 = w < G ? s_wgu[w + 1] : 0;
    int seg = 0, tile = 0, cnt = 0, seg1 = 0, cnt1 = 0;
    if (u1 > u0) {
      seg = last_le(off, nseg + 1, u0);
      tile = u0 - off[seg];
      cnt = in_lds ? s_cnt[seg] : local_count(p, seg / RB);
      const int un = off[seg + 1];          // first unit past the first segment
      if (un < u1) {
        seg1 = last_le(off, nseg + 1, un);
        cnt1 = in_lds ? s_cnt[seg1] : local_count(p, seg1 / RB);
      }
    }
    rec[0] = u1 - u0;
    rec[1] = seg;
    rec[2] = tile;
    rec[3] = cnt;
    rec[4] = seg1;
    rec[5] = cnt1;
  }

  // pieces of each segment (one per non-empty workgroup it meets) and
  // partial slots (only for segments cut into several pieces)
  int ms = 0;
  for (int s = s0; s < s1; ++s) {
    const int o = off[s], n = off[s + 1] - o;
    if (n > 0) {
      const int np = last_le(s_wgu, G, o + n - 1) - last_le(s_wgu, G, o) + 1;
      ms += np > 1 ? np : 0;
    }
  }
  const int2 ex2 = block_excl_scan2(ms, 0, s_wave, tot);
  int slot = ex2.x;
  for (int s = s0; s < s1; ++s) {
    const int o = off[s], n = off[s + 1] - o;
    int np = 0, first = 0;
    if (n > 0) {
      first = last_le(s_wgu, G, o);
      np = last_le(s_wgu, G, o + n - 1) - first + 1;
    }
    p.seg_info[s] = make_int4(slot, np, first, 0);
    slot += np > 1 ? np : 0;
  }
}

// ---------------------------------------------------------------------------
// streaming attention
// ---------------------------------------------------------------------------
// Position in the unit sequence: request, row block, tile, and the request's
// tile count and owned-token count. Wave-uniform.
struct Cursor {
  int b, rb, tile, ntiles, cnt;

  __device__ __forceinline__ void start(const DecodeParams& p, int seg, int t) {
    b = seg / p.row_blocks;
    rb = seg - b * p.row_blocks;
    tile = t;
    cnt = ld_const(p.req_cnt + b);
    ntiles = (cnt + kTile - 1) / kTile;
  }
  __device__ __forceinline__ void start_known(const DecodeParams& p, int seg, int t, int count) {
    b = seg / p.row_blocks;
    rb = seg - b * p.row_blocks;
    tile = t;
    cnt = count;
    ntiles = (cnt + kTile - 1) / kTile;
  }
  // move to the next unit; only called when one exists
  __device__ __forceinline__ void advance(const DecodeParams& p) {
    if (++tile < ntiles) return;
    tile = 0;
    for (;;) {
      if (++rb == p.row_blocks) {
        rb = 0;
        ++b;
        cnt = ld_const(p.req_cnt + b);
        ntiles = (cnt + kTile - 1) / kTile;
      }
      if (ntiles > 0) break;
    }
  }
};

// Row indices of the cursor's tile -> LDS ring slot (32 ints): wave w copies
// the table entries of tokens 8w .. 8w + 7 (one instruction per wave). Past
// the owned range it copies the tile's first entry instead; those tokens are
// masked by the reader.
__device__ __forceinline__ void fetch_rows(const DecodeParams& p, const Cursor& c, uint32_t slot_lds) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (lane < 8) {
    int j = c.tile * kTile + 8 * wave + lane;
    j = j < c.cnt ? j : c.tile * kTile;
    const int32_t* src;
    if (p.local_kv_indices != nullptr)
      src = p.local_kv_indices + (long long)c.b * p.local_kv_stride + j;
    else
      src = p.block_table + (long long)c.b * p.max_pages + ((j * p.num_shards + p.shard) >> 6);
    lds_dma4(src, __builtin_amdgcn_readfirstlane(slot_lds + 32 * wave));
  }
}

// KV row of token `tok` of the cursor's tile from its table entry.
__device__ __forceinline__ int resolve_row(const DecodeParams& p, int tile, int cnt, int tok, int raw) {
  const int j = tile * kTile + tok;
  if (j >= cnt) return kRowPastEnd;
  long long row;
  if (p.local_kv_indices != nullptr) {
    row = raw;
  } else {
    const int t = j * p.num_shards + p.shard;
    row = (raw < 0 || raw >= p.num_pages) ? -1 : (long long)raw * kPage + (t & 63);
  }
  return (row < 0 || row >= (long long)p.num_pages * kPage) ? kRowBad : (int)row;
}

// XOR swizzle of the 16-byte chunks inside each 128-byte group, by token:
// eight consecutive tokens get eight different values, and four consecutive
// tokens differ in the 32-byte pair they select.
__host__ __device__ constexpr int chunk_swz(int t) { return 2 * (t & 3) + ((t >> 2) & 1); }

// Copies of one tile into a stage (issue_tile, or its parts spread over a
// tile loop iteration). Stage layout (token-major, swizzled):
//   chunk c < 64 (dims 8c .. 8c + 7) of token t at byte 1024 t + 16 (c ^ swz(t)),
//   chunk c >= 64 (rope) at kRopeBase + 128 t + 16 ((c - 64) ^ swz(t)).
// Wave w moves tokens 8w .. 8w + 7: one copy per token for its first 1 KB
// (64 lanes over one row, so every copy reads whole 128-byte lines) and one
// copy for the eight 128-byte rope tails. The row of each token comes from
// the ring; the main copies take it as a scalar base address.
// Row of token 8w + (lane >> 3) of the cursor's tile for wave w (0 if the
// token is past the end or its page is outside the pool).
__device__ __forceinline__ int tile_rows(const DecodeParams& p, const Cursor& c, const int32_t* ring_slot) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tk = 8 * wave + (lane >> 3);
  const int row = resolve_row(p, c.tile, c.cnt, tk, ring_slot[tk]);
  return row >= 0 ? row : 0;
}
__device__ __forceinline__ void copy_rope(const DecodeParams& p, int rowc, uint32_t stage_lds) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  lds_dma16(p.kv + (long long)rowc * (2 * kDqk) + 16 * (64 + ((lane & 7) ^ chunk_swz(lane >> 3))),
            __builtin_amdgcn_readfirstlane(stage_lds + kRopeBase + 1024 * wave));
}
template <int kI0, int kI1>
__device__ __forceinline__ void copy_main(const DecodeParams& p, int rowc, uint32_t stage_lds) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int i = kI0; i < kI1; ++i) {
    const int r = __builtin_amdgcn_readlane(rowc, 8 * i);
    const uint8_t* base = p.kv + (long long)r * (2 * kDqk);
    lds_dma16_sbase(base, (uint32_t)(16 * (lane ^ chunk_swz(i))),
                    __builtin_amdgcn_readfirstlane(stage_lds + 1024 * (8 * wave + i)));
  }
}
__device__ __forceinline__ void issue_tile(const DecodeParams& p, const Cursor& c, uint32_t stage_lds,
                                           const int32_t* ring_slot) {
  const int rowc = tile_rows(p, c, ring_slot);
  copy_rope(p, rowc, stage_lds);
  copy_main<0, 8>(p, rowc, stage_lds);
}

// Wait until at most `after` vector-memory operations of this wave are
// outstanding, i.e. everything issued before the last `after` ones landed.
// `after` is wave-uniform; the ladder takes the largest immediate <= after
// (kMax bounds it; waiting longer is always safe).
template <int kMax>
__device__ __forceinline__ void wait_vm_le(int after) {
  if constexpr (kMax == 0) {
    wait_vmcnt<0>();
  } else {
    if (after >= kMax) wait_vmcnt<kMax>();
    else wait_vm_le<kMax - 1>(after);
  }
}

// fp8 tiles: staged as stored (token t at byte 576 t). Wave w moves the 4608
// bytes of tokens 8w .. 8w + 7; copy i covers bytes 1024 i .. + 1023 of them,
// lane l the 16-byte chunk (64 i + l) % 36 of token (64 i + l) / 36, and the
// fifth copy is a half one (32 lanes). rowc: row of token 8w + (lane & 7).
__device__ __forceinline__ int tile_rows8(const DecodeParams& p, const Cursor& c, const int32_t* ring_slot) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tk = 8 * wave + (lane & 7);
  const int row = resolve_row(p, c.tile, c.cnt, tk, ring_slot[tk]);
  return row >= 0 ? row : 0;
}
template <int kI0, int kI1>
__device__ __forceinline__ void copy8(const DecodeParams& p, int rowc, uint32_t stage_lds) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int i = kI0; i < kI1; ++i) {
    const int g = 64 * i + lane;
    const int tl = g / 36, ch = g - 36 * tl;
    const int row = __shfl(rowc, tl);
    const uint8_t* src = p.kv + (long long)row * kDqk + 16 * ch;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(stage_lds + 4608 * wave + 1024 * i);
    if (i < 4 || lane < 32) lds_dma16(src, dst);
  }
}
__device__ __forceinline__ void issue_tile8(const DecodeParams& p, const Cursor& c, uint32_t stage_lds,
                                            const int32_t* ring_slot) {
  const int rowc = tile_rows8(p, c, ring_slot);
  copy8<0, 5>(p, rowc, stage_lds);
}

// fp8 staging -> bf16 stage in the layout of the bf16 tiles (exact: every
// e4m3 value is a bf16 value; the per-tensor scale is applied to the scores
// and the output instead). Thread k converts the 8-dim chunks k + 256 j.
__device__ __forceinline__ void convert_tile8(const uint8_t* stg, uint8_t* dst) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int j = 0; j < kTile * (kDqk / 8) / 256; ++j) {
    const int unit = threadIdx.x + 256 * j;
    const int tkn = unit / (kDqk / 8), c = unit - (kDqk / 8) * tkn;
    const u32x2_t x = *(const u32x2_t*)(stg + kDqk * tkn + 8 * c);
    const bf16x2_t y0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, false);
    const bf16x2_t y1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, true);
    const bf16x2_t y2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, false);
    const bf16x2_t y3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, true);
    const bf16x8_t y = {y0[0], y0[1], y1[0], y1[1], y2[0], y2[1], y3[0], y3[1]};
    const uint32_t a = c < 64 ? (uint32_t)(1024 * tkn + 16 * (c ^ chunk_swz(tkn)))
                              : (uint32_t)(kRopeBase + 128 * tkn + 16 * ((c - 64) ^ chunk_swz(tkn)));
    *(bf16x8_t*)(dst + a) = y;
  }
}

// QK A operand of this wave's i-th k-step (see the kernel for the layout).
template <int kG>
__device__ __forceinline__ bf16x8_t qk_operand(const uint8_t* ks, uint32_t qk0, uint32_t rope0, int i) {
  return i / kG < 8 ? *(const bf16x8_t*)(ks + (qk0 ^ (32u * (i % kG))) + 128 * (i / kG))
                    : *(const bf16x8_t*)(ks + (rope0 ^ (32u * (i % kG))));
}

// PV operand of step st = 2 db + m (db local to the wave's slice): dims
// 32 db .. + 31 of tokens 16 m .. 16 m + 15 in the order of the P values,
// from two transposing loads of four tokens each (the second 8 tokens on).
__device__ __forceinline__ bf16x8_t pv_operand(const uint8_t* ks, uint32_t pv0, int st) {
  const int db = st >> 1, m = st & 1;
  const uint8_t* a = ks + (pv0 ^ (64u * (db & 1))) + 128 * (db >> 1) + 16384 * m;
  const i16x4_t lo = lds_read_tr16(a);
  const i16x4_t hi = lds_read_tr16(a + 8192);
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// x * f for an accumulator element held in an AGPR, in place (VALU cannot
// read AGPRs; keeping the operand constrained to an AGPR stops the compiler
// from moving the whole accumulator to VGPRs around the rare rescale).
__device__ __forceinline__ float acc_scale(float x, float f) {
  float tmp;
  asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
               : "+a"(x), "=&v"(tmp) : "v"(f));
  return x;
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

// Read an accumulator element held in an AGPR (keeps the compiler from
// moving the whole accumulator to VGPRs for the epilogue).
__device__ __forceinline__ float acc_read(float x) {
  float r;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(x));
  return r;
}

// Copy j of kCopies for a tile is issued after MFMA slot
// floor(j * slots / kCopies) of the tile loop (slots: the QK MFMAs, then the
// PV MFMAs); -1 for slots that issue none.
__host__ __device__ constexpr int copy_at_slot(int slot, int slots, int copies) {
  for (int j = 0; j < copies; ++j)
    if (j * slots / copies == slot) return j;
  return -1;
}
// Copy j of a tile: bf16 tiles move the rope tails (j = 0) and the 1 KB main
// part of token 8 w + j - 1 (j >= 1); fp8 tiles move 1 KB slice j.
template <bool kFp8>
__device__ __forceinline__ void issue_copy(const DecodeParams& p, int j, int rows, uint32_t stage_lds) {
  if constexpr (kFp8) {
    switch (j) {
      case 0: copy8<0, 1>(p, rows, stage_lds); break;
      case 1: copy8<1, 2>(p, rows, stage_lds); break;
      case 2: copy8<2, 3>(p, rows, stage_lds); break;
      case 3: copy8<3, 4>(p, rows, stage_lds); break;
      default: copy8<4, 5>(p, rows, stage_lds); break;
    }
  } else {
    switch (j) {
      case 0: copy_rope(p, rows, stage_lds); break;
      case 1: copy_main<0, 1>(p, rows, stage_lds); break;
      case 2: copy_main<1, 2>(p, rows, stage_lds); break;
      case 3: copy_main<2, 3>(p, rows, stage_lds); break;
      case 4: copy_main<3, 4>(p, rows, stage_lds); break;
      case 5: copy_main<4, 5>(p, rows, stage_lds); break;
      case 6: copy_main<5, 6>(p, rows, stage_lds); break;
      case 7: copy_main<6, 7>(p, rows, stage_lds); break;
      default: copy_main<7, 8>(p, rows, stage_lds); break;
    }
  }
}

template <int kDS, bool kFp8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_stream_kernel(DecodeParams p) {
  constexpr int kRG = 4 / kDS;                 // row groups of 32 rows
  constexpr int kRowsBlk = 32 * kRG;
  constexpr int kDb = (kDv / 32) / kDS;        // 32-dim blocks of this wave's V slice
  // stages: copies in flight while one tile is computed, about the same bytes
  // for both KV types (fp8 tiles are staged as stored and converted to one
  // bf16 compute stage per tile)
  constexpr int kNS = kFp8 ? 5 : 3;
  constexpr int kStg = kFp8 ? kStageBytes8 : kStageBytes;   // bytes of a staged tile
  constexpr int kCopies = kFp8 ? 5 : 9;                     // copies per wave per tile
  constexpr int kWaitMax = (kNS - 2) * (kCopies + 1);       // ops after a tile's copies
  constexpr int kAheadRows = 2 * kNS - 2;      // tiles whose row indices are fetched ahead
  // QK: the kDS waves of a row group split the 36 k-steps; wave ds takes the
  // k-steps kk with kk mod 4 in [kG ds, kG ds + kG) and sums the partial
  // scores of all kDS waves in one fixed order (so they agree bit for bit)
  constexpr int kG = 4 / kDS;
  constexpr int kKS = 9 * kG;                  // k-steps per wave
  // Q k-steps kept in LDS rather than VGPRs (with 32 rows x 512 dims of
  // accumulators in AGPRs, this keeps the tile loop spill-free); read back
  // once per tile
  constexpr int kQInLds = kDS == 1 ? 12 : 0;
  constexpr int kQRegSteps = kKS - kQInLds;
  constexpr int kPvSteps = 2 * kDb;
  constexpr int kAhead = 4;
  static_assert(kAheadRows < kRing, "row ring too small");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[kNS * kStg + (kFp8 ? kStageBytes : 0)];
  __shared__ __attribute__((aligned(16))) int32_t ring[kRing * kTile];
  __shared__ __attribute__((aligned(16))) uint8_t qlds[kQInLds > 0 ? 4 * kQInLds * 64 * 16 : 16];
  __shared__ __attribute__((aligned(16))) f32x4_t xbuf[kDS > 1 ? 4 * 4 * 64 : 1];   // [wave][4][lane]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave % kRG, ds = wave / kRG;
  const int tok = lane & 31, hi = lane >> 5;

  // consecutive workgroups of the unit order run on one XCD (blocks are
  // dealt to the 8 XCDs round robin), so the L2 of that XCD serves the
  // repeated reads of a request's Q and KV
  int g = blockIdx.x;
  if ((p.grid & 7) == 0) g = (blockIdx.x & 7) * (p.grid >> 3) + (blockIdx.x >> 3);
  const int G = ld_const(p.plan + 1);   // workgroups in use
  if (g >= G) return;
  const int Uw = ld_const(p.wg_ustart + g + 1) - ld_const(p.wg_ustart + g);
  if (Uw <= 0) return;

  const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(lds_address(smem));
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(lds_address(ring));
  Cursor cf, ci, cc;
  {
    const int2 st = ld_const(p.wg_start + g);
    cf.start(p, st.x, st.y);
    ci = cf;
    cc = cf;
  }

  // QK operand of this wave's i-th k-step kk = 4 (i / kG) + kG ds + i % kG
  // (lane: token tok, chunk 2 kk + hi): kk < 32 at
  // (qk0 ^ 32 (i % kG)) + 128 (i / kG), kk >= 32 (rope) at rope0 ^ 32 (i % kG)
  // (the XOR only touches the swizzled chunk bits 4..6)
  const uint32_t qk0 = (uint32_t)(1024 * tok + 16 * ((2 * kG * ds) ^ hi ^ chunk_swz(tok)));
  const uint32_t rope0 = (uint32_t)(kRopeBase + 128 * tok + 16 * ((2 * kG * ds) ^ hi ^ chunk_swz(tok)));
  // PV transposing loads: in 16-lane group g, lane 4r + q supplies dims
  // 32 db + 16 (g & 1) + 4 q .. + 3 of token 16 m + 8 h + 4 (g >> 1) + r
  // (h = first or second load); pv0 is its address for db = 0, and db = 1
  // differs in bit 6 only (chunk 4 + y instead of y under the swizzle)
  uint32_t pv0;
  {
    const int g16 = lane >> 4, r = (lane >> 2) & 3, q = lane & 3;
    const int tl = 4 * (g16 >> 1) + r;
    const int y = 2 * (g16 & 1) + (q >> 1);
    pv0 = (uint32_t)(1024 * tl + 16 * (y ^ chunk_swz(tl)) + 8 * (q & 1) + 64 * kDb * ds);
  }

  uint8_t* const qmine = qlds + 16 * (kQInLds * 64 * wave + lane);
  bf16x8_t qreg[kQRegSteps];
  // ops: vector-memory operations this wave has issued; pos[i]: ops right
  // after issuing the copies of tile t + i
  int ops = 0;
  int pos[kNS - 1];
#pragma unroll
  for (int i = 0; i < kNS - 1; ++i) pos[i] = 0;
  int t = 0, stage = 0;   // stage holds tile t
  while (t < Uw) {
    const int b = cc.b, rb = cc.rb, tile0 = cc.tile, ntiles = cc.ntiles, cnt = cc.cnt;
    const int n = min(ntiles - tile0, Uw - t);

    // the piece's queries, this wave's k-steps (rows past the last query row
    // read as zero); the last kQInLds k-steps go to this wave's LDS slot
    const int row = rb * kRowsBlk + rg * 32 + tok;
    const bool row_ok = row < p.rows;
    {
      const uint16_t* qrow = p.q + ((long long)b * p.rows + (row_ok ? row : 0)) * kDqk + 8 * hi;
#pragma unroll
      for (int i = 0; i < kKS; ++i) {
        const int kk = 4 * (i / kG) + kG * ds + i % kG;
        bf16x8_t x = *(const bf16x8_t*)(qrow + 16 * kk);
        x = row_ok ? x : bf16x8_t{};
        if (i < kQRegSteps) qreg[i] = x;
        else *(bf16x8_t*)(qmine + 16 * 64 * (i - kQRegSteps)) = x;
      }
    }
    if (t == 0) {
      // row indices of the first tiles, in flight with the queries
#pragma unroll
      for (int k = 0; k < kAheadRows; ++k) {
        if (k < Uw) {
          if (k > 0) cf.advance(p);
          fetch_rows(p, cf, ring_lds + 4 * kTile * (k % kRing));
        }
      }
    }
    // the query loads are the only loads the compiler tracks: waiting for
    // everything here keeps its own waits out of the tile loop (for later
    // pieces the tile copies in flight land meanwhile)
    wait_vmcnt<0>();
    if (t == 0) {
      __syncthreads();
      // the first kNS - 1 tiles
#pragma unroll
      for (int k = 0; k < kNS - 1; ++k) {
        if (k < Uw) {
          if (k > 0) ci.advance(p);
          if constexpr (kFp8) issue_tile8(p, ci, smem_lds + kStg * k, ring + kTile * k);
          else issue_tile(p, ci, smem_lds + kStg * k, ring + kTile * k);
          ops += kCopies;
          pos[k] = ops;
        }
      }
    }
    // owned tokens row (draft i) may see: t = j S + r <= L - q_len + i; the
    // count is computed per draft index with scalar arithmetic and selected
    int jvis = 0;
    {
      int L = ld_const(p.seq_lens + b);
      L = L < 0 ? 0 : min(L, p.max_pages * kPage);
      const int i = (row >= p.heads) + (row >= 2 * p.heads) + (row >= 3 * p.heads);
      for (int k = 0; k < p.q_len; ++k) {
        const int lim = L - p.q_len + k - p.shard;
        const int jl = lim >= 0 ? min(cnt, lim / p.num_shards + 1) : 0;
        jvis = i == k ? jl : jvis;
      }
    }
    // tiles that end at or before jvis_min need no visibility mask (rows
    // past the last query row are never written and do not count)
    int jvis_min = row_ok ? jvis : INT_MAX;
    jvis_min = min(jvis_min, __shfl_xor(jvis_min, 1));
    jvis_min = min(jvis_min, __shfl_xor(jvis_min, 2));
    jvis_min = min(jvis_min, __shfl_xor(jvis_min, 4));
    jvis_min = min(jvis_min, __shfl_xor(jvis_min, 8));
    jvis_min = min(jvis_min, __shfl_xor(jvis_min, 16));
    jvis_min = min(jvis_min, __shfl_xor(jvis_min, 32));
    jvis_min = __builtin_amdgcn_readfirstlane(jvis_min);

    f32x16_t o[kDb];
#pragma unroll
    for (int db = 0; db < kDb; ++db) o[db] = f32x16_t{};
    float m_ref = kNegInf, l_sum = 0.f;

    for (int k = 0; k < n; ++k, ++t) {
      // tile t has landed for this wave, then for all waves; the stage of
      // tile t - 1 is free
      wait_vm_le<kWaitMax>(ops - pos[0]);
      __syncthreads();
#pragma unroll
      for (int i = 0; i + 1 < kNS - 1; ++i) pos[i] = pos[i + 1];
      // row indices kAheadRows tiles ahead: issued before this iteration's
      // tile copies, so that waiting for those copies covers them too
      if (t + kAheadRows < Uw) {
        cf.advance(p);
        fetch_rows(p, cf, ring_lds + 4 * kTile * ((t + kAheadRows) % kRing));
        ops += 1;
      }
      // table entry of this tile's token `tok`, and the rows of tile
      // t + kNS - 1, whose copies go into the stage of tile t - 1 spread over
      // the MFMA sequences below (a burst would stall on the memory queue)
      const int raw_c = ring[kTile * (t % kRing) + tok];
      const bool more = t + kNS - 1 < Uw;
      const uint32_t st_next = smem_lds + kStg * (stage == 0 ? kNS - 1 : stage - 1);   // tile t - 1's
      int rows_next = 0;
      if (more) {
        ci.advance(p);
        const int32_t* rs = ring + kTile * ((t + kNS - 1) % kRing);
        rows_next = kFp8 ? tile_rows8(p, ci, rs) : tile_rows(p, ci, rs);
      }

      if constexpr (kFp8) {
        // the compute stage was last read by tile t - 1 (done at the barrier)
        convert_tile8(smem + kStg * stage, smem + kNS * kStg);
        __syncthreads();
      }
      const uint8_t* ks = kFp8 ? smem + kNS * kStg : smem + kStageBytes * stage;
      const int tile = tile0 + k;
      const int jt = tile * kTile;
      // tokens whose page is outside the pool poison their scores
      const int rr = resolve_row(p, tile, cnt, tok, raw_c);
      const uint64_t bad = __ballot(lane < kTile && rr == kRowBad);

      // S^T[token][row] over this wave's k-steps; K operands are read kAhead
      // steps ahead of their MFMA
      bf16x8_t ka[kAhead];
#pragma unroll
      for (int u = 0; u < kAhead; ++u) ka[u] = qk_operand<kG>(ks, qk0, rope0, u);
      f32x16_t s = f32x16_t{};
#pragma unroll
      for (int i = 0; i < kKS; ++i) {
        const bf16x8_t a = ka[i % kAhead];
        if (i + kAhead < kKS) {
          const int u = i + kAhead;
          ka[i % kAhead] = qk_operand<kG>(ks, qk0, rope0, u);
        }
        const bf16x8_t qb = i < kQRegSteps ? qreg[i < kQRegSteps ? i : 0]
                                           : *(const bf16x8_t*)(qmine + 16 * 64 * (i - kQRegSteps));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb, s, 0, 0, 0);
        constexpr int kSlots = kKS + kPvSteps;
        if (copy_at_slot(i, kSlots, kCopies) >= 0 && more) {
          issue_copy<kFp8>(p, copy_at_slot(i, kSlots, kCopies), rows_next, st_next);
          ops += 1;
        }
      }
      if constexpr (kDS == 2) {
        // the partner wave's partial scores; both waves form s0 + s1
        // (addition commutes exactly), so they agree bit for bit
        f32x4_t* mine = xbuf + (wave * 4) * 64 + lane;
#pragma unroll
        for (int q = 0; q < 4; ++q) mine[64 * q] = f32x4_t{s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]};
        __syncthreads();
        const f32x4_t* src = xbuf + (((1 - ds) * kRG + rg) * 4) * 64 + lane;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4_t v = src[64 * q];
#pragma unroll
          for (int e = 0; e < 4; ++e) s[4 * q + e] += v[e];
        }
      } else if constexpr (kDS > 2) {
        // sum the row group's partial scores in wave order
        f32x4_t* mine = xbuf + (wave * 4) * 64 + lane;
#pragma unroll
        for (int q = 0; q < 4; ++q) mine[64 * q] = f32x4_t{s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]};
        __syncthreads();
        f32x16_t tot = f32x16_t{};
#pragma unroll
        for (int d = 0; d < kDS; ++d) {
          const f32x4_t* src = xbuf + ((d * kRG + rg) * 4) * 64 + lane;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4_t v = src[64 * q];
#pragma unroll
            for (int e = 0; e < 4; ++e) tot[4 * q + e] += v[e];
          }
        }
        s = tot;
      }

      // online softmax in base 2 (this lane: one row, 16 tokens: value v is
      // token 8 (v >> 2) + 4 hi + (v & 3)); the max is taken on the raw
      // scores (scaling by a positive factor commutes with it exactly) and
      // the scale is folded into the exponent's FMA
      float tmax = kNegInf;
      if (jt + kTile <= jvis_min && bad == 0) {
#pragma unroll
        for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, s[v]);
      } else {
        // masks shifted by 4 hi once so each test is against a constant
        const int lim = jvis - jt - 4 * hi;
        const uint32_t badl = (uint32_t)bad >> (4 * hi);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int c = 8 * (v >> 2) + (v & 3);
          float x = c < lim ? s[v] : kNegInf;
          x = ((badl >> c) & 1u) ? __builtin_nanf("") : x;
          s[v] = x;
          tmax = fmaxf(tmax, x);
        }
      }
      tmax = xor32_max(tmax) * p.scale_log2;
      const bool grow = m_ref != kNegInf && tmax > m_ref + kRescaleSlack;
      if (__builtin_expect(__ballot(grow) != 0, 0)) {
        const float f = grow ? exp2_fast(m_ref - tmax) : 1.f;
        l_sum *= f;
        // o[.][v] belongs to row 8 (v >> 2) + 4 hi + (v & 3), whose factor
        // sits in that row's lane
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float fv = __shfl(f, 8 * (v >> 2) + 4 * hi + (v & 3));
#pragma unroll
          for (int db = 0; db < kDb; ++db) o[db][v] = acc_scale(o[db][v], fv);
        }
        m_ref = grow ? tmax : m_ref;
      }
      m_ref = m_ref == kNegInf ? tmax : m_ref;
      const float neg_m = m_ref == kNegInf ? 0.f : -m_ref;
      bf16x8_t pb[2];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float pv = exp2_fast(__builtin_fmaf(s[v], p.scale_log2, neg_m));
        l_sum += pv;
        pb[v >> 3][v & 7] = (__bf16)pv;
      }

      // O[row][dim] += P[row][token] V[token][dim] over this wave's dims: the
      // P registers (lane = row) are the A operand and the transposed V reads
      // (lane = dim) the B operand, both with the same token order in k; the
      // accumulator then holds 32 consecutive dims across lanes, so the
      // output stores write whole lines
      bf16x8_t va[kAhead];
#pragma unroll
      for (int u = 0; u < kAhead; ++u) va[u] = pv_operand(ks, pv0, u);
#pragma unroll
      for (int st = 0; st < kPvSteps; ++st) {
        const bf16x8_t a = va[st % kAhead];
        if (st + kAhead < kPvSteps) va[st % kAhead] = pv_operand(ks, pv0, st + kAhead);
        o[st >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pb[st & 1], a, o[st >> 1], 0, 0, 0);
        constexpr int kSlots = kKS + kPvSteps;
        if (copy_at_slot(kKS + st, kSlots, kCopies) >= 0 && more) {
          issue_copy<kFp8>(p, copy_at_slot(kKS + st, kSlots, kCopies), rows_next, st_next);
          ops += 1;
        }
      }
      if (more) pos[kNS - 2] = ops;
      stage = stage + 1 == kNS ? 0 : stage + 1;
    }

    // piece epilogue: o[db][v] is row 8 (v >> 2) + 4 hi + (v & 3) of the
    // row group, dim 32 (kDb ds + db) + (lane & 31)
    const float l_tot = xor32_sum(l_sum);
    const bool any = l_tot > 0.f || l_tot != l_tot;
    const float inv = any ? p.out_scale / l_tot : 0.f;
    const float lse2 = any ? m_ref + log2_fast(l_tot) : kNegInf;
    const bool single = tile0 == 0 && n == ntiles;
    const int row0 = rb * kRowsBlk + rg * 32;          // first row of the row group
    const int dim = 32 * kDb * ds + (lane & 31);
    long long base;                                    // element index of (row0, dim)
    if (single) {
      base = ((long long)b * p.rows + row0) * kDv + dim;
    } else {
      const int4 si = ld_const(p.seg_info + b * p.row_blocks + rb);
      base = ((long long)(si.x + g - si.z) * kRowsBlk + rg * 32) * kDv + dim;
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 8 * (v >> 2) + 4 * hi + (v & 3);
      const float iv = __shfl(inv, r);
      if (row0 + r < p.rows) {
        const long long e0 = base + (long long)r * kDv;
        if (single && !p.out_bf16) {
          float* dst = (float*)p.out + e0;
#pragma unroll
          for (int db = 0; db < kDb; ++db) dst[32 * db] = acc_read(o[db][v]) * iv;
        } else {
          __bf16* dst = single ? (__bf16*)p.out + e0 : (__bf16*)p.spart_o + e0;
#pragma unroll
          for (int db = 0; db < kDb; ++db) dst[32 * db] = (__bf16)(acc_read(o[db][v]) * iv);
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // one row at a time: short live ranges
    }
    if (row_ok && ds == 0 && hi == 0) {
      if (single) {
        p.lse[(long long)b * p.rows + row] = p.lse_base2 ? lse2 : lse2 * kLn2;
      } else {
        const int4 si = ld_const(p.seg_info + b * p.row_blocks + rb);
        p.spart_lse[(long long)(si.x + g - si.z) * kRowsBlk + (row - rb * kRowsBlk)] = lse2;
      }
    }
    if (t < Uw) {
      cc.tile = ntiles - 1;
      cc.advance(p);
    }
  }
}

// ---------------------------------------------------------------------------
// software-pipelined attention over bf16 KV
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
    te.p0 = (j0 * p.num_shards + p.shard) >> 6;
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
    const int t = j * p.num_shards + p.shard;
    const int d = (t >> 6) - te.p0;
    unsigned eu = (unsigned)te.e0;
    eu += d >= 1 ? (unsigned)te.e1 - (unsigned)te.e0 : 0u;
    eu += d >= 2 ? (unsigned)te.e2 - (unsigned)te.e1 : 0u;
    const int e = (int)eu;
    const bool ok = e >= 0 && e < p.num_pages;
    return ok ? p.kv + ((long long)e * kPage + (t & 63)) * kRowBytes : nan;
  }
}

// Copy j of a bf16 tile into a stage (layout as for the streaming kernel):
// j = 0 moves the eight rope tails of the wave's tokens, j = 1 + i the 1 KB
// main part of token 8 w + i (one row per copy, as a scalar base).
template <int kJ>
__device__ __forceinline__ void copy_tile_part(const uint8_t* src, uint32_t stage_lds, int wave) {
  const int lane = threadIdx.x & 63;
  if constexpr (kJ == 0) {
    lds_dma16(src + 16 * (64 + ((lane & 7) ^ chunk_swz(lane >> 3))),
              __builtin_amdgcn_readfirstlane(stage_lds + kRopeBase + 1024 * wave));
  } else {
    constexpr int i = kJ - 1;
    const uint64_t a = reinterpret_cast<uint64_t>(src);
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)a, 8 * i);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(a >> 32), 8 * i);
    const uint8_t* base = reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
    lds_dma16_sbase(base, (uint32_t)(16 * (lane ^ chunk_swz(i))),
                    __builtin_amdgcn_readfirstlane(stage_lds + 1024 * (8 * wave + i)));
  }
}
__device__ __forceinline__ void copy_tile_part_rt(int j, const uint8_t* src, uint32_t stage_lds, int wave) {
  switch (j) {
    case 0: copy_tile_part<0>(src, stage_lds, wave); break;
    case 1: copy_tile_part<1>(src, stage_lds, wave); break;
    case 2: copy_tile_part<2>(src, stage_lds, wave); break;
    case 3: copy_tile_part<3>(src, stage_lds, wave); break;
    case 4: copy_tile_part<4>(src, stage_lds, wave); break;
    case 5: copy_tile_part<5>(src, stage_lds, wave); break;
    case 6: copy_tile_part<6>(src, stage_lds, wave); break;
    case 7: copy_tile_part<7>(src, stage_lds, wave); break;
    default: copy_tile_part<8>(src, stage_lds, wave); break;
  }
}

// The tile loop overlaps two tiles: while the VALU computes tile k's softmax,
// the MFMAs accumulate tile k - 1's P V. Four stages hold tile k - 1 (V),
// tile k (K) and two tiles in flight. Every tile barrier issues exactly the
// nine copies of the tile two ahead (from the zero row past the workgroup's
// last unit), so the wait before it is a constant vmcnt(9): the only
// vector-memory operations between two tile barriers are those copies (query
// loads and output stores are drained at piece starts).
template <int kDS, bool kLocal>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_pipe_kernel(DecodeParams p) {
  constexpr int kRG = 4 / kDS;                 // row groups of 32 rows
  constexpr int kRowsBlk = 32 * kRG;
  constexpr int kDb = (kDv / 32) / kDS;        // 32-dim blocks of this wave's V slice
  constexpr int kNS = 4;
  constexpr int kCopies = 9;
  constexpr int kG = 4 / kDS;
  constexpr int kKS = 9 * kG;                  // QK k-steps per wave
  constexpr int kPvSteps = 2 * kDb;
  constexpr int kAhead = 4;

  __shared__ __attribute__((aligned(1024))) uint8_t smem[kNS * kStageBytes];
  __shared__ __attribute__((aligned(16))) f32x4_t xbuf[4 * 4 * 64];   // [wave][4][lane]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave % kRG, ds = wave / kRG;
  const int tok = lane & 31, hi = lane >> 5;

  // consecutive workgroups of the unit order run on one XCD (blocks are
  // dealt to the 8 XCDs round robin), so the L2 of that XCD serves the
  // repeated reads of a request's Q and KV
  int g = blockIdx.x;
  if ((p.grid & 7) == 0) g = (blockIdx.x & 7) * (p.grid >> 3) + (blockIdx.x >> 3);
  // the start record: one round of scalar loads, then one for the table
  // entries of the first two tiles, before the first copies
  const int32_t* rec = p.wg_rec + (long long)g * kRecInts;
  const int Uw = ld_const(rec);
  const int rec_seg = ld_const(rec + 1), rec_tile = ld_const(rec + 2), rec_cnt = ld_const(rec + 3);
  const int rec_seg1 = ld_const(rec + 4), rec_cnt1 = ld_const(rec + 5);
  if (Uw <= 0) return;
  const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(lds_address(smem));
  const uint32_t qk0 = (uint32_t)(1024 * tok + 16 * ((2 * kG * ds) ^ hi ^ chunk_swz(tok)));
  const uint32_t rope0 = (uint32_t)(kRopeBase + 128 * tok + 16 * ((2 * kG * ds) ^ hi ^ chunk_swz(tok)));
  uint32_t pv0;
  {
    const int g16 = lane >> 4, r = (lane >> 2) & 3, q = lane & 3;
    const int tl = 4 * (g16 >> 1) + r;
    const int y = 2 * (g16 & 1) + (q >> 1);
    pv0 = (uint32_t)(1024 * tl + 16 * (y ^ chunk_swz(tl)) + 8 * (q & 1) + 64 * kDb * ds);
  }

  // cc: the piece being computed; cl: the next tile to copy
  // cc: the piece being computed; cl: the next tile to copy, te its table
  // entries. The first two tiles' cursors come from the record (the second
  // one may start the next segment).
  Cursor cc, cl;
  cc.start_known(p, rec_seg, rec_tile, rec_cnt);
  cl = cc;
  if (1 < Uw) {
    if (cl.tile + 1 < cl.ntiles) ++cl.tile;
    else cl.start_known(p, rec_seg1, 0, rec_cnt1);
  }
  {
    TileEntries te0, te1;
    load_entries<kLocal>(p, cc, wave, te0);
    if (1 < Uw) load_entries<kLocal>(p, cl, wave, te1);
    const uint8_t* src0 = token_src<kLocal>(p, cc, true, te0, wave);
#pragma unroll
    for (int j = 0; j < kCopies; ++j) copy_tile_part_rt(j, src0, smem_lds, wave);
    const uint8_t* src1 = token_src<kLocal>(p, cl, 1 < Uw, te1, wave);
#pragma unroll
    for (int j = 0; j < kCopies; ++j) copy_tile_part_rt(j, src1, smem_lds + kStageBytes, wave);
  }
  int ncopied = 2;
  TileEntries te;   // entries of tile ncopied, loaded a barrier ahead
  if (2 < Uw) {
    cl.advance(p);
    load_entries<kLocal>(p, cl, wave, te);
  }

  bf16x8_t qreg[kKS];
  const uint8_t* csrc = nullptr;   // copies of this iteration: sources, stage
  uint32_t cst = 0;
  // tile barrier: the tile that the next QK reads has landed in every wave,
  // and the stage of the tile two back is free for tile ncopied; the table
  // entries of the tile after it are loaded here for the next barrier
  auto tile_barrier = [&]() {
    wait_vmcnt<kCopies>();
    __syncthreads();
    csrc = token_src<kLocal>(p, cl, ncopied < Uw, te, wave);
    cst = __builtin_amdgcn_readfirstlane(smem_lds + kStageBytes * (ncopied & (kNS - 1)));
    ++ncopied;
    if (ncopied < Uw) {
      cl.advance(p);
      load_entries<kLocal>(p, cl, wave, te);
    }
  };
  // The MFMAs of one iteration form a sequence of kSlots; copy j of the
  // iteration's tile goes out after MFMA copy_slot(j).
  constexpr int kSlots = kKS + kPvSteps;
  auto after_mfma = [&](int m) {
    if (copy_at_slot(m, kSlots, kCopies) >= 0) copy_tile_part_rt(copy_at_slot(m, kSlots, kCopies), csrc, cst, wave);
  };
  // scores: S^T of a tile over this wave's k-steps, one MFMA per step, K
  // operands read kAhead steps ahead
  bf16x8_t ka[kAhead];
  f32x16_t acc;
  auto qk_start = [&](const uint8_t* ks) {
#pragma unroll
    for (int u = 0; u < kAhead; ++u) ka[u] = qk_operand<kG>(ks, qk0, rope0, u);
    acc = f32x16_t{};
  };
  auto qk_step = [&](const uint8_t* ks, int i) {
    const bf16x8_t a = ka[i % kAhead];
    if (i + kAhead < kKS) ka[i % kAhead] = qk_operand<kG>(ks, qk0, rope0, i + kAhead);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[i], acc, 0, 0, 0);
  };
  // this wave's partial scores to the exchange buffer
  auto xchg_write = [&](const f32x16_t& a) {
    f32x4_t* mine = xbuf + (wave * 4) * 64 + lane;
#pragma unroll
    for (int q = 0; q < 4; ++q) mine[64 * q] = f32x4_t{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
  };
  // the row group's summed scores (after the exchange barrier): both waves
  // of a pair form s0 + s1 (addition commutes exactly); four waves sum in
  // wave order from the buffer
  auto xchg_sum = [&](const f32x16_t& a) {
    f32x16_t r;
    if constexpr (kDS == 2) {
      const f32x4_t* src = xbuf + (((1 - ds) * kRG + rg) * 4) * 64 + lane;
      f32x4_t v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = src[64 * q];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) r[4 * q + e] = a[4 * q + e] + v[q][e];
    } else {
      r = f32x16_t{};
#pragma unroll
      for (int d = 0; d < kDS; ++d) {
        const f32x4_t* src = xbuf + ((d * kRG + rg) * 4) * 64 + lane;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4_t v = src[64 * q];
#pragma unroll
          for (int e = 0; e < 4; ++e) r[4 * q + e] += v[e];
        }
      }
    }
    return r;
  };
  // accumulation O^T[dim][row] += V^T[dim][token] P^T[token][row] over
  // this wave's dims (transposed V reads the A operand, the P registers the
  // B operand, both with the same token order in k); step s2 covers dim
  // block s2 % kDb and token half s2 / kDb, so consecutive MFMAs update
  // different accumulators
  auto pv_index = [](int s2) { return 2 * (s2 % kDb) + s2 / kDb; };
  bf16x8_t va[kAhead];

  int t = 0;   // unit index of the current piece's first tile
  while (t < Uw) {
    const int b = cc.b, rb = cc.rb, tile0 = cc.tile, ntiles = cc.ntiles, cnt = cc.cnt;
    const int n = min(ntiles - tile0, Uw - t);
    const int row = rb * kRowsBlk + rg * 32 + tok;
    const bool row_ok = row < p.rows;
    {
      const uint16_t* qrow = p.q + ((long long)b * p.rows + (row_ok ? row : 0)) * kDqk + 8 * hi;
#pragma unroll
      for (int i = 0; i < kKS; ++i) {
        const int kk = 4 * (i / kG) + kG * ds + i % kG;
        const bf16x8_t x = *(const bf16x8_t*)(qrow + 16 * kk);
        qreg[i] = row_ok ? x : bf16x8_t{};
      }
    }
    // the query loads are the only loads the compiler tracks: waiting for
    // everything here keeps its own waits out of the tile loop
    wait_vmcnt<0>();
    // owned tokens row (draft i) may see: t = j S + r <= L - q_len + i
    int jvis = 0;
    {
      int L = ld_const(p.seq_lens + b);
      L = L < 0 ? 0 : min(L, p.max_pages * kPage);
      const int i = (row >= p.heads) + (row >= 2 * p.heads) + (row >= 3 * p.heads);
      for (int k = 0; k < p.q_len; ++k) {
        const int lim = L - p.q_len + k - p.shard;
        const int jl = lim >= 0 ? min(cnt, lim / p.num_shards + 1) : 0;
        jvis = i == k ? jl : jvis;
      }
    }

    f32x16_t o[kDb];
#pragma unroll
    for (int db = 0; db < kDb; ++db) o[db] = f32x16_t{};
    float m_ref = kNegInf, l_sum = 0.f;

    auto pv_start = [&](const uint8_t* ks) {
#pragma unroll
      for (int u = 0; u < kAhead; ++u) va[u] = pv_operand(ks, pv0, pv_index(u));
    };
    auto pv_step = [&](const uint8_t* ks, const bf16x8_t (&pb)[2], int s2) {
      const int st = pv_index(s2);
      const bf16x8_t a = va[s2 % kAhead];
      if (s2 + kAhead < kPvSteps) va[s2 % kAhead] = pv_operand(ks, pv0, pv_index(s2 + kAhead));
      o[st >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[st & 1], o[st >> 1], 0, 0, 0);
    };
    // online softmax of tile k in base 2 (lane: one row, 16 tokens; value v
    // is token 8 (v >> 2) + 4 hi + (v & 3)); tokens at or past the row's
    // visibility limit are masked; the max is taken on the raw scores
    // (scaling by a positive factor commutes with it exactly) and the scale
    // is folded into the exponent's FMA. Split into kQ1 chunks that run
    // between the score MFMAs of the next tile: chunks 0 and 1 mask and take
    // the max (and move the reference), the rest exponentiate.
    constexpr int kQ1 = kKS / 2;            // score steps before the accumulation starts
    constexpr int kP1 = kPvSteps / 2;       // accumulation steps before the exchange
    static_assert(kQ1 >= 3, "softmax chunks");
    float f = 1.f, tmax = kNegInf, neg_m = 0.f;
    bool grow = false;
    int lim = 0;
    auto softmax_chunk = [&](int c, int k, f32x16_t& sc, bf16x8_t (&pb)[2]) {
      if (c == 0) {
        lim = jvis - (tile0 + k) * kTile - 4 * hi;
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
        grow = m_ref != kNegInf && tm > m_ref + kRescaleSlack;
        f = grow ? exp2_fast(m_ref - tm) : 1.f;
        l_sum *= f;
        m_ref = grow || m_ref == kNegInf ? tm : m_ref;
        neg_m = m_ref == kNegInf ? 0.f : -m_ref;
      }
      if (c >= 2) {
        constexpr int kE = kQ1 - 2;         // exponent chunks
        const int v0 = (c - 2) * 16 / kE, v1 = (c - 1) * 16 / kE;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          if (v >= v0 && v < v1) {
            const float pr = exp2_fast(__builtin_fmaf(sc[v], p.scale_log2, neg_m));
            l_sum += pr;
            pb[v >> 3][v & 7] = (__bf16)pr;
          }
        }
      }
      if (c == kQ1 - 1) {
        // the results exist before the rescale branch (otherwise they are
        // sunk below it, away from the MFMAs they overlap)
        asm volatile("" :: "v"(l_sum), "v"(pb[0]), "v"(pb[1]));
      }
    };
    // the rare rescale of the accumulators (every value a lane holds
    // belongs to its own row)
    auto rescale = [&]() {
      if (__builtin_expect(__ballot(grow) != 0, 0)) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
#pragma unroll
          for (int db = 0; db < kDb; ++db) o[db][v] = acc_scale(o[db][v], f);
      }
    };

    // tile 0: its scores; the copies of its barrier all go out here
    f32x16_t s_cur;
    {
      tile_barrier();
      const uint8_t* ksq = smem + kStageBytes * (t & (kNS - 1));
      qk_start(ksq);
#pragma unroll
      for (int i = 0; i < kKS; ++i) {
        qk_step(ksq, i);
        after_mfma(i);
      }
      xchg_write(acc);
      __syncthreads();
      s_cur = xchg_sum(acc);
#pragma unroll
      for (int m = kKS; m < kSlots; ++m) after_mfma(m);
    }
    // tiles k + 1 <= n - 1: the scores of tile k + 1 run with the softmax
    // and then the accumulation of tile k
    for (int k = 0; k + 1 < n; ++k) {
      tile_barrier();
      const uint8_t* ksq = smem + kStageBytes * ((t + k + 1) & (kNS - 1));
      const uint8_t* ksv = smem + kStageBytes * ((t + k) & (kNS - 1));
      bf16x8_t pb[2];
      qk_start(ksq);
#pragma unroll
      for (int i = 0; i < kQ1; ++i) {
        qk_step(ksq, i);
        after_mfma(i);
        softmax_chunk(i, k, s_cur, pb);
        __builtin_amdgcn_sched_barrier(0);
      }
      rescale();
      pv_start(ksv);
      // the remaining score steps alternate with the first accumulation
      // steps (independent MFMAs back to back)
      constexpr int kMix = (kKS - kQ1) > kP1 ? (kKS - kQ1) : kP1;
#pragma unroll
      for (int j = 0; j < kMix; ++j) {
        if (kQ1 + j < kKS) {
          qk_step(ksq, kQ1 + j);
          after_mfma(kQ1 + 2 * j);
        }
        if (j < kP1) {
          pv_step(ksv, pb, j);
          after_mfma(kQ1 + 2 * j + 1);
        }
      }
      xchg_write(acc);
      __syncthreads();
      if constexpr (kDS == 2) {
        // the partner's partial scores are read first and added after the
        // accumulation steps, whose MFMAs cover the reads' latency
        const f32x4_t* src = xbuf + (((1 - ds) * kRG + rg) * 4) * 64 + lane;
        f32x4_t pv4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) pv4[q] = src[64 * q];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s2 = kP1; s2 < kPvSteps; ++s2) {
          pv_step(ksv, pb, s2);
          after_mfma(kKS + s2);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) s_cur[4 * q + e] = acc[4 * q + e] + pv4[q][e];
      } else {
#pragma unroll
        for (int s2 = kP1; s2 < kPvSteps; ++s2) {
          pv_step(ksv, pb, s2);
          after_mfma(kKS + s2);
        }
        s_cur = xchg_sum(acc);
      }
      // keep the accumulators in AGPRs across iterations (left to itself
      // the register allocator moves them through VGPRs and spills)
#pragma unroll
      for (int db = 0; db < kDb; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) asm volatile("" : "+a"(o[db][v]));
    }
    // the last tile of the piece
    {
      bf16x8_t pb[2];
#pragma unroll
      for (int c = 0; c < kQ1; ++c) softmax_chunk(c, n - 1, s_cur, pb);
      rescale();
      const uint8_t* ksv = smem + kStageBytes * ((t + n - 1) & (kNS - 1));
      pv_start(ksv);
#pragma unroll
      for (int s2 = 0; s2 < kPvSteps; ++s2) pv_step(ksv, pb, s2);
    }

    // piece epilogue: the accumulators hold O^T (V^T is the A operand): lane
    // l has row rg * 32 + (l & 31) and o[db][v] is its dim
    // 32 (kDb ds + db) + 8 (v >> 2) + 4 hi + (v & 3)
    const float l_tot = xor32_sum(l_sum);
    const bool any = l_tot > 0.f || l_tot != l_tot;
    const float inv = any ? p.out_scale / l_tot : 0.f;
    const float lse2 = any ? m_ref + log2_fast(l_tot) : kNegInf;
    const bool single = tile0 == 0 && n == ntiles;
    const int row0 = rb * kRowsBlk + rg * 32;          // first row of the row group
    if (single && !p.out_bf16) {
      // f32 output: four consecutive dims per lane and store
      if (row_ok) {
        float* dst = (float*)p.out + ((long long)b * p.rows + row) * kDv + 32 * kDb * ds + 4 * hi;
#pragma unroll
        for (int db = 0; db < kDb; ++db)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4_t x = {acc_read(o[db][4 * q]) * inv, acc_read(o[db][4 * q + 1]) * inv,
                               acc_read(o[db][4 * q + 2]) * inv, acc_read(o[db][4 * q + 3]) * inv};
            *(f32x4_t*)(dst + 32 * db + 8 * q) = x;
          }
      }
    } else {
      // bf16 output through LDS: each wave writes its 32 rows x (kDb * 32)
      // dims row-major (rows padded to 528 bytes) into the stages of the
      // piece's last two tiles, free once every wave has passed this
      // barrier, and stores whole rows (16 bytes a lane)
      constexpr int kRowPitch = 528;
      static_assert(2 * 32 * kRowPitch <= kStageBytes, "two waves' rows per stage");
      __syncthreads();
      uint8_t* tb = smem + kStageBytes * ((t + n - 1 - (wave >> 1)) & (kNS - 1)) + (wave & 1) * 32 * kRowPitch;
      typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int db = 0; db < kDb; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bf16x4_t x = {(__bf16)(acc_read(o[db][4 * q]) * inv), (__bf16)(acc_read(o[db][4 * q + 1]) * inv),
                              (__bf16)(acc_read(o[db][4 * q + 2]) * inv), (__bf16)(acc_read(o[db][4 * q + 3]) * inv)};
          *(bf16x4_t*)(tb + kRowPitch * tok + 2 * (32 * db + 8 * q + 4 * hi)) = x;
        }
      __bf16* obase;
      long long pitch_rows;
      if (single) {
        obase = (__bf16*)p.out + ((long long)b * p.rows + row0) * kDv;
      } else {
        const int4 si = ld_const(p.seg_info + b * p.row_blocks + rb);
        obase = (__bf16*)p.spart_o + ((long long)(si.x + g - si.z) * kRowsBlk + rg * 32) * kDv;
      }
      (void)pitch_rows;
      constexpr int kLanesPerRow = kDb * 32 / 8;        // 16-byte pieces of a row's slice
      constexpr int kRowsPerStore = 64 / kLanesPerRow;
      const int rr0 = lane / kLanesPerRow, cc = lane % kLanesPerRow;
#pragma unroll
      for (int i = 0; i < 32 / kRowsPerStore; ++i) {
        const int rr = kRowsPerStore * i + rr0;
        const bf16x8_t x = *(const bf16x8_t*)(tb + kRowPitch * rr + 16 * cc);
        if (row0 + rr < p.rows) *(bf16x8_t*)(obase + (long long)rr * kDv + 32 * kDb * ds + 8 * cc) = x;
      }
    }
    if (row_ok && ds == 0 && hi == 0) {
      if (single) {
        p.lse[(long long)b * p.rows + row] = p.lse_base2 ? lse2 : lse2 * kLn2;
      } else {
        const int4 si = ld_const(p.seg_info + b * p.row_blocks + rb);
        p.spart_lse[(long long)(si.x + g - si.z) * kRowsBlk + (row - rb * kRowsBlk)] = lse2;
      }
    }
    t += n;
    if (t < Uw) {
      cc.tile = ntiles - 1;
      cc.advance(p);
    }
  }
  // no copy may still be writing this workgroup's LDS when it exits
  wait_vmcnt<0>();
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
template <int kJ>
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
    lds_dma16(reinterpret_cast<const uint8_t*>(row) + 16 * c,
              __builtin_amdgcn_readfirstlane(stage_lds + 512 * (8 * wave + 2 * kJ)));
  } else {
    const int tl = (lane >> 2) & 7;
    const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)a, 8 * tl);
    const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(a >> 32), 8 * tl);
    const uint8_t* row = reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
    const int t = 8 * wave + tl;
    const int r = (lane & 3) ^ ((t >> 2) & 3);
    if (lane < 32) lds_dma16(row + 512 + 16 * r, __builtin_amdgcn_readfirstlane(stage_lds + kRope8 + 512 * wave));
  }
}
__device__ __forceinline__ void copy8_tile_part_rt(int j, const uint8_t* srcw, uint32_t stage_lds, int wave) {
  switch (j) {
    case 0: copy8_tile_part<0>(srcw, stage_lds, wave); break;
    case 1: copy8_tile_part<1>(srcw, stage_lds, wave); break;
    case 2: copy8_tile_part<2>(srcw, stage_lds, wave); break;
    case 3: copy8_tile_part<3>(srcw, stage_lds, wave); break;
    default: copy8_tile_part<4>(srcw, stage_lds, wave); break;
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

template <bool kLocal, bool kFp8>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_ws_kernel(DecodeParams p) {
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
    const uint32_t qk0 = (uint32_t)(1024 * tok + 16 * ((2 * kG * ds) ^ hi ^ chunk_swz(tok)));
    const uint32_t rope0 = (uint32_t)(kRopeBase + 128 * tok + 16 * ((2 * kG * ds) ^ hi ^ chunk_swz(tok)));
    // fp8: score step i = 2 j + u uses 16-dim chunk 2 m + hi of the lane's
    // token, m = 2 j + ds (m = 16, 17: rope), its 8-byte half u; the query
    // registers follow the same order of the dims
    const uint32_t qk8 = (uint32_t)(512 * tok + 16 * (hi ^ (tok & 15) ^ (4 * hi)));
    const uint32_t rope8 = (uint32_t)(kRope8 + 64 * tok + 16 * ((2 * ds + hi) ^ ((tok >> 2) & 3)));
    Cursor cc;
    cc.start_known(p, rec_seg, rec_tile, rec_cnt);
    bf16x8_t qreg[kKS];
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
      if constexpr (kFp8) {
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

    int t = 0;
    while (t < Uw) {
      const int b = cc.b, rb = cc.rb, tile0 = cc.tile, ntiles = cc.ntiles, cnt = cc.cnt;
      const int n = min(ntiles - tile0, Uw - t);
      const int row = rb * kWsRows + rg * 32 + tok;
      const bool row_ok = row < p.rows;
      {
        const uint16_t* qrow = p.q + ((long long)b * p.rows + (row_ok ? row : 0)) * kDqk;
#pragma unroll
        for (int i = 0; i < kKS; ++i) {
          int d0;
          if constexpr (kFp8) d0 = 32 * (2 * (i >> 1) + ds) + 16 * hi + 8 * (i & 1);
          else d0 = 16 * (4 * (i / kG) + kG * ds + i % kG) + 8 * hi;
          const bf16x8_t x = *(const bf16x8_t*)(qrow + d0);
          qreg[i] = row_ok ? x : bf16x8_t{};
        }
      }
      wait_vmcnt<0>();
      // owned tokens row (draft i) may see: t = j S + r <= L - q_len + i
      int jvis = 0;
      {
        int L = ld_const(p.seq_lens + b);
        L = L < 0 ? 0 : min(L, p.max_pages * kPage);
        const int i = (row >= p.heads) + (row >= 2 * p.heads) + (row >= 3 * p.heads);
        for (int k = 0; k < p.q_len; ++k) {
          const int lim = L - p.q_len + k - p.shard;
          const int jl = lim >= 0 ? min(cnt, lim / p.num_shards + 1) : 0;
          jvis = i == k ? jl : jvis;
        }
      }
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
          lim = jvis - (tile0 + k) * kTile - 4 * hi;
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
          constexpr int kE = kChunks - 2;
          const int v0 = (c - 2) * 16 / kE, v1 = (c - 1) * 16 / kE;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            if (v >= v0 && v < v1) {
              const float pr = exp2_fast(__builtin_fmaf(sc[v], p.scale_log2, neg_m));
              l_sum += pr;
              pb[v >> 3][v & 7] = (__bf16)pr;
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
        __syncthreads();   // tile t + k + 1 landed
        const uint8_t* ksq = smem + kStageB * ((t + k + 1) & (kNS - 1));
        qk_start(ksq);
        if (ds == 0) {
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
      // the last tile's softmax; row sums and LSE of the piece
      const bool single = tile0 == 0 && n == ntiles;
      if (ds == 0) {
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
            const int4 si = ld_const(p.seg_info + b * p.row_blocks + rb);
            p.spart_lse[(long long)(si.x + g - si.z) * kWsRows + (row - rb * kWsRows)] = lse2;
          }
        }
      }
      __syncthreads();   // P of the last tile and the row sums written
      __syncthreads();   // every output wave is done with the stages
      t += n;
      if (t < Uw) {
        cc.tile = ntiles - 1;
        cc.advance(p);
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
      if constexpr (kFp8) copy8_tile_part_rt(j, src, st, wq);
      else copy_tile_part_rt(j, src, st, wq);
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
      cl.advance(p);
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
        cl.advance(p);
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
      const int b = cc.b, rb = cc.rb, tile0 = cc.tile, ntiles = cc.ntiles;
      const int n = min(ntiles - tile0, Uw - t);
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
      // 128 wq + 32 db + 8 (v >> 2) + 4 hi + (v & 3)
      float inv[2];
      {
        const bool a0 = l0 > 0.f || l0 != l0, a1 = l1 > 0.f || l1 != l1;
        inv[0] = a0 ? p.out_scale / l0 : 0.f;
        inv[1] = a1 ? p.out_scale / l1 : 0.f;
      }
      const bool single = tile0 == 0 && n == ntiles;
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
                *(f32x4_t*)(dst + 32 * db + 8 * q) = x;
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
          const int4 si = ld_const(p.seg_info + b * p.row_blocks + rb);
          obase = (__bf16*)p.spart_o + ((long long)(si.x + g - si.z) * kWsRows) * kDv;
        }
        const int rr0 = lane >> 4, c16 = lane & 15;
#pragma unroll
        for (int i = 0; i < kWsRows / 4; ++i) {
          const int rr = 4 * i + rr0;
          const bf16x8_t x = *(const bf16x8_t*)(sb + kWsStagePitch * rr + 16 * c16);
          if (row0 + rr < p.rows) *(bf16x8_t*)(obase + (long long)rr * kDv + 128 * wq + 8 * c16) = x;
        }
      }
      t += n;
      if (t < Uw) {
        cc.tile = ntiles - 1;
        cc.advance(p);
      }
    }
    // no copy may still be writing this workgroup's LDS when it exits
    wait_vmcnt<0>();
  }
}

// ---------------------------------------------------------------------------
// combine the pieces of segments cut at workgroup boundaries; neutral rows
// for requests with no owned token
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void stream_combine_kernel(DecodeParams p) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  const int rb = row / p.rows_blk;
  const int4 si = p.seg_info[b * p.row_blocks + rb];
  const int np = si.y;
  if (np == 1) return;
  const long long orow = (long long)b * p.rows + row;
  f32x4_t acc0 = f32x4_t{}, acc1 = f32x4_t{};
  float mx = kNegInf, wsum = 0.f;
  if (np > 1) {
    const long long prow0 = (long long)si.x * p.rows_blk + (row - rb * p.rows_blk);
    for (int c = 0; c < np; ++c) mx = fmaxf(mx, p.spart_lse[prow0 + (long long)c * p.rows_blk]);
    if (mx != kNegInf) {
      for (int c = 0; c < np; ++c) {
        const long long prow = prow0 + (long long)c * p.rows_blk;
        const float w = exp2_fast(p.spart_lse[prow] - mx);
        const u32x4_t x = *(const u32x4_t*)(p.spart_o + prow * kDv + 8 * lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc0[e] += w * __uint_as_float(x[e >> 1] << (16 * ((e & 1) ^ 1)) & 0xFFFF0000u);
          acc1[e] += w * __uint_as_float(x[2 + (e >> 1)] << (16 * ((e & 1) ^ 1)) & 0xFFFF0000u);
        }
        wsum += w;
      }
    }
  }
  const bool any = wsum > 0.f;
  const float inv = any ? 1.f / wsum : 0.f;
  acc0 *= inv;
  acc1 *= inv;
  if (p.out_bf16) {
    __bf16* dst = (__bf16*)p.out + orow * kDv + 8 * lane;
    bf16x8_t v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = (__bf16)acc0[e];
      v[4 + e] = (__bf16)acc1[e];
    }
    *(bf16x8_t*)dst = v;
  } else {
    f32x4_t* dst = (f32x4_t*)((float*)p.out + orow * kDv + 8 * lane);
    dst[0] = acc0;
    dst[1] = acc1;
  }
  if (lane == 0) {
    const float lse2 = any ? mx + log2_fast(wsum) : kNegInf;
    p.lse[orow] = p.lse_base2 ? lse2 : lse2 * kLn2;
  }
}

}  // namespace

// 64-row blocks run the warp-specialised kernel (fp8 KV too)
constexpr bool kUseWs = true;
constexpr bool kUseWsFp8 = true;

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
  const bool local = p.local_kv_indices != nullptr;
  const bool ws = kUseWs && p.rows_blk == kWsRows && (!p.kv_fp8 || kUseWsFp8);
  if (p.kv_fp8 && !ws)
    fn = p.rows_blk == 32 ? reinterpret_cast<const void*>(&attn_stream_kernel<4, true>)
                          : reinterpret_cast<const void*>(&attn_stream_kernel<2, true>);
  else if (p.kv_fp8)
    fn = local ? reinterpret_cast<const void*>(&attn_ws_kernel<true, true>)
               : reinterpret_cast<const void*>(&attn_ws_kernel<false, true>);
  else if (ws)
    fn = local ? reinterpret_cast<const void*>(&attn_ws_kernel<true, false>)
               : reinterpret_cast<const void*>(&attn_ws_kernel<false, false>);
  else
    fn = p.rows_blk == 32 ? (local ? reinterpret_cast<const void*>(&attn_pipe_kernel<4, true>)
                                   : reinterpret_cast<const void*>(&attn_pipe_kernel<4, false>))
                          : (local ? reinterpret_cast<const void*>(&attn_pipe_kernel<2, true>)
                                   : reinterpret_cast<const void*>(&attn_pipe_kernel<2, false>));
  err = hipExtLaunchKernel(fn, dim3(p.grid), dim3(ws ? 512 : 256), args, 0, stream, ev_begin, ev_end, 0);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(stream_combine_kernel, dim3(p.batch, (p.rows + 3) / 4), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
