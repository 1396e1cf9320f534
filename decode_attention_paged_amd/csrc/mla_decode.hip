// Rank-local paged MLA decode for gfx950 (MI355X).
//
// Computes, for one context shard r of S, softmax attention of every query
// row over the KV tokens the shard owns (token t belongs to shard t mod S;
// prhub.com.cn digest of sgl-project/sglang PR 33926, sections 功能与动机 and
// 实现拆解 step 3), emitting (out, lse) with the neutral (0, -inf) for rows
// that see no owned token.
//
// Three kernels per call, all on the caller's stream:
//   plan_kernel    splits the shard's tokens into equal chunks over the
//                  compute units (split-KV schedule derived on device from the
//                  lengths, so the call needs no host synchronisation);
//   attn_kernel    one workgroup per (chunk, 128-query-row block): KV tiles of
//                  32 tokens are gathered from their pages into LDS once and
//                  shared by four waves of 32 query rows each; S^T = K Q^T and
//                  O^T += V^T P^T run on 32x32x16 bf16 MFMA with an online
//                  base-2 softmax; a request held by one chunk is finalised in
//                  place, otherwise a normalised partial goes to workspace;
//   combine_kernel LSE-weighted combine of a request's chunk partials.
//
// Data layout in LDS per stage (one 32-token tile):
//   K tile  [32 tokens][72 chunks of 16 B], chunk c of token t stored at
//           slot 72 t + (c ^ h(t)) with h(t) = (t & 7) ^ ((t >> 3) & 1):
//           the MFMA A-operand reads (token = lane % 32) hit distinct banks.
//   Vt tile [512 dims][4 groups of 8 tokens] (bf16), the transposed V needed
//           as the A operand of O^T += V^T P^T. The token order inside a
//           group matches the order of P values that the S^T accumulator
//           leaves in each lane, so P never leaves registers.
#include "mla_device.h"

#include <hip/hip_ext.h>
#include <limits.h>

namespace mla {
namespace {

// The exponent reference of a row is fixed at the max of the first tile that
// holds a visible token, so the output accumulator is never rescaled inside
// the tile loop. Unnormalised probabilities stay below 2^kOverflowSlack; a
// later tile whose max exceeds the reference by more than that makes the
// workgroup redo the chunk with the chunk's true max as the reference.
constexpr float kOverflowSlack = 64.0f;

constexpr int kKBytes = kTile * kDqk * 2;        // 36864
constexpr int kVtBytes = kDv * 4 * 16;           // 32768
constexpr int kStageBytes = kKBytes + kVtBytes;  // 69632
constexpr int kChunks = kDqk / 8;                // 72 chunks of 8 dims per row

// Physical KV row of the shard's j-th owned token of request b (j < count),
// or -1 when the page id / row is outside the pool.
__device__ __forceinline__ int kv_row(const DecodeParams& p, int b, int j) {
  long long row;
  if (p.local_kv_indices != nullptr) {
    row = p.local_kv_indices[(long long)b * p.local_kv_stride + j];
  } else {
    const int t = j * p.num_shards + p.shard;
    const int page = p.block_table[(long long)b * p.max_pages + (t >> 6)];
    row = (page < 0 || page >= p.num_pages) ? -1 : (long long)page * kPage + (t & 63);
  }
  return (row < 0 || row >= (long long)p.num_pages * kPage) ? -1 : (int)row;
}

// ---------------------------------------------------------------------------
// plan: chunk size and the (request, chunk) work list
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void plan_kernel(DecodeParams p) {
  __shared__ long long s_part[16];
  __shared__ int s_scan[1024];
  __shared__ int s_chunk;
  __shared__ int s_base;
  const int tid = threadIdx.x;

  long long tot = 0;
  for (int b = tid; b < p.batch; b += 1024) tot += local_count(p, b);
  for (int off = 32; off > 0; off >>= 1) tot += __shfl_xor(tot, off);
  if ((tid & 63) == 0) s_part[tid >> 6] = tot;
  __syncthreads();
  if (tid == 0) {
    long long all = 0;
    for (int w = 0; w < 16; ++w) all += s_part[w];
    const long long target = p.split_target;
    long long c = (all + target - 1) / target;
    c = ((c + kTile - 1) / kTile) * kTile;
    if (c < kMinChunk) c = kMinChunk;
    if (c > INT_MAX / 4) c = INT_MAX / 4;
    s_chunk = (int)c;
    s_base = 0;
  }
  __syncthreads();
  const int C = s_chunk;

  for (int base = 0; base < p.batch; base += 1024) {
    const int b = base + tid;
    int n = 0;
    if (b < p.batch) {
      const int cnt = local_count(p, b);
      n = cnt > 0 ? (cnt + C - 1) / C : 1;   // an empty request still gets one item
    }
    s_scan[tid] = n;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int v = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    const int first = s_base + s_scan[tid] - n;
    if (b < p.batch) {
      p.req_info[b] = make_int2(first, n);
      for (int c = 0; c < n; ++c) p.items[first + c] = make_int2(b, c);
    }
    __syncthreads();
    if (tid == 1023) s_base += s_scan[1023];
    __syncthreads();
  }
  if (tid == 0) {
    p.plan[0] = s_base;
    p.plan[1] = C;
  }
}

// ---------------------------------------------------------------------------
// tile staging
// ---------------------------------------------------------------------------
// Token of tile position p (0..7) in group G (0..3): groups hold the tokens
// whose P values sit in k-slots of one half of one PV MFMA.
__device__ __forceinline__ int group_token(int G, int pidx) {
  return 16 * (G >> 1) + 4 * (G & 1) + 8 * (pidx >> 2) + (pidx & 3);
}

__device__ __forceinline__ int k_slot(int tok, int chunk) {
  const int h = (tok & 7) ^ ((tok >> 3) & 1);
  return kChunks * tok + (chunk ^ h);
}

// Vt slot (16-byte units) of (dim, group): the low four bits mix dim bits so
// that both the MFMA reads (consecutive dims) and the loader's writes (dims
// eight apart) spread over all banks.
__device__ __forceinline__ int vt_slot(int dim, int G) {
  const int b0 = dim & 1, b1 = (dim >> 1) & 1, b2 = (dim >> 2) & 1, b3 = (dim >> 3) & 1;
  const int b4 = (dim >> 4) & 1, b5 = (dim >> 5) & 1, b6 = (dim >> 6) & 1;
  const int low = (b0 ^ b4) | ((b1 ^ b5) << 1) | ((b2 ^ b3 ^ b6) << 2) | (b3 << 3);
  return 16 * (4 * (dim >> 4) + G) + low;
}

template <bool kFp8> struct Raw;
template <> struct Raw<false> { u32x4_t v[8]; u32x4_t rope; };
template <> struct Raw<true> { u32x2_t v[8]; u32x2_t rope; };

// OCP e4m3 -> bf16 bit pattern, exact. Normal codes (exponent field >= 1)
// move into the bf16 fields with the exponent rebiased from 7 to 127;
// subnormal codes are m * 2^-9 (m <= 7), exact in float; S.1111.111 is NaN.
__device__ __forceinline__ uint32_t e4m3_to_bf16_bits(uint32_t x) {
  const uint32_t em = x & 0x7Fu;
  const uint32_t sign = (x & 0x80u) << 8;
  const uint32_t normal = (em << 4) + (120u << 7);
  const uint32_t sub = __float_as_uint((float)em * 0x1p-9f) >> 16;
  const uint32_t mag = em == 0x7Fu ? 0x7FC0u : (em >= 8u ? normal : sub);
  return sign | mag;
}

// 8 e4m3 bytes -> 8 bf16 (as four 32-bit words)
__device__ __forceinline__ u32x4_t e4m3x8_to_bf16x8(u32x2_t w) {
  u32x4_t r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t word = w[k >> 1] >> (16 * (k & 1));
    r[k] = e4m3_to_bf16_bits(word & 0xFFu) | (e4m3_to_bf16_bits((word >> 8) & 0xFFu) << 16);
  }
  return r;
}

template <bool kFp8>
__device__ __forceinline__ void load_tile(const DecodeParams& p, int b, int jt, int j1, Raw<kFp8>& raw) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int G = __builtin_amdgcn_readfirstlane(tid >> 6);
  // rows of the tile's 32 tokens, computed by lanes 0..31 of every wave:
  // -2 = past the chunk end (zero fill), -1 = bad page (NaN fill). Loads are
  // issued unconditionally from row 0 for those and replaced afterwards, so
  // the loader has no branches.
  int my_row = -2;
  if (lane < kTile && jt + lane < j1) my_row = kv_row(p, b, jt + lane);
  constexpr int row_bytes = kFp8 ? kDqk : 2 * kDqk;
  constexpr int chunk_bytes = kFp8 ? 8 : 16;
  constexpr uint32_t kNanFill = kFp8 ? 0x7F7F7F7Fu : 0x7FC07FC0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = __builtin_amdgcn_readlane(my_row, group_token(G, i));
    const uint8_t* src = p.kv + (long long)(r >= 0 ? r : 0) * row_bytes + lane * chunk_bytes;
    const uint32_t fill = r == -1 ? kNanFill : 0u;
    if constexpr (kFp8) {
      const u32x2_t x = *(const u32x2_t*)src;
      raw.v[i] = r >= 0 ? x : u32x2_t{fill, fill};
    } else {
      const u32x4_t x = *(const u32x4_t*)src;
      raw.v[i] = r >= 0 ? x : u32x4_t{fill, fill, fill, fill};
    }
  }
  // rope dims (chunks 64..71): token tid / 8, chunk 64 + tid % 8
  const int r = __shfl(my_row, tid >> 3);
  const uint8_t* src = p.kv + (long long)(r >= 0 ? r : 0) * row_bytes + (64 + (tid & 7)) * chunk_bytes;
  const uint32_t fill = r == -1 ? kNanFill : 0u;
  if constexpr (kFp8) {
    const u32x2_t x = *(const u32x2_t*)src;
    raw.rope = r >= 0 ? x : u32x2_t{fill, fill};
  } else {
    const u32x4_t x = *(const u32x4_t*)src;
    raw.rope = r >= 0 ? x : u32x4_t{fill, fill, fill, fill};
  }
}

template <bool kFp8>
__device__ __forceinline__ void store_tile(uint8_t* stage, const Raw<kFp8>& raw) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int G = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint8_t* ks = stage;
  uint8_t* vt = stage + kKBytes;
  u32x4_t d[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if constexpr (kFp8) d[i] = e4m3x8_to_bf16x8(raw.v[i]);
    else d[i] = raw.v[i];
    *(u32x4_t*)(ks + 16 * k_slot(group_token(G, i), lane)) = d[i];
  }
  {
    u32x4_t rp;
    if constexpr (kFp8) rp = e4m3x8_to_bf16x8(raw.rope);
    else rp = raw.rope;
    *(u32x4_t*)(ks + 16 * k_slot(tid >> 3, 64 + (tid & 7))) = rp;
  }
  // transpose the 8 tokens x 8 dims block: column e holds dim 8*lane+e of
  // the group's tokens in position order
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    u32x4_t col;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t lo = d[2 * w][e >> 1], hi = d[2 * w + 1][e >> 1];
      col[w] = (e & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
    }
    *(u32x4_t*)(vt + 16 * vt_slot(8 * lane + e, G)) = col;
  }
}

// ---------------------------------------------------------------------------
// attention over one chunk for 128 query rows
// ---------------------------------------------------------------------------
template <bool kFp8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  int item, rbk;
  if (p.row_blocks == 1) {
    item = blockIdx.x;
    rbk = 0;
  } else {
    // the row blocks of one chunk get ids congruent mod 8, i.e. the same XCD,
    // so their repeated reads of the chunk's KV are served by that XCD's L2
    const int x = blockIdx.x & 7, s = blockIdx.x >> 3;
    item = (s / p.row_blocks) * 8 + x;
    rbk = s % p.row_blocks;
  }
  if (item >= p.plan[0]) return;
  const int2 it = p.items[item];
  const int b = it.x;
  const int chunk = p.plan[1];
  const int cnt = local_count(p, b);
  const int j0 = it.y * chunk;
  const int j1 = min(cnt, j0 + chunk);
  const int L = req_len(p, b);
  const bool single = p.req_info[b].y == 1;

  const int row = rbk * kRowsPerBlock + wave * kRowsPerWave + (lane & 31);
  const bool row_ok = row < p.rows;
  const bool wave_active = rbk * kRowsPerBlock + wave * kRowsPerWave < p.rows;

  // local index bound of the tokens this row may see: t = j*S + r <= L - q + i
  int jvis = j1;
  if (row_ok) {
    const int i = row / p.heads;
    const int lim = L - p.q_len + i - p.shard;
    const int jl = lim >= 0 ? lim / p.num_shards + 1 : 0;
    jvis = min(j1, jl);
  }

  bf16x8_t qreg[kDqk / 16];
  {
    // rows past the end load row 0 and are zeroed (branch-free)
    const uint16_t* qrow = p.q + ((long long)b * p.rows + (row_ok ? row : 0)) * kDqk + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < kDqk / 16; ++ks) {
      const bf16x8_t x = *(const bf16x8_t*)(qrow + 16 * ks);
      qreg[ks] = row_ok ? x : bf16x8_t{};
    }
  }

  // per-lane LDS offsets of the MFMA operands
  const int tok = lane & 31, hi = lane >> 5;
  const int h_tok = (tok & 7) ^ ((tok >> 3) & 1);
  const int ntiles = j1 > j0 ? (j1 - j0 + kTile - 1) / kTile : 0;

  f32x16_t o[kDv / 32];
  float m_ref = kNegInf;   // exponent reference (log2 domain)
  float m_all = kNegInf;   // true max over the chunk's visible scores
  float l_sum = 0.f;
  for (int attempt = 0; attempt < 2; ++attempt) {
#pragma unroll
    for (int db = 0; db < kDv / 32; ++db) o[db] = f32x16_t{};
    l_sum = 0.f;
    m_ref = attempt == 0 ? kNegInf : m_all;
    bool overflow = false;

    Raw<kFp8> raw;
    if (ntiles > 0) {
      load_tile<kFp8>(p, b, j0, j1, raw);
      store_tile<kFp8>(smem, raw);
    }
    __syncthreads();

    for (int tile = 0; tile < ntiles; ++tile) {
      const int jt = j0 + tile * kTile;
      const bool more = tile + 1 < ntiles;
      if (more) load_tile<kFp8>(p, b, jt + kTile, j1, raw);
      const uint8_t* ks = smem + (tile & 1) * kStageBytes;
      const uint8_t* vt = ks + kKBytes;

      if (wave_active) {
        // S^T[token][row] = sum_d K[token][d] Q[row][d]
        f32x16_t s = f32x16_t{};
#pragma unroll
        for (int kk = 0; kk < kDqk / 16; ++kk) {
          const int c = 2 * kk + hi;
          const bf16x8_t a = *(const bf16x8_t*)(ks + 16 * (kChunks * tok + (c ^ h_tok)));
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], s, 0, 0, 0);
        }
        // softmax numerators, base 2; a lane holds row (lane % 32) and 16 tokens
        float tmax = kNegInf;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = jt + 8 * (v >> 2) + 4 * hi + (v & 3);
          s[v] = j < jvis ? s[v] * p.scale_log2 : kNegInf;
          tmax = fmaxf(tmax, s[v]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        m_all = fmaxf(m_all, tmax);
        m_ref = m_ref == kNegInf ? tmax : m_ref;
        overflow = overflow || tmax > m_ref + kOverflowSlack;
        const float m_use = m_ref == kNegInf ? 0.f : m_ref;
        bf16x8_t pb[2];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float pv = exp2_fast(s[v] - m_use);
          l_sum += pv;
          pb[v >> 3][v & 7] = (__bf16)pv;
        }
        // O^T[dim][row] += sum_token V^T[dim][token] P^T[token][row]
#pragma unroll
        for (int db = 0; db < kDv / 32; ++db) {
          const int dim = 32 * db + tok;
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            const bf16x8_t a = *(const bf16x8_t*)(vt + 16 * vt_slot(dim, 2 * m + hi));
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[m], o[db], 0, 0, 0);
          }
        }
      }
      if (more) store_tile<kFp8>(smem + ((tile + 1) & 1) * kStageBytes, raw);
      __syncthreads();
    }
    if (!__syncthreads_or(overflow ? 1 : 0)) break;
  }

  if (!wave_active) return;
  const float l_tot = l_sum + __shfl_xor(l_sum, 32);
  const bool any = l_tot > 0.f;
  const float inv = any ? p.out_scale / l_tot : 0.f;
  const float lse2 = any ? m_ref + log2_fast(l_tot) : kNegInf;
  if (!row_ok) return;

  // a request held by one chunk is final here; otherwise write the chunk's
  // normalised partial (f32, base-2 lse) for the combine kernel
  const long long orow = (long long)b * p.rows + row;
  const long long prow = (long long)item * p.rows + row;
  if (single && p.out_bf16) {
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
    __bf16* dst = (__bf16*)p.out + orow * kDv + 4 * hi;
#pragma unroll
    for (int db = 0; db < kDv / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4_t v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(o[db][4 * g + e] * inv);
        *(bf16x4_t*)(dst + 32 * db + 8 * g) = v4;
      }
  } else {
    float* dst = (single ? (float*)p.out + orow * kDv : p.part_o + prow * kDv) + 4 * hi;
#pragma unroll
    for (int db = 0; db < kDv / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4_t v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = o[db][4 * g + e] * inv;
        *(f32x4_t*)(dst + 32 * db + 8 * g) = v4;
      }
  }
  if (hi == 0) {
    if (single) p.lse[orow] = p.lse_base2 ? lse2 : lse2 * kLn2;
    else p.part_lse[prow] = lse2;
  }
}

// ---------------------------------------------------------------------------
// bf16 KV: direct HBM -> LDS tiles, V^T read with transposing LDS loads
// ---------------------------------------------------------------------------
// A stage holds one 32-token tile chunk-major: 16-byte chunk c (dims
// 8c .. 8c+7) of tile token t sits at slot 32 c + (t ^ 4 (c & 3)).
//  * global_load_lds_dwordx4 moves 64 consecutive slots (1 KB) per
//    instruction = chunks 2q, 2q+1 of all 32 tokens, each lane keeping one
//    token, so a tile needs two row lookups per lane;
//  * the QK A operand (lane = token, 8 dims) of k-step kk is the contiguous
//    1 KB of chunks 2kk, 2kk+1;
//  * the PV A operand (V^T: lane = dim, 8 tokens) comes from two
//    ds_read_b64_tr_b16: in each 16-lane group, lane 4r + s supplies dims
//    4s .. 4s+3 of token r and lane i receives dim i of the four tokens (a
//    4 x 16 transpose), so V is never copied; the XOR term puts the four
//    chunks a 32-lane half reads in distinct 64-byte bank segments.
constexpr int kKTileBytes = kTile * kDqk * 2;   // 36864
constexpr int kDirectStages = 2;

// Row indices of a tile are fetched one iteration before they are used and
// validated only after the loop-top wait, so fetching them never forces a wait
// on the KV loads in flight. Lanes 0..31 hold token jt + lane.
constexpr int kRowPastEnd = -2;   // token past the chunk end: loads row 0, masked
constexpr int kRowBad = -1;       // page outside the pool: loads row 0, score NaN

__device__ __forceinline__ int fetch_row_raw(const DecodeParams& p, int b, int jt, int j1, int lane) {
  if (lane >= kTile || jt + lane >= j1) return INT_MIN;
  const int j = jt + lane;
  if (p.local_kv_indices != nullptr) return p.local_kv_indices[(long long)b * p.local_kv_stride + j];
  const int t = j * p.num_shards + p.shard;
  return p.block_table[(long long)b * p.max_pages + (t >> 6)];
}

__device__ __forceinline__ int resolve_row(const DecodeParams& p, int raw, int jt, int lane) {
  if (raw == INT_MIN) return kRowPastEnd;
  long long row;
  if (p.local_kv_indices != nullptr) {
    row = raw;
  } else {
    const int t = (jt + lane) * p.num_shards + p.shard;
    row = (raw < 0 || raw >= p.num_pages) ? -1 : (long long)raw * kPage + (t & 63);
  }
  return (row < 0 || row >= (long long)p.num_pages * kPage) ? kRowBad : (int)row;
}

// Direct loads of one tile into a stage. Block q (1 KB) of the stage holds
// chunks 2q + hi of tokens (lane % 32) ^ 4 (c & 3); `my_row` is the row of
// token (lane % 32) of the tile, valid in lanes 0..31. prepare() fetches the
// two source rows this lane needs; issue(i) sends the wave's i-th block.
template <int kNW>
struct TileDma {
  static constexpr int kBlocks = kKTileBytes / 1024;   // 36 instructions of 1 KB
  static constexpr int kPerWave = kBlocks / kNW;
  const uint8_t* src_even;
  const uint8_t* src_odd;
  uint32_t lds0;

  __device__ __forceinline__ void prepare(const DecodeParams& p, const uint8_t* stage, int my_row) {
    const int lane = threadIdx.x & 63, hi = lane >> 5;
    const int r_even = __shfl(my_row, (lane & 31) ^ (4 * hi));
    const int r_odd = __shfl(my_row, (lane & 31) ^ (8 + 4 * hi));
    src_even = p.kv + (long long)(r_even >= 0 ? r_even : 0) * (2 * kDqk) + 16 * hi;
    src_odd = p.kv + (long long)(r_odd >= 0 ? r_odd : 0) * (2 * kDqk) + 16 * hi;
    lds0 = __builtin_amdgcn_readfirstlane(lds_address(stage));
  }
  __device__ __forceinline__ void issue(int i) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q = wave * kPerWave + i;
    // the parity of q selects the source row (c & 3 = 2 (q & 1) + hi)
    const uint8_t* src = ((kPerWave & 1) == 0 ? (i & 1) : (q & 1)) ? src_odd : src_even;
    lds_dma16(src + 32 * q, __builtin_amdgcn_readfirstlane(lds0 + 1024 * q));
  }
  __device__ __forceinline__ void issue_all() const {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) issue(i);
  }
};

// PV A operand of step st = 2 db + m: dims 32 db .. + 31 of tokens
// 16 m .. 16 m + 15 (two transposing loads of four tokens each).
__device__ __forceinline__ bf16x8_t pv_operand(const uint8_t* ks, const uint32_t (&pv_base)[2], int st) {
  const int db = st >> 1, m = st & 1;
  const i16x4_t lo = lds_read_tr16(ks + pv_base[0] + 2048 * db + 256 * m);
  const i16x4_t hi = lds_read_tr16(ks + pv_base[1] + 2048 * db + 256 * m);
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int kNW>
__global__ __launch_bounds__(64 * kNW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_direct_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kDirectStages * kKTileBytes];
  // the last kQInLds k-steps of each lane's Q operands live in LDS rather than
  // VGPRs (read back once per tile), which keeps the tile loop free of spills
  constexpr int kQInLds = kNW <= 2 ? 3 : 2;
  constexpr int kQRegSteps = kDqk / 16 - kQInLds;
  __shared__ __attribute__((aligned(16))) uint8_t qlds[kNW * kQInLds * 64 * 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int kRowsWG = kNW * kRowsPerWave;

  int item, rbk;
  if (p.row_blocks == 1) {
    item = blockIdx.x;
    rbk = 0;
  } else {
    // the row blocks of one chunk get ids congruent mod 8, i.e. the same XCD,
    // so their repeated reads of the chunk's KV are served by that XCD's L2
    const int x = blockIdx.x & 7, sx = blockIdx.x >> 3;
    item = (sx / p.row_blocks) * 8 + x;
    rbk = sx % p.row_blocks;
  }
  if (item >= p.plan[0]) return;
  const int2 it = p.items[item];
  const int b = it.x;
  const int chunk = p.plan[1];
  const int cnt = local_count(p, b);
  const int j0 = it.y * chunk;
  const int j1 = min(cnt, j0 + chunk);
  const int L = req_len(p, b);
  const bool single = p.req_info[b].y == 1;

  const int row = rbk * kRowsWG + wave * kRowsPerWave + (lane & 31);
  const bool row_ok = row < p.rows;
  const bool wave_active = rbk * kRowsWG + wave * kRowsPerWave < p.rows;
  int jvis = j1;
  if (row_ok) {
    const int i = row / p.heads;
    const int lim = L - p.q_len + i - p.shard;
    const int jl = lim >= 0 ? lim / p.num_shards + 1 : 0;
    jvis = min(j1, jl);
  }

  // row indices of the first two tiles are requested before the Q loads so
  // their latency overlaps
  const int raw0 = fetch_row_raw(p, b, j0, j1, lane);
  const int raw1 = fetch_row_raw(p, b, j0 + kTile, j1, lane);

  bf16x8_t qreg[kQRegSteps];
  uint8_t* const qmine = qlds + 16 * (kQInLds * 64 * wave + lane);
  {
    const uint16_t* qrow = p.q + ((long long)b * p.rows + (row_ok ? row : 0)) * kDqk + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < kDqk / 16; ++ks) {
      bf16x8_t x = *(const bf16x8_t*)(qrow + 16 * ks);
      x = row_ok ? x : bf16x8_t{};
      if (ks < kQRegSteps) qreg[ks] = x;
      else *(bf16x8_t*)(qmine + 16 * 64 * (ks - kQRegSteps)) = x;
    }
  }

  const int tok = lane & 31, hi = lane >> 5;
  const int ntiles = j1 > j0 ? (j1 - j0 + kTile - 1) / kTile : 0;
  // QK operand of k-step kk: slot 32 (2 kk + hi) + (tok ^ (8 (kk & 1) + 4 hi))
  const uint32_t qk_base[2] = {512u * hi + 16u * (tok ^ (4 * hi)), 512u * hi + 16u * (tok ^ (8 + 4 * hi))};
  // PV transposing loads: this lane supplies token t = 16 m + 8 k + 4 hi + r,
  // dims 32 db + 16 g1 + 4 s .. + 3 (chunk 4 db + cl, cl = 2 g1 + (s >> 1))
  uint32_t pv_base[2];
  {
    const int g1 = (lane >> 4) & 1, r = (lane & 15) >> 2, sq = lane & 3;
    const int cl = 2 * g1 + (sq >> 1);
#pragma unroll
    for (int k = 0; k < 2; ++k)
      pv_base[k] = (uint32_t)(512 * cl + 128 * (k ^ g1) + 64 * (hi ^ (sq >> 1)) + 16 * r + 8 * (sq & 1));
  }

  f32x16_t o[kDv / 32];
  float m_ref = kNegInf, m_all = kNegInf, l_sum = 0.f;
  for (int attempt = 0; attempt < 2; ++attempt) {
#pragma unroll
    for (int db = 0; db < kDv / 32; ++db) o[db] = f32x16_t{};
    l_sum = 0.f;
    m_ref = attempt == 0 ? kNegInf : m_all;
    bool overflow = false;

    int rows_cur = kRowPastEnd;
    int raw_next = INT_MIN;
    TileDma<kNW> dma;
    if (ntiles > 0) {
      rows_cur = resolve_row(p, raw0, j0, lane);
      dma.prepare(p, smem, rows_cur);
      dma.issue_all();
      raw_next = raw1;
    }

    for (int tile = 0; tile < ntiles; ++tile) {
      const int jt = j0 + tile * kTile;
      const bool more = tile + 1 < ntiles;
      // tokens of this tile whose page is outside the pool poison their scores
      const uint64_t bad = __ballot(lane < kTile && rows_cur == kRowBad);
      __builtin_amdgcn_s_waitcnt(0);     // this tile's loads (and the next rows) have landed
      __syncthreads();                   // ... for every wave; the other stage is free
      if (more) {
        rows_cur = resolve_row(p, raw_next, jt + kTile, lane);
        dma.prepare(p, smem + ((tile + 1) & 1) * kKTileBytes, rows_cur);
        dma.issue_all();
        raw_next = fetch_row_raw(p, b, jt + 2 * kTile, j1, lane);
      }
      const uint8_t* ks = smem + (tile & 1) * kKTileBytes;
      // every wave runs the MFMAs (a wave past the last row works on zero
      // queries and writes nothing): keeping the accumulators out of a
      // conditional block lets them stay in AGPRs across the tile loop
      {
        // S^T[token][row]; K operands are read two steps ahead of their MFMA
        constexpr int kKSteps = kDqk / 16;
        constexpr int kAhead = 2;
        bf16x8_t ka[kAhead];
#pragma unroll
        for (int u = 0; u < kAhead; ++u) ka[u] = *(const bf16x8_t*)(ks + qk_base[u & 1] + 1024 * u);
        f32x16_t s = f32x16_t{};
#pragma unroll
        for (int kk = 0; kk < kKSteps; ++kk) {
          const bf16x8_t a = ka[kk % kAhead];
          if (kk + kAhead < kKSteps) {
            const int kn = kk + kAhead;
            ka[kk % kAhead] = *(const bf16x8_t*)(ks + qk_base[kn & 1] + 1024 * kn);
          }
          const bf16x8_t qb = kk < kQRegSteps ? qreg[kk < kQRegSteps ? kk : 0]
                                              : *(const bf16x8_t*)(qmine + 16 * 64 * (kk - kQRegSteps));
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb, s, 0, 0, 0);
        }
        float tmax = kNegInf;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int tl = 8 * (v >> 2) + 4 * hi + (v & 3);
          const int j = jt + tl;
          float x = j < jvis ? s[v] * p.scale_log2 : kNegInf;
          x = ((bad >> tl) & 1) ? __builtin_nanf("") : x;
          s[v] = x;
          tmax = fmaxf(tmax, x);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        m_all = fmaxf(m_all, tmax);
        m_ref = m_ref == kNegInf ? tmax : m_ref;
        overflow = overflow || tmax > m_ref + kOverflowSlack;
        const float m_use = m_ref == kNegInf ? 0.f : m_ref;
        bf16x8_t pb[2];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float pv = exp2_fast(s[v] - m_use);
          l_sum += pv;
          pb[v >> 3][v & 7] = (__bf16)pv;
        }
        // O^T[dim][row] += V^T[dim][token] P^T[token][row]
        constexpr int kPvSteps = 2 * (kDv / 32);
        bf16x8_t va[kAhead];
#pragma unroll
        for (int u = 0; u < kAhead; ++u) va[u] = pv_operand(ks, pv_base, u);
#pragma unroll
        for (int st = 0; st < kPvSteps; ++st) {
          const bf16x8_t a = va[st % kAhead];
          if (st + kAhead < kPvSteps) va[st % kAhead] = pv_operand(ks, pv_base, st + kAhead);
          o[st >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[st & 1], o[st >> 1], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 1);
#pragma unroll
        for (int st = 0; st < kPvSteps; ++st) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
          if (st + kAhead < kPvSteps) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        }
      }
    }
    if (!__syncthreads_or(overflow ? 1 : 0)) break;
  }

  if (!wave_active) return;
  const float l_tot = l_sum + __shfl_xor(l_sum, 32);
  const bool any = l_tot > 0.f || l_tot != l_tot;
  const float inv = any ? p.out_scale / l_tot : 0.f;
  const float lse2 = any ? m_ref + log2_fast(l_tot) : kNegInf;
  if (!row_ok) return;
  const long long orow = (long long)b * p.rows + row;
  const long long prow = (long long)item * p.rows + row;
  if (single && p.out_bf16) {
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
    __bf16* dst = (__bf16*)p.out + orow * kDv + 4 * hi;
#pragma unroll
    for (int db = 0; db < kDv / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4_t v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(o[db][4 * g + e] * inv);
        *(bf16x4_t*)(dst + 32 * db + 8 * g) = v4;
      }
  } else {
    float* dst = (single ? (float*)p.out + orow * kDv : p.part_o + prow * kDv) + 4 * hi;
#pragma unroll
    for (int db = 0; db < kDv / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4_t v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = o[db][4 * g + e] * inv;
        *(f32x4_t*)(dst + 32 * db + 8 * g) = v4;
      }
  }
  if (hi == 0) {
    if (single) p.lse[orow] = p.lse_base2 ? lse2 : lse2 * kLn2;
    else p.part_lse[prow] = lse2;
  }
}

// ---------------------------------------------------------------------------
// combine the chunk partials of requests split over several workgroups
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(DecodeParams p) {
  const int b = blockIdx.x;
  const int2 ri = p.req_info[b];
  if (ri.y <= 1) return;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (row >= p.rows) return;

  float mx = kNegInf;
  for (int c = 0; c < ri.y; ++c) mx = fmaxf(mx, p.part_lse[(long long)(ri.x + c) * p.rows + row]);
  f32x4_t acc0 = f32x4_t{}, acc1 = f32x4_t{};
  float wsum = 0.f;
  if (mx != kNegInf) {
    for (int c = 0; c < ri.y; ++c) {
      const long long prow = (long long)(ri.x + c) * p.rows + row;
      const float w = exp2_fast(p.part_lse[prow] - mx);
      const f32x4_t* src = (const f32x4_t*)(p.part_o + prow * kDv + 8 * lane);
      acc0 += w * src[0];
      acc1 += w * src[1];
      wsum += w;
    }
  }
  const bool any = wsum > 0.f;
  const float inv = any ? 1.f / wsum : 0.f;
  acc0 *= inv;
  acc1 *= inv;
  const long long orow = (long long)b * p.rows + row;
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

hipError_t launch_decode(const DecodeParams& p, bool fp8, hipEvent_t ev_begin, hipEvent_t ev_end,
                         hipStream_t stream) {
  if (p.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int items = p.batch + p.split_target;
  const int grid = p.row_blocks == 1 ? items : ((items + 7) / 8) * 8 * p.row_blocks;
  const int nw = p.rows >= 128 ? 4 : (p.rows + 31) / 32;
  void* args[] = {const_cast<DecodeParams*>(&p)};
  const void* fn;
  dim3 block(256);
  if (fp8) fn = reinterpret_cast<const void*>(&attn_kernel<true>);
  else if (nw == 4 || nw == 3) fn = reinterpret_cast<const void*>(&attn_direct_kernel<4>);
  else if (nw == 2) {
    fn = reinterpret_cast<const void*>(&attn_direct_kernel<2>);
    block = dim3(128);
  } else {
    fn = reinterpret_cast<const void*>(&attn_direct_kernel<1>);
    block = dim3(64);
  }
  // the events, when given, take the attention kernel's own start and end times
  err = hipExtLaunchKernel(fn, dim3(grid), block, args, 0, stream, ev_begin, ev_end, 0);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(combine_kernel, dim3(p.batch, (p.rows + 3) / 4), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
