// Combine of a shard's pieces for gfx950: segments (request, 64-row block)
// that the attention kernel's schedule cut at workgroup boundaries leave one
// bf16 partial (and LSE) per piece; this kernel merges them with the same
// LSE-weighted softmax reduction the cross-shard merge uses (github.com
// sgl-project/sglang PR 33364, Modifications, the fourth kernel) into the
// shard's (out, lse), and writes the neutral (0, -inf) for requests whose
// shard owns no token (prhub.com.cn digest of sgl-project/sglang PR 33926,
// 实现拆解 step 3). When one launch runs every shard, the pieces of all
// shards' segments of a row block are merged here in one pass, which is the
// cross-shard merge of the same paragraph fused with the piece combine.
#include "mla_device.h"

namespace mla {
namespace {

// Max over the wave that propagates NaN: a piece that read a poisoned KV
// row carries a NaN LSE, and the row it contributes to must come out NaN
// (out and LSE), not be skipped as if it were empty (fmaxf alone drops NaN).
__device__ __forceinline__ float wave_max(float x) {
  const bool nan = __ballot(x != x) != 0;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return nan ? __builtin_nanf("") : x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

// One wave per query row of a segment cut into np pieces: the LSE of piece c
// sits in lane c (64 pieces at a time), and the bf16 partials of kPieces
// pieces (8 dims per lane) are loaded together, the first group in the same
// round trip as the LSEs; pieces are then accumulated in order. Four pieces
// at a time rather than eight: fewer registers, more waves in flight
// (9.0 -> 8.2 µs per shard on average over the kimi-like, fp8 and skewed
// workloads).
__global__ __launch_bounds__(256) void stream_combine_kernel(DecodeParams p) {
  constexpr int kPieces = 4;
  const int b = blockIdx.x;
  // the attention launch before this kernel is complete: its row-block
  // groups' rendezvous counters go back to zero for the next launch
  if (b == 0 && blockIdx.y == 0 && p.fold > 1) {
    for (int q = threadIdx.x; q < kMaxGrid; q += blockDim.x) p.grp_sync[q] = 0;
  }
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  const int rb = row / p.rows_blk;
  // pieces of the row block: those of its one segment (a segment held by one
  // workgroup was finalised in place), or, when the launch runs several
  // shards, those of its shards' neighbouring segments, whose partial slots
  // are consecutive
  const int s0 = (b * p.row_blocks + rb) * p.fold;
  const int4 si = p.seg_info[s0];
  int np = si.y;
  if (p.fold == 1 && np == 1) return;
  if (p.fold > 1) {
    const int4 sl = p.seg_info[s0 + p.fold - 1];
    np = sl.x + sl.y - si.x;
  }
  const long long orow = (long long)b * p.rows + row;
  f32x4_t acc0 = f32x4_t{}, acc1 = f32x4_t{};
  float mx = kNegInf, wsum = 0.f;
  if (np > 0) {
    const long long prow0 = (long long)si.x * p.rows_blk + (row - rb * p.rows_blk);
    auto piece_lse = [&](int c) { return c < np ? p.spart_lse[prow0 + (long long)c * p.rows_blk] : kNegInf; };
    auto piece_o = [&](int c) {
      return *(const u32x4_t*)(p.spart_o + (prow0 + (long long)c * p.rows_blk) * kDv + 8 * lane);
    };
    const float lse_lo = piece_lse(lane);
    u32x4_t xs[kPieces];
#pragma unroll
    for (int u = 0; u < kPieces; ++u)
      if (u < np) xs[u] = piece_o(u);
    mx = wave_max(lse_lo);
    for (int c0 = 64; c0 < np; c0 += 64) {
      const float m2 = wave_max(piece_lse(c0 + lane));
      mx = (m2 != m2 || mx != mx) ? __builtin_nanf("") : fmaxf(mx, m2);
    }
    if (mx != kNegInf) {
      for (int c0 = 0; c0 < np; c0 += 64) {
        const float l = c0 == 0 ? lse_lo : piece_lse(c0 + lane);
        const float w = exp2_fast(l - mx);            // 0 for pieces past np (lse -inf)
        wsum += wave_sum(w);
        const int n = min(64, np - c0);
        for (int u0 = 0; u0 < n; u0 += kPieces) {
          if (c0 + u0 > 0) {
#pragma unroll
            for (int u = 0; u < kPieces; ++u)
              if (u0 + u < n) xs[u] = piece_o(c0 + u0 + u);
          }
#pragma unroll
          for (int u = 0; u < kPieces; ++u) {
            if (u0 + u < n) {
              const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u0 + u));
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                acc0[e] += wu * __uint_as_float(xs[u][e >> 1] << (16 * ((e & 1) ^ 1)) & 0xFFFF0000u);
                acc1[e] += wu * __uint_as_float(xs[u][2 + (e >> 1)] << (16 * ((e & 1) ^ 1)) & 0xFFFF0000u);
              }
            }
          }
        }
      }
    }
  }
  // wsum is NaN when a piece was poisoned: then out and LSE are NaN too
  const bool any = wsum > 0.f || wsum != wsum;
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

hipError_t launch_combine(const DecodeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(stream_combine_kernel, dim3(p.batch, (p.rows + 3) / 4), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
