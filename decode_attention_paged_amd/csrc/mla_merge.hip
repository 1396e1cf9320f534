// Cross-shard LSE-weighted merge and shard-local metadata for gfx950.
//
// Merge: the LSE-weighted softmax reduction of every shard's partial output
// into the full-context result (github.com sgl-project/sglang PR 33364,
// "[Attention][DCP] Add symm_a2a ...", Modifications, the fourth kernel; the
// LSE base is resolved here, at the merge site, as the prhub.com.cn digest of
// sgl-project/sglang PR 33926 notes under its related PRs). Bandwidth-bound:
// one wave per (row, head) vector, each lane owning 8 consecutive elements,
// so every shard's vector is read with one coalesced 16- or 32-byte load per
// lane, all shards' loads in flight at once, and the output written once.
//
// Metadata: the shard-local lengths and token-granular KV indices of the
// rank's cyclic slice (prhub.com.cn digest of sgl-project/sglang PR 33926,
// 关键源码片段: the DCP metadata helpers).
#include "mla_internal.h"

#include <hip/hip_ext.h>

namespace mla {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
constexpr float kNegInf = -__builtin_inff();

// Vectors per wave (all their loads in flight together) and whether the
// partials are read and the result written with non-temporal hints (each
// byte is touched once).
constexpr int kMergeVecsPerWave = 1;
constexpr bool kMergeNonTemporal = true;
constexpr int kMergeWaves = 4;   // waves per workgroup

template <typename T>
__device__ __forceinline__ T load_stream(const T* p) {
  if constexpr (kMergeNonTemporal) return __builtin_nontemporal_load(p);
  else return *p;
}
template <typename T>
__device__ __forceinline__ void store_stream(T* p, const T& v) {
  if constexpr (kMergeNonTemporal) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// Eight consecutive elements of shard r's partials at element index e, as
// stored: one 16-byte word group for bf16 (kept packed until they are
// accumulated, which halves the registers that hold every shard's chunk),
// two for f32.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <bool kBf16>
struct Raw8 {
  u32x4_t w[kBf16 ? 1 : 2];
};
template <bool kBf16>
__device__ __forceinline__ Raw8<kBf16> load8(const MergeParams& p, int r, long long e) {
  Raw8<kBf16> x;
  if constexpr (kBf16) {
    x.w[0] = load_stream((const u32x4_t*)((const __bf16*)p.outs[r] + e));
  } else {
    const u32x4_t* q = (const u32x4_t*)((const float*)p.outs[r] + e);
    x.w[0] = load_stream(q);
    x.w[1] = load_stream(q + 1);
  }
  return x;
}
// element k (0..7) of a chunk as fp32 (bf16: the upper half of a binary32)
template <bool kBf16>
__device__ __forceinline__ float elem(const Raw8<kBf16>& x, int k) {
  if constexpr (kBf16) return __uint_as_float((x.w[0][k >> 1] << (16 * ((k & 1) ^ 1))) & 0xFFFF0000u);
  else return __uint_as_float(x.w[k >> 2][k & 3]);
}

// kS: shard count rounded up to a power of two (registers for kS vectors);
// kV: vectors per wave; kBf16: partials stored as bf16 (else f32).
template <int kS, int kV, bool kBf16>
__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(MergeParams p) {
  const long long vec0 =
      (long long)__builtin_amdgcn_readfirstlane((int)(blockIdx.x * kMergeWaves + (threadIdx.x >> 6))) * kV;
  if (vec0 >= p.vectors) return;
  const int lane = threadIdx.x & 63;
  const int S = p.num_shards;

  // every load of the wave is issued before any result is used: the shards'
  // LSEs (scalar loads, the vector index is wave-uniform) and the first
  // 512-element chunk of every shard's vector (one 16- or 32-byte load per
  // lane); a shard with weight 0 holds zeros, so loading it is harmless
  float lse2[kV][kS];
  Raw8<kBf16> x[kV][kS];
  const int e_first = 8 * lane;
  const bool have = e_first < p.dv;
#pragma unroll
  for (int u = 0; u < kV; ++u) {
    const long long vec = vec0 + u < p.vectors ? vec0 + u : p.vectors - 1;
#pragma unroll
    for (int r = 0; r < kS; ++r) {
      if (r < S) {
        lse2[u][r] = *(const __attribute__((address_space(4))) float*)(p.lses[r] + vec) * p.lse_to_log2[r];
        if (have) x[u][r] = load8<kBf16>(p, r, vec * p.dv + e_first);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kV; ++u) {
    const long long vec = vec0 + u;
    if (vec >= p.vectors) break;
    // the max propagates NaN (a poisoned shard poisons the merged row, out
    // and LSE); -inf stays -inf (multiplier > 0)
    float mx = kNegInf;
    bool nan = false;
#pragma unroll
    for (int r = 0; r < kS; ++r) {
      if (r < S) {
        mx = fmaxf(mx, lse2[u][r]);
        nan |= lse2[u][r] != lse2[u][r];
      }
    }
    if (nan) mx = __builtin_nanf("");
    float w[kS];
    float wsum = 0.f;
#pragma unroll
    for (int r = 0; r < kS; ++r) {
      if (r < S) {
        w[r] = mx == kNegInf ? 0.f : __builtin_amdgcn_exp2f(lse2[u][r] - mx);
        wsum += w[r];
      }
    }
    const bool any = wsum > 0.f || wsum != wsum;
    const float inv = any ? 1.f / wsum : 0.f;

    for (int e0 = e_first; e0 < p.dv; e0 += 512) {
      if (e0 != e_first) {
#pragma unroll
        for (int r = 0; r < kS; ++r)
          if (r < S) x[u][r] = load8<kBf16>(p, r, vec * p.dv + e0);
      }
      f32x4_t a0 = f32x4_t{}, a1 = f32x4_t{};
#pragma unroll
      for (int r = 0; r < kS; ++r) {
        if (r < S && w[r] != 0.f) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            a0[k] += w[r] * elem<kBf16>(x[u][r], k);
            a1[k] += w[r] * elem<kBf16>(x[u][r], 4 + k);
          }
        }
      }
      a0 *= inv;
      a1 *= inv;
      if (p.out_bf16) {
        bf16x8_t y;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          y[k] = (__bf16)a0[k];
          y[4 + k] = (__bf16)a1[k];
        }
        store_stream((bf16x8_t*)((__bf16*)p.out + vec * p.dv + e0), y);
      } else {
        f32x4_t* y = (f32x4_t*)((float*)p.out + vec * p.dv + e0);
        store_stream(y, a0);
        store_stream(y + 1, a1);
      }
    }
    if (lane == 0 && p.lse_out != nullptr) {
      const float l2 = any ? mx + __builtin_amdgcn_logf(wsum) : kNegInf;
      p.lse_out[vec] = l2 * p.lse_out_from_log2;
    }
  }
}

__global__ __launch_bounds__(256) void metadata_kernel(const int32_t* seq_lens, const int32_t* block_table,
                                                       int32_t batch, int32_t max_pages, int32_t shard,
                                                       int32_t num_shards, int32_t* local_seq_lens,
                                                       int32_t* local_kv_indices, int32_t stride) {
  const long long total = local_kv_indices ? (long long)batch * stride : (long long)batch;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    const int b = local_kv_indices ? (int)(e / stride) : (int)e;
    const int j = local_kv_indices ? (int)(e % stride) : 0;
    int L = seq_lens[b];
    L = L < 0 ? 0 : L;
    const int n = L / num_shards + (shard < L % num_shards ? 1 : 0);
    if (j == 0) local_seq_lens[b] = n;
    if (local_kv_indices) {
      int v = -1;
      if (j < n) {
        const int t = j * num_shards + shard;
        const int pg = t >> 6;
        if (pg < max_pages) {
          const int page = block_table[(long long)b * max_pages + pg];
          v = page * kPage + (t & 63);
        }
      }
      local_kv_indices[e] = v;
    }
  }
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, hipEvent_t ev_begin, hipEvent_t ev_end, hipStream_t stream) {
  if (p.vectors == 0) return hipSuccess;
  // more than 8 shards: one vector per wave (registers)
  const int vpw = p.num_shards <= 8 ? kMergeVecsPerWave : 1;
  const long long blocks = (p.vectors + kMergeWaves * vpw - 1) / (kMergeWaves * vpw);
  const void* fn;
  if (p.in_bf16) {
    if (p.num_shards <= 1) fn = reinterpret_cast<const void*>(&merge_kernel<1, kMergeVecsPerWave, true>);
    else if (p.num_shards <= 2) fn = reinterpret_cast<const void*>(&merge_kernel<2, kMergeVecsPerWave, true>);
    else if (p.num_shards <= 4) fn = reinterpret_cast<const void*>(&merge_kernel<4, kMergeVecsPerWave, true>);
    else if (p.num_shards <= 8) fn = reinterpret_cast<const void*>(&merge_kernel<8, kMergeVecsPerWave, true>);
    else fn = reinterpret_cast<const void*>(&merge_kernel<16, 1, true>);
  } else {
    if (p.num_shards <= 1) fn = reinterpret_cast<const void*>(&merge_kernel<1, kMergeVecsPerWave, false>);
    else if (p.num_shards <= 2) fn = reinterpret_cast<const void*>(&merge_kernel<2, kMergeVecsPerWave, false>);
    else if (p.num_shards <= 4) fn = reinterpret_cast<const void*>(&merge_kernel<4, kMergeVecsPerWave, false>);
    else if (p.num_shards <= 8) fn = reinterpret_cast<const void*>(&merge_kernel<8, kMergeVecsPerWave, false>);
    else fn = reinterpret_cast<const void*>(&merge_kernel<16, 1, false>);
  }
  // the events, when given, take the kernel's own dispatch start and end
  void* args[] = {const_cast<MergeParams*>(&p)};
  return hipExtLaunchKernel(fn, dim3((unsigned)blocks), dim3(64 * kMergeWaves), args, 0, stream, ev_begin, ev_end, 0);
}

hipError_t launch_metadata(const int32_t* seq_lens, const int32_t* block_table, int32_t batch,
                           int32_t max_pages, int32_t shard, int32_t num_shards,
                           int32_t* local_seq_lens, int32_t* local_kv_indices, int32_t stride,
                           hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  const long long total = local_kv_indices ? (long long)batch * stride : (long long)batch;
  long long blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(metadata_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, seq_lens, block_table,
                     batch, max_pages, shard, num_shards, local_seq_lens, local_kv_indices, stride);
  return hipGetLastError();
}

}  // namespace mla
