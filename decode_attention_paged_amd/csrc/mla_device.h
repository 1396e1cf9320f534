// Device-side helpers shared by the attention translation units.
#pragma once

#include "mla_internal.h"

namespace mla {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Global length of request b, clamped to what its block-table row can hold.
__device__ __forceinline__ int req_len(const DecodeParams& p, int b) {
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : L;
  const int cap = p.max_pages * kPage;
  return L > cap ? cap : L;
}

// Number of tokens of request b shard r owns (before any causal limit).
__device__ __forceinline__ int owned_count(const DecodeParams& p, int b, int r) {
  if (p.local_seq_lens != nullptr) {
    int n = p.local_seq_lens[b];
    n = n < 0 ? 0 : n;
    return n > p.local_kv_stride ? p.local_kv_stride : n;
  }
  const int L = req_len(p, b);
  return L / p.num_shards + (r < L % p.num_shards ? 1 : 0);
}

// Request, row block and shard of segment s of the schedule.
struct SegId {
  int b, rb, r, ri;   // ri: index of the shard among those of the launch
};
__device__ __forceinline__ SegId seg_id(const DecodeParams& p, int s) {
  SegId id;
  const int q = s / p.fold;
  id.ri = s - q * p.fold;
  id.b = q / p.row_blocks;
  id.rb = q - id.b * p.row_blocks;
  id.r = p.fold > 1 ? id.ri : p.shard;
  return id;
}

// Load through the constant address space: a wave-uniform address becomes a
// scalar load. Only for data no kernel of the same launch writes.
template <typename T>
__device__ __forceinline__ T ld_const(const T* ptr) {
  static_assert(sizeof(T) % 4 == 0, "whole dwords only");
  constexpr int kWords = sizeof(T) / 4;
  const __attribute__((address_space(4))) int32_t* q = (const __attribute__((address_space(4))) int32_t*)ptr;
  int32_t w[kWords];
#pragma unroll
  for (int i = 0; i < kWords; ++i) w[i] = q[i];
  T r;
  __builtin_memcpy(&r, w, sizeof(T));
  return r;
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(size_t)((__attribute__((address_space(3))) const void*)p);
}

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// (i & 3) of the 4-element rows that lanes 4r + (i >> 2) point at, r = 0..3.
__device__ __forceinline__ i16x4_t lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p);
}

// global_load_lds_dwordx4: each active lane's 16 bytes from `src` go to LDS
// at lds_base + 16 * lane. Issued as inline assembly so
// that the compiler's wait-count bookkeeping does not make later LDS reads of
// other buffers wait for them; every caller waits for completion explicitly
// (s_waitcnt vmcnt + barrier) before any wave reads the destination. M0 holds
// the LDS base (one wait state after writing it). kNT: the non-temporal
// (streaming) cache policy, for data that no other workgroup reads again.
template <bool kNT>
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_base) {
  if constexpr (kNT)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :: "v"(src), "s"(lds_base));
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"(lds_base));
}
// Same copy with a wave-uniform 64-bit base in SGPRs and a per-lane 32-bit
// byte offset.
template <bool kNT>
__device__ __forceinline__ void lds_dma16_sbase(const void* base, uint32_t offset, uint32_t lds_base) {
  if constexpr (kNT)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :: "v"(offset), "s"(base), "s"(lds_base));
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(offset), "s"(base), "s"(lds_base));
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt low bits [3:0] and high bits [15:14]; expcnt and lgkmcnt at maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// s_waitcnt lgkmcnt(0) alone (vmcnt and expcnt at maximum): every LDS and
// scalar-memory operation the wave issued has completed.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

}  // namespace mla
