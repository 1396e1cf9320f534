// KV append into the owning shard for gfx950.
//
// A decode step appends the newest token(s) of each request; under context
// sharding only the rank that owns a token, t mod S, holds its KV row
// (prhub.com.cn digest of sgl-project/sglang PR 33926, 关键源码片段: the
// layout test in which exactly one rank's local length grows per appended
// token, the rank (L - 1) mod S). The row goes through the pool's plain row
// write (实现拆解 step 4: the fused bf16 KV write is disabled under DCP), and
// fp8 pools store it quantised (实现拆解 step 3: the fp8 KV path). The same
// step prepares the query for an fp8 pool by one fused pass that puts its
// latent and rope dims side by side and quantises them (quantize_q_kernel),
// with the same rounding rule.
//
// One wave per appended token: 72 lanes' worth of 8-value chunks (64 latent
// + 8 rope) spread over the wave's 64 lanes, 16-byte loads, 16-byte (bf16)
// or 8-byte (fp8) stores. Bandwidth is trivial; the kernel exists so that
// the owner test, the page arithmetic and the quantisation run on device.
#include "mla_internal.h"

namespace mla {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kChunks = kDqk / 8;      // 72 chunks of 8 values per row
constexpr int kNopeChunks = 512 / 8;   // 64 of them from k_nope

// OCP e4m3 ("fn") code of a float32, from the format: 1 sign, 4 exponent
// (bias 7) and 3 mantissa bits, subnormals at exponent field 0, no
// infinities, S.1111.111 = NaN, largest finite 448. Round to nearest, ties
// to even; magnitudes above 448 (infinities too) saturate to 448.
// Every case is computed and the result selected (no branches: the lanes
// of a wave hold values of every kind).
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t mag = u & 0x7FFFFFFFu;
  // normal (>= 2^-6): keep 3 of the 23 mantissa bits, round the other 20 to
  // nearest even, then move the exponent bias from 127 to 7
  const uint32_t r = (mag + 0x7FFFFu + ((mag >> 20) & 1u)) >> 20;
  const uint32_t normal = min(r - (120u << 3), 0x7Eu);
  // subnormal: value k * 2^-9, k = |y| * 512 rounded to nearest even (k = 8
  // is the smallest normal, code 0x08)
  const uint32_t sub = (uint32_t)__builtin_rintf(__uint_as_float(mag) * 512.0f);
  uint32_t code = mag >= 0x3C800000u ? normal : sub;
  code = mag >= 0x43E00000u ? 0x7Eu : code;                // >= 448 (incl. inf)
  code = mag > 0x7F800000u ? 0x7Fu : code;                 // NaN
  return sign | code;
}

// e4m3 codes of eight bf16 values (one 16-byte chunk) divided by `scale`
// (finite, > 0): NaN keeps the input's sign; otherwise the fp32 quotient
// (IEEE division; finite or infinite) is rounded by e4m3_code.
__device__ __forceinline__ u32x2_t quantize8(const u32x4_t x, float scale) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t bits = (x[e >> 1] >> (16 * (e & 1))) << 16;   // bf16 -> f32, exact
    const uint32_t q = e4m3_code(__uint_as_float(bits) / scale);   // both cases computed, then selected
    const uint32_t code = (bits & 0x7FFFFFFFu) > 0x7F800000u ? (((bits >> 24) & 0x80u) | 0x7Fu) : q;
    w[e >> 2] |= code << (8 * (e & 3));
  }
  return u32x2_t{w[0], w[1]};
}

__global__ __launch_bounds__(64) void append_kernel(AppendParams p) {
  const int token = blockIdx.x;                 // b * n_new + i
  const int b = token / p.n_new, i = token - b * p.n_new;
  const int lane = threadIdx.x;
  const int L = p.seq_lens[b];
  const int t = L - p.n_new + i;
  if (t < 0 || t % p.num_shards != p.shard) return;
  const int pg = t >> 6;
  if (pg >= p.max_pages) return;
  const int page = p.block_table[(long long)b * p.max_pages + pg];
  if (page < 0 || page >= p.num_pages) return;
  const long long row = (long long)page * kPage + (t & 63);
  const uint16_t* nope = p.k_nope + (long long)token * 512;
  const uint16_t* rope = p.k_rope + (long long)token * 64;
  for (int c = lane; c < kChunks; c += 64) {
    const u32x4_t x = c < kNopeChunks ? *(const u32x4_t*)(nope + 8 * c)
                                      : *(const u32x4_t*)(rope + 8 * (c - kNopeChunks));
    if (!p.fp8) *(u32x4_t*)((uint16_t*)p.kv + row * kDqk + 8 * c) = x;
    else *(u32x2_t*)((uint8_t*)p.kv + row * kDqk + 8 * c) = quantize8(x, p.kv_scale);
  }
}

// Query concat-and-quantise: one thread per 8-value chunk of a row (64
// latent chunks from q, 8 rope chunks from q_rope), grid-stride.
__global__ __launch_bounds__(256) void quantize_q_kernel(QuantizeQParams p) {
  const long long total = p.rows * kChunks;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
    const long long n = i / kChunks;
    const int c = (int)(i - n * kChunks);
    const u32x4_t x = c < kNopeChunks ? *(const u32x4_t*)(p.q + n * p.q_stride + 8 * c)
                                      : *(const u32x4_t*)(p.q_rope + n * p.q_rope_stride + 8 * (c - kNopeChunks));
    *(u32x2_t*)(p.out + n * kDqk + 8 * c) = quantize8(x, p.q_scale);
  }
}

}  // namespace

hipError_t launch_quantize_q(const QuantizeQParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  const long long blocks = (p.rows * kChunks + 255) / 256;
  hipLaunchKernelGGL(quantize_q_kernel, dim3((unsigned)(blocks < 2048 ? blocks : 2048)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
  const long long tokens = (long long)p.batch * p.n_new;
  if (tokens == 0) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)tokens), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
