// Host side of the C ABI declared in include/mla_dcp.h: argument checks,
// workspace layout, launch configuration and error reporting. Every check
// runs before any device work is enqueued.
#include "mla_dcp.h"
#include "mla_internal.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

namespace {

thread_local std::string g_last_error;

mla_status_t fail(mla_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

mla_status_t ok() {
  g_last_error.clear();
  return MLA_STATUS_OK;
}

mla_status_t device_fail(hipError_t err, const char* what) {
  return fail(MLA_STATUS_DEVICE_ERROR, "%s: %s", what, hipGetErrorString(err));
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Compute units of the current device, cached per device ordinal.
int device_cus(int* out) {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return -1;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    err = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess || n <= 0) return -1;
    cache[dev] = n;
  }
  *out = cache[dev];
  return 0;
}

// Scratch of the allocation-free decode (mla_decode_partial_noalloc): the
// work schedule and the piece partials live in this file-scope device array
// instead of a caller's workspace. Each device the library runs on holds its
// own copy until the process ends; host code reaches it only through the
// address hipGetSymbolAddress returns for the current device (the array's
// name is a host-side stand-in, not a device address).
constexpr size_t kScratchBytes = size_t(80) << 20;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

// Device address of `scratch` on the current device, looked up once per
// device (that device current) and cached; nullptr if the lookup fails.
void* scratch_address() {
  static std::mutex mu;
  static std::vector<void*> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, nullptr);
  if (cache[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    cache[dev] = ptr;
  }
  return cache[dev];
}

}  // namespace

namespace mla {

WorkspaceLayout decode_workspace_layout(int32_t batch, int32_t rows, int32_t max_slots) {
  WorkspaceLayout w{};
  const int32_t rows_blk = stream_rows_per_block(rows);
  const int64_t nseg = (int64_t)batch * ((rows + rows_blk - 1) / rows_blk);
  // a segment is cut into pieces only at workgroup boundaries
  w.max_slots = max_slots >= 0 ? max_slots : (int32_t)(nseg + kMaxGrid);
  size_t off = 0;
  w.plan = off;      off = align_up(off + 64, 256);
  w.req_cnt = off;   off = align_up(off + sizeof(int32_t) * (size_t)batch, 256);
  w.seg_off = off;   off = align_up(off + sizeof(int32_t) * (size_t)(nseg + 1), 256);
  w.seg_coff = off;  off = align_up(off + sizeof(int32_t) * (size_t)(nseg + 1), 256);
  w.seg_info = off;  off = align_up(off + sizeof(int4) * (size_t)nseg, 256);
  w.wg_start = off;  off = align_up(off + sizeof(int2) * (size_t)kMaxGrid, 256);
  w.wg_ustart = off; off = align_up(off + sizeof(int32_t) * (size_t)(kMaxGrid + 1), 256);
  w.wg_rec = off;    off = align_up(off + sizeof(int32_t) * (size_t)kMaxGrid * kRecInts, 256);
  w.grp_sync = off;  off = align_up(off + sizeof(int32_t) * (size_t)kMaxGrid, 256);
  w.spart_lse = off; off = align_up(off + sizeof(float) * (size_t)w.max_slots * rows_blk, 256);
  w.spart_o = off;   off = align_up(off + sizeof(uint16_t) * (size_t)w.max_slots * rows_blk * kDv, 256);
  w.total = off;
  return w;
}

}  // namespace mla

extern "C" {

const char* mla_status_string(mla_status_t status) {
  switch (status) {
    case MLA_STATUS_OK: return "ok";
    case MLA_STATUS_INVALID_ARGUMENT: return "invalid argument";
    case MLA_STATUS_UNSUPPORTED: return "unsupported";
    case MLA_STATUS_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MLA_STATUS_DEVICE_ERROR: return "device error";
  }
  return "unknown status";
}

const char* mla_last_error(void) { return g_last_error.c_str(); }
int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }
size_t mla_sizeof_decode_args(void) { return sizeof(mla_decode_args_t); }
size_t mla_sizeof_merge_args(void) { return sizeof(mla_merge_args_t); }
size_t mla_sizeof_append_args(void) { return sizeof(mla_append_args_t); }

mla_status_t mla_build_shard_metadata(const int32_t* seq_lens, const int32_t* block_table,
                                      int32_t batch, int32_t max_pages, int32_t page_size,
                                      int32_t max_seq_len, int32_t shard_id, int32_t num_shards,
                                      int32_t* local_seq_lens, int32_t* local_kv_indices,
                                      int32_t local_kv_stride, int32_t* local_max_out,
                                      void* stream) {
  if (batch < 0) return fail(MLA_STATUS_INVALID_ARGUMENT, "batch must be >= 0 (got %d)", batch);
  if (num_shards < 1 || num_shards > MLA_MAX_SHARDS)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "num_shards must be in [1, %d] (got %d)", MLA_MAX_SHARDS, num_shards);
  if (shard_id < 0 || shard_id >= num_shards)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "shard_id %d outside [0, %d)", shard_id, num_shards);
  if (page_size != MLA_PAGE_SIZE)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "page_size must be %d (got %d)", MLA_PAGE_SIZE, page_size);
  if (max_pages < 1) return fail(MLA_STATUS_INVALID_ARGUMENT, "max_pages must be >= 1 (got %d)", max_pages);
  if (max_seq_len < 0) return fail(MLA_STATUS_INVALID_ARGUMENT, "max_seq_len must be >= 0 (got %d)", max_seq_len);
  const int32_t lmax_raw = max_seq_len / num_shards + (shard_id < max_seq_len % num_shards ? 1 : 0);
  const int32_t lmax = lmax_raw > 1 ? lmax_raw : 1;
  if (batch > 0 && (seq_lens == nullptr || local_seq_lens == nullptr))
    return fail(MLA_STATUS_INVALID_ARGUMENT, "seq_lens and local_seq_lens are required");
  if (local_kv_indices != nullptr) {
    if (block_table == nullptr && batch > 0)
      return fail(MLA_STATUS_INVALID_ARGUMENT, "block_table is required with local_kv_indices");
    if (local_kv_stride < lmax)
      return fail(MLA_STATUS_INVALID_ARGUMENT, "local_kv_stride %d is below the local max %d", local_kv_stride, lmax);
  }
  if (local_max_out) *local_max_out = lmax;
  hipError_t err = mla::launch_metadata(seq_lens, block_table, batch, max_pages, shard_id, num_shards,
                                        local_seq_lens, local_kv_indices, local_kv_stride,
                                        (hipStream_t)stream);
  if (err != hipSuccess) return device_fail(err, "metadata launch");
  return ok();
}

mla_status_t mla_quantize_q(const void* q, const void* q_rope, int64_t q_row_stride, int64_t q_rope_row_stride,
                            int64_t rows, float q_scale, void* out, void* stream) {
  if (rows < 0) return fail(MLA_STATUS_INVALID_ARGUMENT, "rows must be >= 0 (got %lld)", (long long)rows);
  if (!(q_scale > 0.f) || !isfinite(q_scale))
    return fail(MLA_STATUS_INVALID_ARGUMENT, "q_scale must be finite and > 0");
  const bool split = q_rope != nullptr;
  const int64_t qs = q_row_stride == 0 ? (split ? 512 : MLA_D_QK) : q_row_stride;
  const int64_t rs = q_rope_row_stride == 0 ? 64 : q_rope_row_stride;
  if (qs < (split ? 512 : MLA_D_QK) || qs % 8 != 0)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "q_row_stride %lld must be a multiple of 8 and >= %d",
                (long long)q_row_stride, split ? 512 : MLA_D_QK);
  if (split && (rs < 64 || rs % 8 != 0))
    return fail(MLA_STATUS_INVALID_ARGUMENT, "q_rope_row_stride %lld must be a multiple of 8 and >= 64",
                (long long)q_rope_row_stride);
  if (rows > 0 && (q == nullptr || out == nullptr))
    return fail(MLA_STATUS_INVALID_ARGUMENT, "q and out are required");
  if (((uintptr_t)q & 15) != 0 || ((uintptr_t)q_rope & 15) != 0 || ((uintptr_t)out & 15) != 0)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "q, q_rope and out must be 16-byte aligned");
  if (rows == 0) return ok();
  mla::QuantizeQParams p;
  p.q = (const uint16_t*)q;
  p.q_rope = split ? (const uint16_t*)q_rope : p.q + 512;
  p.q_stride = qs;
  p.q_rope_stride = split ? rs : qs;
  p.rows = rows;
  p.q_scale = q_scale;
  p.out = (uint8_t*)out;
  hipError_t err = mla::launch_quantize_q(p, (hipStream_t)stream);
  if (err != hipSuccess) return fail(MLA_STATUS_DEVICE_ERROR, "quantize_q launch: %s", hipGetErrorString(err));
  return ok();
}

mla_status_t mla_append_kv(const mla_append_args_t* a, void* stream) {
  if (a == nullptr) return fail(MLA_STATUS_INVALID_ARGUMENT, "args is NULL");
  if (a->batch < 0) return fail(MLA_STATUS_INVALID_ARGUMENT, "batch must be >= 0 (got %d)", a->batch);
  if (a->n_new < 1 || a->n_new > MLA_MAX_Q_LEN)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "n_new must be in [1, %d] (got %d)", MLA_MAX_Q_LEN, a->n_new);
  if (a->num_shards < 1 || a->num_shards > MLA_MAX_SHARDS)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "num_shards must be in [1, %d] (got %d)", MLA_MAX_SHARDS, a->num_shards);
  if (a->shard_id < 0 || a->shard_id >= a->num_shards)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "shard_id %d outside [0, %d)", a->shard_id, a->num_shards);
  if (a->max_pages < 1) return fail(MLA_STATUS_INVALID_ARGUMENT, "max_pages must be >= 1 (got %d)", a->max_pages);
  if (a->num_pages < 1) return fail(MLA_STATUS_INVALID_ARGUMENT, "num_pages must be >= 1 (got %d)", a->num_pages);
  if (a->kv_dtype != MLA_DTYPE_BF16 && a->kv_dtype != MLA_DTYPE_FP8_E4M3)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "kv_dtype must be BF16 or FP8_E4M3");
  if (a->kv_dtype == MLA_DTYPE_FP8_E4M3 && !(a->kv_scale > 0.f && a->kv_scale <= 3.4028235e38f))
    return fail(MLA_STATUS_INVALID_ARGUMENT, "kv_scale must be finite and > 0 for an fp8 pool");
  if (a->batch > 0 && (a->k_nope == nullptr || a->k_rope == nullptr || a->seq_lens == nullptr ||
                       a->block_table == nullptr || a->kv_pages == nullptr))
    return fail(MLA_STATUS_INVALID_ARGUMENT, "k_nope, k_rope, seq_lens, block_table and kv_pages are required");
  mla::AppendParams p;
  p.k_nope = a->k_nope;
  p.k_rope = a->k_rope;
  p.seq_lens = a->seq_lens;
  p.block_table = a->block_table;
  p.kv = a->kv_pages;
  p.batch = a->batch;
  p.n_new = a->n_new;
  p.max_pages = a->max_pages;
  p.num_pages = a->num_pages;
  p.shard = a->shard_id;
  p.num_shards = a->num_shards;
  p.fp8 = a->kv_dtype == MLA_DTYPE_FP8_E4M3;
  p.kv_scale = a->kv_scale;
  hipError_t err = mla::launch_append(p, (hipStream_t)stream);
  if (err != hipSuccess) return device_fail(err, "append launch");
  return ok();
}

size_t mla_decode_workspace_bytes(int32_t batch, int32_t num_heads, int32_t q_len) {
  if (batch < 0 || num_heads < 16 || num_heads > MLA_MAX_HEADS || num_heads % 16 != 0 || q_len < 1 ||
      q_len > MLA_MAX_Q_LEN)
    return 0;
  return mla::decode_workspace_layout(batch, num_heads * q_len).total;
}

size_t mla_decode_all_shards_workspace_bytes(int32_t batch, int32_t num_heads, int32_t q_len, int32_t num_shards) {
  if (num_shards < 1 || num_shards > MLA_MAX_SHARDS) return 0;
  if ((int64_t)batch * num_shards > 0x7FFFFFFFLL) return 0;
  return mla_decode_workspace_bytes(batch * num_shards, num_heads, q_len);
}

}  // extern "C"

// Validates the arguments and fills the kernels' parameters; `launch` is
// false when there is nothing to run (batch 0). `all_shards`: one launch for
// every shard (shard_id ignored, no shard metadata, merged output).
static mla_status_t prepare_decode(const mla_decode_args_t* a, mla::DecodeParams& p, bool& launch,
                                   bool all_shards = false, bool noalloc = false) {
  launch = false;
  if (a == nullptr) return fail(MLA_STATUS_INVALID_ARGUMENT, "args is NULL");
  if (a->batch < 0) return fail(MLA_STATUS_INVALID_ARGUMENT, "batch must be >= 0 (got %d)", a->batch);
  if (a->num_heads < 16 || a->num_heads > MLA_MAX_HEADS || a->num_heads % 16 != 0)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "num_heads must be a multiple of 16 in [16, %d] (got %d)", MLA_MAX_HEADS,
                a->num_heads);
  if (a->q_len < 1 || a->q_len > MLA_MAX_Q_LEN)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "q_len must be in [1, %d] (got %d)", MLA_MAX_Q_LEN, a->q_len);
  if (a->page_size != MLA_PAGE_SIZE)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "page_size must be %d (got %d)", MLA_PAGE_SIZE, a->page_size);
  if (a->num_shards < 1 || a->num_shards > MLA_MAX_SHARDS)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "num_shards must be in [1, %d] (got %d)", MLA_MAX_SHARDS, a->num_shards);
  if (!all_shards && (a->shard_id < 0 || a->shard_id >= a->num_shards))
    return fail(MLA_STATUS_INVALID_ARGUMENT, "shard_id %d outside [0, %d)", a->shard_id, a->num_shards);
  if (a->max_pages < 1) return fail(MLA_STATUS_INVALID_ARGUMENT, "max_pages must be >= 1 (got %d)", a->max_pages);
  if (a->num_pages < 1) return fail(MLA_STATUS_INVALID_ARGUMENT, "num_pages must be >= 1 (got %d)", a->num_pages);
  if ((long long)a->num_pages * MLA_PAGE_SIZE > 0x7FFFFFFFLL)
    return fail(MLA_STATUS_UNSUPPORTED, "num_pages %d exceeds 2^31 KV rows", a->num_pages);
  if ((long long)a->max_pages * MLA_PAGE_SIZE > 0x7FFFFFFFLL)
    return fail(MLA_STATUS_UNSUPPORTED, "max_pages %d exceeds 2^31 tokens per request", a->max_pages);
  if (a->kv_dtype != MLA_DTYPE_BF16 && a->kv_dtype != MLA_DTYPE_FP8_E4M3)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "kv_dtype must be BF16 or FP8_E4M3");
  if (a->out_dtype != MLA_DTYPE_F32 && a->out_dtype != MLA_DTYPE_BF16)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "out_dtype must be F32 or BF16");
  if (a->lse_base != MLA_LSE_BASE_E && a->lse_base != MLA_LSE_BASE_2)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "lse_base must be E or 2");
  if (!(a->softmax_scale > 0.f) || !isfinite(a->softmax_scale))
    return fail(MLA_STATUS_INVALID_ARGUMENT, "softmax_scale must be positive and finite");
  if (!(a->kv_scale > 0.f) || !isfinite(a->kv_scale))
    return fail(MLA_STATUS_INVALID_ARGUMENT, "kv_scale must be positive and finite");
  if ((a->local_seq_lens == nullptr) != (a->local_kv_indices == nullptr))
    return fail(MLA_STATUS_INVALID_ARGUMENT, "local_seq_lens and local_kv_indices go together");
  if (all_shards && a->local_seq_lens != nullptr)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "the all-shards decode reads the global block table: no shard metadata");
  if (a->local_kv_indices != nullptr && a->local_kv_stride < 1)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "local_kv_stride must be >= 1 (got %d)", a->local_kv_stride);
  if (a->reuse_plan != 0 && a->reuse_plan != 1)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "reuse_plan must be 0 or 1 (got %d)", a->reuse_plan);
  if (a->split_target < 0 || a->split_target > mla::kMaxGrid)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "split_target must be in [0, %d] (got %d)", mla::kMaxGrid, a->split_target);
  if (noalloc && a->reuse_plan != 0)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "the allocation-free decode rebuilds its schedule in every call: reuse_plan must be 0");
  if (a->batch > 0) {
    if (!a->q || !a->kv_pages || !a->block_table || !a->seq_lens || !a->out || !a->lse || (!a->workspace && !noalloc))
      return fail(MLA_STATUS_INVALID_ARGUMENT, "q, kv_pages, block_table, seq_lens, out, lse and workspace are required");
  }
  if (!(a->q_scale >= 0.f) || !isfinite(a->q_scale))
    return fail(MLA_STATUS_INVALID_ARGUMENT, "q_scale must be 0 (bf16 query) or finite and > 0 (e4m3 query codes)");
  const bool q8 = a->q_scale > 0.f;
  if (q8) {
    if (a->kv_dtype != MLA_DTYPE_FP8_E4M3)
      return fail(MLA_STATUS_INVALID_ARGUMENT, "an e4m3 query (q_scale > 0) needs an FP8_E4M3 KV pool");
    if (a->q_rope != nullptr)
      return fail(MLA_STATUS_INVALID_ARGUMENT, "an e4m3 query holds all 576 dims of a row: q_rope must be NULL");
    const int64_t qs = a->q_row_stride == 0 ? MLA_D_QK : a->q_row_stride;
    if (qs < MLA_D_QK || qs % 16 != 0)
      return fail(MLA_STATUS_INVALID_ARGUMENT, "q_row_stride %lld of the e4m3 query must be a multiple of 16 and >= %d",
                  (long long)a->q_row_stride, MLA_D_QK);
    if (((uintptr_t)a->q & 15) != 0) return fail(MLA_STATUS_INVALID_ARGUMENT, "q must be 16-byte aligned");
  } else {
    const bool split = a->q_rope != nullptr;
    const int64_t qs = a->q_row_stride == 0 ? (split ? 512 : MLA_D_QK) : a->q_row_stride;
    const int64_t rs = a->q_rope_row_stride == 0 ? 64 : a->q_rope_row_stride;
    if (qs < (split ? 512 : MLA_D_QK) || qs % 8 != 0)
      return fail(MLA_STATUS_INVALID_ARGUMENT, "q_row_stride %lld must be a multiple of 8 and >= %d",
                  (long long)a->q_row_stride, split ? 512 : MLA_D_QK);
    if (split && (rs < 64 || rs % 8 != 0))
      return fail(MLA_STATUS_INVALID_ARGUMENT, "q_rope_row_stride %lld must be a multiple of 8 and >= 64",
                  (long long)a->q_rope_row_stride);
    if (((uintptr_t)a->q & 15) != 0 || ((uintptr_t)a->q_rope & 15) != 0)
      return fail(MLA_STATUS_INVALID_ARGUMENT, "q and q_rope must be 16-byte aligned");
  }
  const int32_t rows = a->num_heads * a->q_len;
  const int32_t fold = all_shards ? a->num_shards : 1;
  if ((int64_t)a->batch * fold > 0x7FFFFFFFLL)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "batch %d x %d shards is too large", a->batch, fold);
  {
    // the schedule counts tiles and their costs in 32-bit integers: bound
    // them from the sizes alone (every request as long as its block-table
    // row allows)
    const int64_t rb = (rows + mla::stream_rows_per_block(rows) - 1) / mla::stream_rows_per_block(rows);
    const int64_t local_tokens = ((int64_t)a->max_pages * MLA_PAGE_SIZE + a->num_shards - 1) / a->num_shards;
    const int64_t tiles = (local_tokens + mla::kTile - 1) / mla::kTile;
    const int64_t segs = (int64_t)a->batch * fold * rb;
    if (segs * (tiles + mla::kPieceCostMax) > 0x7FFFFFFFLL)
      return fail(MLA_STATUS_UNSUPPORTED,
                  "batch %d x %lld row blocks x %lld tiles per request (max_pages %d) exceeds the schedule's 2^31 "
                  "tiles; split the batch", a->batch, (long long)(fold * rb), (long long)tiles, a->max_pages);
  }
  mla::WorkspaceLayout w = mla::decode_workspace_layout(a->batch * fold, rows);
  if (!noalloc && a->batch > 0 && a->workspace_bytes < w.total)
    return fail(MLA_STATUS_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes (got %zu)", w.total, a->workspace_bytes);
  if (a->batch == 0) return ok();

  int cus = 0;
  if (device_cus(&cus) != 0) return fail(MLA_STATUS_DEVICE_ERROR, "cannot query the current device");
  int32_t grid;
  const int32_t rows_blk = mla::stream_rows_per_block(rows);
  const int32_t row_blocks = (rows + rows_blk - 1) / rows_blk;
  // a request of several row blocks runs them on a group of that many
  // neighbouring workgroups walking the same tiles, so that each tile is
  // fetched from HBM once for all its row blocks
  const int32_t rgroup = row_blocks;
  {
    // one persistent workgroup per CU but one in 16 (a multiple of 8 so that
    // the workgroup order can follow the XCDs) unless the caller fixes the
    // count: the free CUs run the small kernels of concurrent shards (their
    // combine) alongside, which shortens a step of concurrent partials of
    // one-row-block requests. Requests of several row blocks (row-block
    // groups, every XCD holding whole groups) and the single launch of every
    // shard (nothing runs beside it) take every CU the group size fits:
    // there the extra workgroups gain more than free CUs would (deepseek-like
    // fp8 step 0.424 -> 0.403 ms, q_len 4 0.438 -> 0.390, skewed 0.645 ->
    // 0.628; kimi-like single launch 96.4 -> 94.1 µs).
    const bool all_cus = rgroup > 1 || (all_shards && a->num_shards > 1);
    if (a->split_target > 0) {
      grid = a->split_target;
    } else {
      const int32_t per_xcd = cus / 8;
      const int32_t slots = all_cus ? (per_xcd / rgroup) * rgroup : per_xcd - per_xcd / 16;
      grid = 8 * (slots > 0 ? slots : 1);
    }
    if (a->split_target <= 0) {
      // a small step has less work than CUs: the schedule uses at most one
      // group per cost unit, and the cost (tiles + the piece cost of each
      // super-segment) is bounded from the batch, the row blocks, the shards
      // and the block table's width (no request reads past max_pages x 64
      // tokens), so only that many workgroups are launched and the rest are
      // not dispatched just to exit
      const int64_t local_tokens = ((int64_t)a->max_pages * MLA_PAGE_SIZE + a->num_shards - 1) / a->num_shards;
      const int64_t tiles = (local_tokens + mla::kTile - 1) / mla::kTile;
      const int64_t supers = (int64_t)a->batch * fold * (rgroup == 1 ? row_blocks : 1);
      const int64_t need = supers * (tiles + mla::kPieceCostMax) * rgroup;
      if (need < grid) grid = (int32_t)((need + 7) / 8 * 8);
    }
    if (grid < 8) grid = 8;
    if (grid > mla::kMaxGrid) grid = mla::kMaxGrid;
    grid = (grid / rgroup) * rgroup;
    if (grid < rgroup) grid = rgroup;
  }
  uint8_t* ws = (uint8_t*)a->workspace;
  if (noalloc) {
    // only segments cut at a workgroup boundary take partial slots, one per
    // piece: at most two per boundary, so 2 x grid slots always suffice
    w = mla::decode_workspace_layout(a->batch, rows, 2 * grid);
    if (w.total > kScratchBytes)
      return fail(MLA_STATUS_WORKSPACE_TOO_SMALL,
                  "batch %d x %d rows with %d workgroups needs %zu bytes of scratch; the allocation-free decode "
                  "holds %zu", a->batch, rows, grid, w.total, kScratchBytes);
    ws = (uint8_t*)scratch_address();
    if (ws == nullptr) return fail(MLA_STATUS_DEVICE_ERROR, "cannot resolve the scratch address on the current device");
  }
  p = mla::DecodeParams{};
  p.q = (const uint16_t*)a->q;
  if (q8) {
    p.q8 = (const uint8_t*)a->q;
    p.q8_stride = a->q_row_stride == 0 ? MLA_D_QK : a->q_row_stride;
    p.q_rope = p.q;
  } else if (a->q_rope != nullptr) {
    p.q_rope = (const uint16_t*)a->q_rope;
    p.q_stride = a->q_row_stride == 0 ? 512 : a->q_row_stride;
    p.q_rope_stride = a->q_rope_row_stride == 0 ? 64 : a->q_rope_row_stride;
  } else {
    p.q_rope = p.q + 512;
    p.q_stride = a->q_row_stride == 0 ? MLA_D_QK : a->q_row_stride;
    p.q_rope_stride = p.q_stride;
  }
  p.kv = (const uint8_t*)a->kv_pages;
  p.block_table = a->block_table;
  p.seq_lens = a->seq_lens;
  p.local_seq_lens = a->local_seq_lens;
  p.local_kv_indices = a->local_kv_indices;
  p.local_kv_stride = a->local_kv_stride;
  p.q_lens = a->q_lens;
  p.batch = a->batch;
  p.heads = a->num_heads;
  p.q_len = a->q_len;
  p.rows = rows;
  p.max_pages = a->max_pages;
  p.num_pages = a->num_pages;
  p.shard = all_shards ? 0 : a->shard_id;
  p.num_shards = a->num_shards;
  p.fold = fold;
  const float kv_scale = a->kv_dtype == MLA_DTYPE_FP8_E4M3 ? a->kv_scale : 1.f;
  p.scale_log2 = (float)((double)a->softmax_scale * (double)kv_scale * (q8 ? (double)a->q_scale : 1.0) *
                         1.4426950408889634);
  p.out_scale = kv_scale;
  p.lse_base2 = a->lse_base == MLA_LSE_BASE_2;
  p.out_bf16 = a->out_dtype == MLA_DTYPE_BF16;
  p.out = a->out;
  p.lse = a->lse;
  p.plan = (int32_t*)(ws + w.plan);
  p.req_cnt = (int32_t*)(ws + w.req_cnt);
  p.seg_off = (int32_t*)(ws + w.seg_off);
  p.seg_coff = (int32_t*)(ws + w.seg_coff);
  p.wg_ustart = (int32_t*)(ws + w.wg_ustart);
  p.seg_info = (int4*)(ws + w.seg_info);
  p.wg_start = (int2*)(ws + w.wg_start);
  p.wg_rec = (int32_t*)(ws + w.wg_rec);
  p.grp_sync = (int32_t*)(ws + w.grp_sync);
  p.spart_lse = (float*)(ws + w.spart_lse);
  p.spart_o = (uint16_t*)(ws + w.spart_o);
  p.rows_blk = rows_blk;
  p.row_blocks = row_blocks;
  p.rgroup = rgroup;
  p.kv_fp8 = a->kv_dtype == MLA_DTYPE_FP8_E4M3;
  p.grid = grid;
  launch = true;
  return ok();
}

extern "C" {

mla_status_t mla_decode_partial(const mla_decode_args_t* a, mla_lse_base_t* lse_base_written, void* stream) {
  mla::DecodeParams p;
  bool launch = false;
  const mla_status_t st = prepare_decode(a, p, launch);
  if (st != MLA_STATUS_OK) return st;
  if (lse_base_written) *lse_base_written = a->lse_base;
  if (!launch) return ok();
  hipError_t err = mla::launch_decode_stream(p, a->reuse_plan == 0, (hipEvent_t)a->event_begin,
                                             (hipEvent_t)a->event_end, (hipStream_t)stream);
  if (err != hipSuccess) return device_fail(err, "decode launch");
  return ok();
}

mla_status_t mla_decode_all_shards(const mla_decode_args_t* a, mla_lse_base_t* lse_base_written, void* stream) {
  mla::DecodeParams p;
  bool launch = false;
  const mla_status_t st = prepare_decode(a, p, launch, true);
  if (st != MLA_STATUS_OK) return st;
  if (lse_base_written) *lse_base_written = a->lse_base;
  if (!launch) return ok();
  hipError_t err = mla::launch_decode_stream(p, a->reuse_plan == 0, (hipEvent_t)a->event_begin,
                                             (hipEvent_t)a->event_end, (hipStream_t)stream);
  if (err != hipSuccess) return device_fail(err, "decode launch");
  return ok();
}

mla_status_t mla_decode_partial_noalloc(const mla_decode_args_t* a, mla_lse_base_t* lse_base_written,
                                        void* stream) {
  mla::DecodeParams p;
  bool launch = false;
  const mla_status_t st = prepare_decode(a, p, launch, false, true);
  if (st != MLA_STATUS_OK) return st;
  if (lse_base_written) *lse_base_written = a->lse_base;
  if (!launch) return ok();
  hipError_t err = mla::launch_decode_stream(p, true, (hipEvent_t)a->event_begin, (hipEvent_t)a->event_end,
                                             (hipStream_t)stream);
  if (err != hipSuccess) return device_fail(err, "decode launch");
  return ok();
}

mla_status_t mla_decode_plan(const mla_decode_args_t* a, void* stream) {
  mla::DecodeParams p;
  bool launch = false;
  const mla_status_t st = prepare_decode(a, p, launch);
  if (st != MLA_STATUS_OK || !launch) return st;
  hipError_t err = mla::launch_decode_plan(p, (hipStream_t)stream);
  if (err != hipSuccess) return device_fail(err, "plan launch");
  return ok();
}

mla_status_t mla_merge_partials(const mla_merge_args_t* a, void* stream) {
  if (a == nullptr) return fail(MLA_STATUS_INVALID_ARGUMENT, "args is NULL");
  if (a->num_shards < 1 || a->num_shards > MLA_MAX_SHARDS)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "num_shards must be in [1, %d] (got %d)", MLA_MAX_SHARDS, a->num_shards);
  if (a->rows < 0) return fail(MLA_STATUS_INVALID_ARGUMENT, "rows must be >= 0 (got %d)", a->rows);
  if (a->num_heads < 1) return fail(MLA_STATUS_INVALID_ARGUMENT, "num_heads must be >= 1 (got %d)", a->num_heads);
  if (a->dv < 8 || a->dv % 8 != 0) return fail(MLA_STATUS_INVALID_ARGUMENT, "dv must be a positive multiple of 8 (got %d)", a->dv);
  if (a->in_dtype != MLA_DTYPE_F32 && a->in_dtype != MLA_DTYPE_BF16)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "in_dtype must be F32 or BF16");
  if (a->out_dtype != MLA_DTYPE_F32 && a->out_dtype != MLA_DTYPE_BF16)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "out_dtype must be F32 or BF16");
  if (a->lse_out_base != MLA_LSE_BASE_E && a->lse_out_base != MLA_LSE_BASE_2)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "lse_out_base must be E or 2");
  if (a->outs == nullptr || a->lses == nullptr || a->bases == nullptr)
    return fail(MLA_STATUS_INVALID_ARGUMENT, "outs, lses and bases arrays are required");
  mla::MergeParams p{};
  p.num_shards = a->num_shards;
  for (int r = 0; r < a->num_shards; ++r) {
    if (a->rows > 0 && (a->outs[r] == nullptr || a->lses[r] == nullptr))
      return fail(MLA_STATUS_INVALID_ARGUMENT, "shard %d has a NULL out or lse pointer", r);
    if (a->bases[r] != MLA_LSE_BASE_E && a->bases[r] != MLA_LSE_BASE_2)
      return fail(MLA_STATUS_INVALID_ARGUMENT, "shard %d has an invalid LSE base", r);
    p.outs[r] = a->outs[r];
    p.lses[r] = a->lses[r];
    p.lse_to_log2[r] = a->bases[r] == MLA_LSE_BASE_E ? 1.4426950408889634f : 1.f;
  }
  if (a->rows > 0 && a->out == nullptr) return fail(MLA_STATUS_INVALID_ARGUMENT, "out is required");
  p.vectors = (int64_t)a->rows * a->num_heads;
  p.dv = a->dv;
  p.in_bf16 = a->in_dtype == MLA_DTYPE_BF16;
  p.out_bf16 = a->out_dtype == MLA_DTYPE_BF16;
  p.out = a->out;
  p.lse_out = a->lse_out;
  p.lse_out_from_log2 = a->lse_out_base == MLA_LSE_BASE_E ? 0.69314718055994531f : 1.f;
  hipError_t err = mla::launch_merge(p, (hipEvent_t)a->event_begin, (hipEvent_t)a->event_end, (hipStream_t)stream);
  if (err != hipSuccess) return device_fail(err, "merge launch");
  return ok();
}

}  // extern "C"
