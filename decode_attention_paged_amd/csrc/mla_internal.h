// Internal declarations shared by the HIP translation units of libmla_dcp.
// Not part of the C ABI (see include/mla_dcp.h for that).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

constexpr int kPage = 64;
constexpr int kDqk = 576;       // latent 512 + rope 64
constexpr int kDv = 512;        // V = first 512 latent dims
constexpr int kTile = 32;       // KV tokens per attention tile
// the schedule's cost of a piece (its query load and epilogue) in tiles: a
// bf16 tile's time is mostly its 36 KB read, an fp8 tile's mostly its
// MFMA work, so a piece weighs more bf16 tiles than fp8 ones (fits of
// per-workgroup times: ~3.2-3.7 and ~2.4; interleaved sweeps of the
// schedule: 5 and 3 best)
constexpr int kPieceCostBf16 = 5;
constexpr int kPieceCostFp8 = 3;
constexpr int kPieceCostMax = kPieceCostBf16 > kPieceCostFp8 ? kPieceCostBf16 : kPieceCostFp8;
constexpr int kMaxShards = 16;

// Everything the plan / attention / combine kernels need for one shard.
struct DecodeParams {
  const uint16_t* q;              // bf16 query rows, dims 0..511 (and 512..575 unless q_rope)
  const uint16_t* q_rope;         // bf16 rope dims 512..575 of every row (q + 512 when not split)
  int64_t q_stride, q_rope_stride;   // elements between consecutive query rows
  // the query as e4m3 codes [rows][576] (row n at byte n * q8_stride), or
  // null: the bf16 query above; only with e4m3 KV
  const uint8_t* q8;
  int64_t q8_stride;
  const uint8_t* kv;              // [num_pages][64][576] bf16 or e4m3
  const int32_t* block_table;     // [B][max_pages]
  const int32_t* seq_lens;        // [B] global lengths
  const int32_t* local_seq_lens;  // optional [B]
  const int32_t* local_kv_indices;// optional [B][stride]
  const int32_t* q_lens;          // optional [B] decode depth per request (<= q_len)
  int32_t local_kv_stride;
  int32_t batch, heads, q_len, rows, row_blocks;
  int32_t max_pages, num_pages, shard, num_shards;
  // shards this launch computes: 1 (shard `shard` alone), or num_shards when
  // every shard of the batch runs in one launch; then a segment is (request,
  // row block, shard), the shards of one row block are neighbours in the
  // schedule, every piece leaves a partial and the combine merges all pieces
  // of all shards into the full-context result
  int32_t fold;
  float scale_log2;               // softmax_scale * kv_scale (* q_scale) * log2(e)
  float out_scale;                // kv_scale (fp8) or 1
  int32_t lse_base2;              // write lse in base 2 (else natural)
  int32_t out_bf16;               // out dtype bf16 (else f32)
  void* out;
  float* lse;
  // workspace
  int32_t* plan;                  // [0] units, [1] workgroups in use
  // persistent schedule of the streaming kernel: the shard's work is the
  // sequence of units (request b, row block rb, shard, 32-token tile),
  // ordered by segment s = (b * row_blocks + rb) * fold + (shard index) and
  // tile; workgroup g takes a contiguous range of units of about equal cost
  // (tiles plus a charge per segment)
  int32_t* req_cnt;               // [B * fold] owned tokens per request and shard
  int32_t* seg_off;               // [B * row_blocks * fold + 1] first unit of each segment
  int32_t* seg_coff;              // [B * row_blocks * fold + 1] cost offset of each segment
  int32_t* wg_ustart;             // [grid + 1] first unit of each workgroup
  int4* seg_info;                 // [B * row_blocks * fold] (slot base, pieces, first workgroup, -)
  int2* wg_start;                 // [grid] (segment, tile) of each workgroup's first unit
  // [grid][kRecInts] start record of each workgroup: units, first segment and
  // tile, owned-token count of that request, then the KV rows of the tokens
  // of its first two tiles (-1: the zero row, -2: the NaN row)
  int32_t* wg_rec;
  uint16_t* spart_o;              // [slots][rows_blk][512] bf16, normalised, scaled
  float* spart_lse;               // [slots][rows_blk] base 2
  int32_t rows_blk;               // query rows per workgroup (64)
  int32_t kv_fp8;                 // KV pages hold e4m3 (else bf16)
  int32_t grid;                   // persistent workgroups
  // workgroups per row-block group: a request's row_blocks row blocks run on
  // that many neighbouring workgroups over the same tiles (1: plain schedule)
  int32_t rgroup;
  // [kMaxGrid] arrival counters of the row-block groups' rendezvous in the
  // launch of every shard (zeroed by the schedule and after every launch by
  // the piece combine)
  int32_t* grp_sync;
};

constexpr int kMaxGrid = 1024;  // persistent workgroups of the streaming kernel
constexpr int kRecInts = 8;     // start record of a workgroup: 6 ints used

// Query rows one workgroup covers: two row groups of 32 (a request with fewer
// rows leaves the rest empty: they compute on zero queries and are never
// stored); more rows take several row blocks, whose workgroups read the same
// KV tiles at about the same time (neighbours in the schedule), mostly from
// cache.
inline int32_t stream_rows_per_block(int32_t) { return 64; }

struct WorkspaceLayout {
  size_t plan, req_cnt, seg_off, seg_coff, seg_info, wg_start, wg_ustart, wg_rec, grp_sync, spart_lse, spart_o, total;
  int32_t max_slots;
};
// max_slots < 0: the bound every schedule fits (segments + the largest grid)
WorkspaceLayout decode_workspace_layout(int32_t batch, int32_t rows, int32_t max_slots = -1);

struct MergeParams {
  const void* outs[kMaxShards];
  const float* lses[kMaxShards];
  float lse_to_log2[kMaxShards];  // multiplier taking shard r's lse to base 2
  int32_t num_shards;
  int64_t vectors;                // rows * heads
  int32_t dv;
  int32_t in_bf16, out_bf16;
  void* out;
  float* lse_out;
  float lse_out_from_log2;        // multiplier from base 2 to the output base
};

struct AppendParams {
  const uint16_t* k_nope;         // [batch * n_new][512] bf16
  const uint16_t* k_rope;         // [batch * n_new][64] bf16
  const int32_t* seq_lens;
  const int32_t* block_table;
  void* kv;                       // [num_pages][64][576] bf16 | e4m3
  int32_t batch, n_new, max_pages, num_pages, shard, num_shards;
  int32_t fp8;
  float kv_scale;
};

struct QuantizeQParams {
  const uint16_t* q;              // bf16, dims 0..511 of row n at n * q_stride
  const uint16_t* q_rope;         // bf16, dims 512..575 of row n at n * q_rope_stride
  int64_t q_stride, q_rope_stride, rows;
  float q_scale;                  // divisor, finite and > 0
  uint8_t* out;                   // [rows][576] e4m3 codes
};

hipError_t launch_metadata(const int32_t* seq_lens, const int32_t* block_table, int32_t batch,
                           int32_t max_pages, int32_t shard, int32_t num_shards,
                           int32_t* local_seq_lens, int32_t* local_kv_indices,
                           int32_t stride, hipStream_t stream);
hipError_t launch_decode_plan(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_stream(const DecodeParams& p, bool run_plan, hipEvent_t ev_begin, hipEvent_t ev_end,
                                hipStream_t stream);
hipError_t launch_combine(const DecodeParams& p, hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, hipEvent_t ev_begin, hipEvent_t ev_end, hipStream_t stream);
hipError_t launch_append(const AppendParams& p, hipStream_t stream);
hipError_t launch_quantize_q(const QuantizeQParams& p, hipStream_t stream);

}  // namespace mla
