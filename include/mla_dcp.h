/*
 * mla_dcp.h -- C ABI of the MI355X (gfx950) paged MLA decode over a
 * context-sharded KV cache, with the LSE-weighted merge of shard partials.
 *
 * Pages cited (address and section heading as printed):
 *   [DCP decode] prhub.com.cn digest of sgl-project/sglang PR 33926 (the
 *                trtllm_mla decode path gains DCP support); sections
 *                "功能与动机" (motivation), "实现拆解" (implementation steps
 *                1-4) and "关键源码片段" (key code: the DCP metadata helpers).
 *   [symm_a2a]   github.com sgl-project/sglang PR 33364 "[Attention][DCP] Add
 *                symm_a2a: single-node symmetric-memory A2A backend for MLA
 *                decode"; sections Motivation and Modifications.
 *   [next_n]     prhub.com.cn digest of vllm-project/vllm PR 52164 (native
 *                next_n decode); section "功能与动机" (motivation).
 *
 * Conventions for every entry point:
 *   - Device pointers point to memory on the current HIP device; the caller
 *     owns every buffer (inputs, outputs and workspace). The library allocates
 *     no device memory and keeps no state besides cached device properties.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *     device work is enqueued asynchronously on it, with no host
 *     synchronisation, so a call can be captured into a HIP graph.
 *   - Failures return a status code; nothing unwinds across the ABI.
 *     mla_last_error() returns a message for the calling thread's last
 *     failure. Argument checks run before any device work, so an
 *     INVALID_ARGUMENT / UNSUPPORTED return enqueues nothing.
 *   - Geometry is MLA's: QK dim 576 (latent 512 + rope 64), V dim 512 = the
 *     first 512 latent dims, page size 64 tokens.
 *   - An empty shard or request is not an error: it yields (0, -inf).
 */
#ifndef MLA_DCP_H
#define MLA_DCP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 8
#define MLA_PAGE_SIZE 64
#define MLA_D_QK 576
#define MLA_D_V 512
#define MLA_MAX_SHARDS 16
#define MLA_MAX_Q_LEN 4
/* query heads per request: with q_len <= 4, a request's rows then fill at
 * most 1024 blocks of 64, the most workgroups a decode launch uses */
#define MLA_MAX_HEADS 16384

typedef enum mla_status {
  MLA_STATUS_OK = 0,
  MLA_STATUS_INVALID_ARGUMENT = 1,   /* null pointer, bad size, out-of-range id */
  MLA_STATUS_UNSUPPORTED = 2,        /* well-formed but not implemented      */
  MLA_STATUS_WORKSPACE_TOO_SMALL = 3,
  MLA_STATUS_DEVICE_ERROR = 4        /* a HIP call or launch failed          */
} mla_status_t;

typedef enum mla_dtype {
  MLA_DTYPE_F32 = 0,
  MLA_DTYPE_BF16 = 1,
  MLA_DTYPE_FP8_E4M3 = 2             /* OCP e4m3 ("fn"): bias 7, max 448, no inf */
} mla_dtype_t;

typedef enum mla_lse_base {
  MLA_LSE_BASE_E = 0,                /* natural log                          */
  MLA_LSE_BASE_2 = 1                 /* log2                                 */
} mla_lse_base_t;

/* ------------------------------------------------------------------------
 * Shard-local metadata.
 *
 * Follows [DCP decode] key code (the rank-local length, rank-local max and
 * page-table-on-the-cyclic-slice helpers) and motivation (token t of a
 * request belongs to shard t mod S). For shard r of S and each request b of
 * global length L_b = seq_lens[b]:
 *   local_seq_lens[b]      = L_b / S + (r < L_b % S)        (tokens it owns)
 *   local_kv_indices[b][j] = block_table[b][t / 64] * 64 + t % 64
 *                            with t = j * S + r, for j < local_seq_lens[b];
 *                            -1 for local_seq_lens[b] <= j < local_kv_stride
 *   *local_max_out         = max(M / S + (r < M % S), 1) with M = max_seq_len
 *                            (computed on the host, never 0).
 * Layout: seq_lens [batch] i32 (device); block_table [batch][max_pages] i32
 * (device, row-major); local_seq_lens [batch] i32 (device, written);
 * local_kv_indices [batch][local_kv_stride] i32 (device, written; may be
 * NULL to skip the index table); local_max_out (host, may be NULL).
 * Preconditions (not checked on device): seq_lens[b] <= max_seq_len and
 * seq_lens[b] <= max_pages * 64. local_kv_stride must be >= the local max.
 * Errors: INVALID_ARGUMENT for null required pointers, batch < 0,
 * num_shards < 1 or > MLA_MAX_SHARDS, shard_id outside [0, num_shards),
 * page_size != 64, max_pages < 1, max_seq_len < 0, local_kv_stride < local
 * max when local_kv_indices is given.
 * ---------------------------------------------------------------------- */
mla_status_t mla_build_shard_metadata(const int32_t* seq_lens, const int32_t* block_table,
                                      int32_t batch, int32_t max_pages, int32_t page_size,
                                      int32_t max_seq_len, int32_t shard_id, int32_t num_shards,
                                      int32_t* local_seq_lens, int32_t* local_kv_indices,
                                      int32_t local_kv_stride, int32_t* local_max_out,
                                      void* stream);

/* ------------------------------------------------------------------------
 * Rank-local partial decode.
 *
 * Follows [DCP decode] motivation and implementation step 3: each shard
 * attends over only the tokens it owns and returns its rank-local (out, lse);
 * a row whose shard owns no visible token is written as the neutral state
 * out = +0, lse = -inf. Implementation step 4 (first fix): kernels differ in
 * LSE base; the base written is returned so the merge site can rebase.
 * [next_n] motivation: q_len > 1 query rows of one request read each KV
 * tile once, not once per row.
 *
 * For request b (global KV length L = seq_lens[b], which includes the q_len
 * draft rows), query row i in [0, q_len) and head h:
 *   visible owned tokens O = { t < L : t mod S == r, t <= L - q_b + i }
 *   with q_b = q_len, or the request's own depth q_lens[b] when given (rows
 *   i >= q_b are padding: O is empty)
 *   s_t = softmax_scale * sum_{d<576} Q[b,i,h,d] * K_t[d]
 *   out[b,i,h,:] = sum_{t in O} exp(s_t) K_t[0:512] / sum_{t in O} exp(s_t)
 *   lse[b,i,h]   = log sum_{t in O} exp(s_t)   in `lse_base`
 * with K_t the latent row of token t (fp8 rows are multiplied by kv_scale).
 * ---------------------------------------------------------------------- */
typedef struct mla_decode_args {
  /* inputs (device) */
  const void* q;                 /* [batch][q_len][num_heads][576] bf16, or the
                                    512 latent dims only when q_rope is given   */
  const void* kv_pages;          /* [num_pages][64][576] bf16 or fp8 e4m3        */
  const int32_t* block_table;    /* [batch][max_pages] i32, page ids             */
  const int32_t* seq_lens;       /* [batch] i32, global KV length per request    */
  /* optional shard metadata from mla_build_shard_metadata (both or neither):
   * when given, KV rows are gathered through local_kv_indices instead of
   * being derived from block_table (the same rows; deriving them from the
   * block table reads one shared entry per 64 tokens instead of a private
   * one per token and measured 3-7% faster per launch on MI355X). */
  const int32_t* local_seq_lens;   /* [batch] i32 or NULL                        */
  const int32_t* local_kv_indices; /* [batch][local_kv_stride] i32 or NULL       */
  int32_t local_kv_stride;
  /* sizes */
  int32_t batch;
  int32_t num_heads;             /* multiple of 16 in [16, MLA_MAX_HEADS]         */
  int32_t q_len;                 /* 1 .. MLA_MAX_Q_LEN                            */
  int32_t max_pages;
  int32_t num_pages;             /* page ids outside [0, num_pages) read as NaN   */
  int32_t page_size;             /* must be 64                                    */
  int32_t shard_id;
  int32_t num_shards;
  mla_dtype_t kv_dtype;          /* BF16 or FP8_E4M3                              */
  float kv_scale;                /* per-tensor dequant scale (fp8); 1 for bf16    */
  float softmax_scale;
  mla_lse_base_t lse_base;       /* base requested for `lse`                      */
  /* outputs (device) */
  void* out;                     /* [batch][q_len][num_heads][512] f32 or bf16    */
  mla_dtype_t out_dtype;         /* F32 or BF16                                   */
  float* lse;                    /* [batch][q_len][num_heads] f32, required       */
  /* scratch (device), size from mla_decode_workspace_bytes */
  void* workspace;
  size_t workspace_bytes;
  /* tuning: number of persistent workgroups the shard's work is spread
   * over, 1 .. 1024 (0 = one per compute unit but one in 16, rounded down
   * to a multiple of 8) */
  int32_t split_target;
  /* optional hipEvent_t pair (created with timing) that receive the start
   * and end times of the attention kernel's dispatch (NULL = none) */
  void* event_begin;
  void* event_end;
  /* 0: build the work schedule in this call (a small kernel before the
   * attention kernel). 1: `workspace` already holds the schedule that
   * mla_decode_plan built for the same batch, num_heads, q_len, shard_id,
   * num_shards, max_pages, split_target, metadata pointers and the same
   * contents of seq_lens / local_seq_lens (the schedule depends on nothing
   * else), so one schedule serves every layer of a decode step. */
  int32_t reuse_plan;
  /* optional [batch] i32 (device) or NULL: the decode depth q_b of each
   * request when requests of one step differ ([next_n] implementation
   * step 3: the kernel receives the step's largest depth of query rows).
   * Rows i < q_b are real and see owned tokens t <= L - q_b + i; rows
   * q_b <= i < q_len are padding and are written as (0, -inf). Values are
   * clamped to [0, q_len]. NULL: every request is q_len deep. The work
   * schedule does not depend on it. */
  const int32_t* q_lens;
  /* optional split query ([DCP decode] 实现拆解 steps 3-4: the fused
   * concat-and-write of q_nope and q_pe into one query buffer is what the
   * DCP path turns off): when q_rope is not NULL, `q` holds the 512 latent
   * dims of every query row and q_rope its 64 rope dims, each read in place
   * with its own row stride, so no concatenation pass runs before the
   * decode. Query rows are ordered (b, i, h) as in the [batch][q_len]
   * [num_heads] layout; row n starts at element n * q_row_stride of `q` and
   * n * q_rope_row_stride of q_rope. q_row_stride = 0 means 576 (512 with
   * q_rope), q_rope_row_stride = 0 means 64. Strides must be multiples of 8
   * elements and both pointers 16-byte aligned (rows are read 16 bytes at a
   * time); e.g. two slices of one [rows][576] buffer are
   * (q, q + 512) with strides (576, 576). The query is never quantised: it
   * is read as bf16 for either KV dtype. */
  const void* q_rope;            /* [rows] x 64 bf16 at q_rope_row_stride, or NULL */
  int64_t q_row_stride;
  int64_t q_rope_row_stride;
  /* query as e4m3 codes ([DCP decode] 实现拆解 step 3: with an fp8 KV pool
   * the query is prepared by a fused concat-and-quantise, mla_quantize_q).
   * 0: `q` is the bf16 query above (exact, the default). > 0 and finite:
   * `q` holds [rows][576] e4m3 codes (row n at byte n * q_row_stride,
   * q_row_stride = 0 meaning 576, a multiple of 16), the query value being
   * code x q_scale; q_rope must be NULL and kv_dtype FP8_E4M3. The scores
   * then run on the fp8 matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4:
   * code x code, accumulated in fp32); P V stays bf16. Results match the
   * oracle's decode of the same codes; against the bf16 query they carry the
   * query's quantisation error (measured: 2e-2 in LSE, 5e-2 in out on the
   * 16-32K-token deepseek-like workload; several times that on contexts of a
   * few hundred tokens, where the softmax is sharper). */
  float q_scale;
} mla_decode_args_t;

/* Bytes of workspace mla_decode_partial needs for these sizes (host only,
 * no device call). Returns 0 for invalid sizes. */
size_t mla_decode_workspace_bytes(int32_t batch, int32_t num_heads, int32_t q_len);

/* Errors: INVALID_ARGUMENT for a null q / kv_pages / block_table / seq_lens /
 * out / lse / workspace, only one of the two metadata pointers, batch < 0,
 * a query stride that is negative, not a multiple of 8 or below the dims it
 * holds (576, or 512 with q_rope; 64 for q_rope), a query pointer that is
 * not 16-byte aligned,
 * num_heads not a multiple of 16 in [16, MLA_MAX_HEADS], q_len outside
 * [1, 4],
 * page_size != 64, bad shard ids, num_pages < 1, max_pages < 1,
 * split_target outside [0, 1024], a dtype other than those listed;
 * UNSUPPORTED when num_pages * 64 (rows of the pool) or max_pages * 64
 * (tokens a request can hold) exceeds 2^31 - 1, or when batch x 64-row
 * blocks x 32-token tiles a request can hold (per shard) reaches 2^31;
 * WORKSPACE_TOO_SMALL; DEVICE_ERROR if a launch
 * fails. `lse_base_written` (host, may be NULL) receives the base of `lse`,
 * which is always the requested one. */
mla_status_t mla_decode_partial(const mla_decode_args_t* args, mla_lse_base_t* lse_base_written,
                                void* stream);

/* Allocation-free variant of mla_decode_partial, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same decode and results, with the
 * work schedule and the piece partials in a scratch array the library holds
 * in device memory (80 MiB, one copy per device the library runs on, kept
 * until the process ends) instead of args->workspace, which is ignored (may
 * be NULL). The call allocates nothing and calls no allocating routine.
 * Limits: the schedule is rebuilt by every call (reuse_plan must be 0), and
 * the scratch holds the schedule of `batch` requests of num_heads * q_len
 * rows plus 2 x (workgroups) partial slots of (64 or 128 rows) x 512 bf16:
 * with the default workgroup count (split_target 0) that covers every
 * num_heads <= 128, q_len <= 4 and batch up to tens of thousands; larger
 * sizes or split_target return WORKSPACE_TOO_SMALL with the bytes needed.
 * Every call on a device shares that device's scratch: calls that overlap
 * in time on one device (different streams, or graph replays in flight
 * together) race and must be serialised by the caller. No part of the
 * scratch needs to start at zero; every call writes what it later reads.
 * Other arguments and errors as mla_decode_partial; DEVICE_ERROR if the
 * scratch's device address cannot be resolved. */
mla_status_t mla_decode_partial_noalloc(const mla_decode_args_t* args, mla_lse_base_t* lse_base_written,
                                        void* stream);

/* Builds the work schedule of a partial decode into args->workspace without
 * running the decode (same arguments and errors as mla_decode_partial; the
 * inputs are not read beyond seq_lens / local_seq_lens and the output
 * pointers not written). A later mla_decode_partial with reuse_plan = 1 and
 * the same workspace skips the schedule. Like the shard metadata it is built
 * once per decode step and serves every layer: the schedule is the
 * workgroups' shares of (request, row block, 32-token tile) units, balanced
 * by cost, with the pieces of requests cut at workgroup boundaries. */
mla_status_t mla_decode_plan(const mla_decode_args_t* args, void* stream);

/* ------------------------------------------------------------------------
 * Single-launch decode of every shard, merge fused.
 *
 * Runs all num_shards shards of the cyclic split in one schedule ([DCP
 * decode] 功能与动机 and 实现拆解 step 3: shard r attends over the tokens
 * t = j S + r it owns) and merges their partials with the LSE-weighted
 * reduction of [symm_a2a] Modifications (fourth kernel) inside the same
 * call: the shards of a row block are neighbours in the schedule and a
 * workgroup's online softmax runs on from one shard's tokens to the next
 * (the merge of two shards' states is exact arithmetic), and the pieces a
 * row block is cut into are combined in one pass, so no per-shard
 * (out, lse) is written or re-read. `out` / `lse`
 * receive the merged result, which is the full-context attention of every
 * query row (the per-shard formula above with O the union over r):
 *   out[b,i,h,:] = merge_r (out_r, lse_r),  lse[b,i,h] = log sum_r exp(lse_r)
 * and (0, -inf) for a row that sees no token (L = 0, or a padding row).
 * Arguments as mla_decode_partial, except: shard_id is ignored; shard
 * metadata (local_seq_lens / local_kv_indices) must be NULL (KV rows come
 * from block_table); the workspace size comes from
 * mla_decode_all_shards_workspace_bytes; reuse_plan = 1 reuses the schedule
 * a previous mla_decode_all_shards call (reuse_plan = 0) built in the same
 * workspace for the same batch, num_heads, q_len, num_shards, max_pages,
 * split_target and seq_lens contents; event_begin / event_end time the
 * attention kernel. Errors: those of mla_decode_partial, and
 * INVALID_ARGUMENT for shard metadata or batch x num_shards >= 2^31.
 * Nothing is allocated; every kernel of the call is safe to capture in a
 * HIP graph (no memset nodes). */
mla_status_t mla_decode_all_shards(const mla_decode_args_t* args, mla_lse_base_t* lse_base_written,
                                   void* stream);

/* Workspace bytes of mla_decode_all_shards (host only; 0 for invalid sizes). */
size_t mla_decode_all_shards_workspace_bytes(int32_t batch, int32_t num_heads, int32_t q_len,
                                             int32_t num_shards);

/* ------------------------------------------------------------------------
 * Cross-shard merge.
 *
 * Follows [symm_a2a] Modifications, fourth kernel (LSE-weighted softmax
 * reduction over all ranks' partial outputs; also the correction/combine
 * steps of the ag_rs and a2a backends under Motivation) and [DCP decode]'s
 * note that the LSE base is handled at the merge site. With lse_r rebased to
 * a common base, M = max_r lse_r and w_r = exp(lse_r - M):
 *   out = sum_r w_r out_r / sum_r w_r,  lse = M + log sum_r w_r.
 * Rows where every shard is neutral (lse_r = -inf) give out = 0, lse = -inf.
 * Layout: outs[r] -> [rows][num_heads][dv] (in_dtype), lses[r] -> [rows]
 * [num_heads] f32 in bases[r]; out -> [rows][num_heads][dv] (out_dtype);
 * lse_out -> [rows][num_heads] f32 in lse_out_base, or NULL.
 * `outs`, `lses` and `bases` are host arrays of num_shards entries.
 * Errors: INVALID_ARGUMENT for null arrays / pointers, num_shards outside
 * [1, MLA_MAX_SHARDS], rows < 0, num_heads < 1, dv not a positive multiple of
 * 8, dtypes other than F32 / BF16; DEVICE_ERROR if the launch fails.
 * ---------------------------------------------------------------------- */
typedef struct mla_merge_args {
  const void* const* outs;
  const float* const* lses;
  const mla_lse_base_t* bases;
  int32_t num_shards;
  int32_t rows;                  /* decode tokens (query rows)                  */
  int32_t num_heads;
  int32_t dv;
  mla_dtype_t in_dtype;
  void* out;
  mla_dtype_t out_dtype;
  float* lse_out;
  mla_lse_base_t lse_out_base;
  /* optional hipEvent_t pair (created with timing) that receive the start
   * and end times of the merge kernel's dispatch (NULL = none) */
  void* event_begin;
  void* event_end;
} mla_merge_args_t;

mla_status_t mla_merge_partials(const mla_merge_args_t* args, void* stream);

/* ------------------------------------------------------------------------
 * KV append into the owning shard.
 *
 * Follows [DCP decode] key code (the layout test: a decode step appends one
 * token per request, and exactly one rank's local length grows, the rank
 * (L - 1) mod S) and implementation steps 3-4 (under DCP the KV row is
 * written through the pool's plain row write, not the fused bf16 write; fp8
 * pools store the row quantised). For request b with new global length
 * L = seq_lens[b] and i in [0, n_new), token t = L - n_new + i is written
 * by shard t mod S only, into pool row
 *   block_table[b][t / 64] * 64 + t % 64
 * as the 576 values [k_nope[b][i][0:512] | k_rope[b][i][0:64]]:
 *   - kv_dtype BF16: the bf16 values as given;
 *   - kv_dtype FP8_E4M3: code = e4m3(x / kv_scale), the division in IEEE
 *     fp32 (x is the bf16 value widened exactly), then rounded to the
 *     nearest e4m3 value, ties to even; magnitudes above 448 (and
 *     infinities) saturate to +-448; NaN gives 0x7F with the input's sign.
 * Tokens with t < 0, t / 64 >= max_pages, or a page id outside
 * [0, num_pages) are skipped (nothing is written for them). Rows of other
 * shards' tokens are never written.
 * Layout: k_nope [batch][n_new][512] bf16, k_rope [batch][n_new][64] bf16
 * (device, contiguous); seq_lens [batch] i32 and block_table
 * [batch][max_pages] i32 (device); kv_pages [num_pages][64][576] of
 * kv_dtype (device, written in place).
 * Errors: INVALID_ARGUMENT for null pointers (batch > 0), batch < 0,
 * n_new outside [1, MLA_MAX_Q_LEN], num_shards outside [1, MLA_MAX_SHARDS],
 * shard_id outside [0, num_shards), max_pages < 1, num_pages < 1, a kv_dtype
 * other than BF16 / FP8_E4M3, kv_scale not finite and > 0 (fp8);
 * DEVICE_ERROR if the launch fails.
 * ---------------------------------------------------------------------- */
typedef struct mla_append_args {
  const uint16_t* k_nope;        /* [batch][n_new][512] bf16 bits */
  const uint16_t* k_rope;        /* [batch][n_new][64]  bf16 bits */
  const int32_t* seq_lens;       /* [batch] new global lengths    */
  const int32_t* block_table;    /* [batch][max_pages]            */
  void* kv_pages;                /* [num_pages][64][576]          */
  int32_t batch;
  int32_t n_new;
  int32_t max_pages;
  int32_t num_pages;
  int32_t shard_id;
  int32_t num_shards;
  mla_dtype_t kv_dtype;
  float kv_scale;
} mla_append_args_t;

mla_status_t mla_append_kv(const mla_append_args_t* args, void* stream);

/* ------------------------------------------------------------------------
 * Query concat-and-quantise ([DCP decode] 实现拆解 step 3: with an fp8 KV
 * pool the decode's query is prepared by one fused pass that puts the 512
 * latent dims and the 64 rope dims of each row side by side and quantises
 * them to fp8). Writes the e4m3 codes of `rows` query rows:
 * out[n][d] = nearest e4m3 value to the fp32 quotient q[n][d] / q_scale,
 * ties to the even code, magnitudes above 448 (and infinities) saturating
 * to +-448, NaN giving the NaN code with the input's sign (the rule of the
 * fp8 KV rows in mla_append_kv).
 * q: bf16 (device); row n's dims 0..511 at element n * q_row_stride, dims
 * 512..575 following them when q_rope is NULL, else at element
 * n * q_rope_row_stride of q_rope (bf16, device). Strides are in elements,
 * multiples of 8 (0 = 576, 512 with q_rope; 0 = 64 for q_rope); q and
 * q_rope 16-byte aligned. out: [rows][576] uint8 (device, contiguous,
 * 16-byte aligned; the `q` of an mla_decode_args_t with q_scale > 0).
 * Errors: INVALID_ARGUMENT for null q / out (rows > 0), rows < 0, a stride
 * or alignment outside the above, q_scale not finite and > 0;
 * DEVICE_ERROR if the launch fails.
 * ---------------------------------------------------------------------- */
mla_status_t mla_quantize_q(const void* q, const void* q_rope, int64_t q_row_stride, int64_t q_rope_row_stride,
                            int64_t rows, float q_scale, void* out, void* stream);

/* ------------------------------------------------------------------------
 * Introspection.
 * ---------------------------------------------------------------------- */
const char* mla_status_string(mla_status_t status);
const char* mla_last_error(void);
int32_t mla_abi_version(void);
/* sizeof the argument structs as compiled, for binding layout checks */
size_t mla_sizeof_decode_args(void);
size_t mla_sizeof_merge_args(void);
size_t mla_sizeof_append_args(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_DCP_H */
