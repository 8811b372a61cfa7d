/*
 * sda.h - DSA sparse decode attention over a paged KV cache, for MI355X
 * (gfx950).  C ABI of libsda.so.
 *
 * The operation is the one the page "vllm.models.step5.nvidia.ops.
 * sparse_decode_attention" documents: in its module docstring, in the
 * `sparse_decode_attention` section (arguments, shapes and asserts) and in the
 * `sparse_decode_splits` section (split heuristic).  Each row is one
 * (token, KV group) pair.  It holds up to 16 GQA-packed query heads of dim 192,
 * and it attends only over its selected regions, which are read in place from
 * the paged cache.  The shape and stride eligibility rules follow
 * `_direct_sparse_decode` on the page "vllm.models.step5.nvidia.
 * flashinfer_sparse".
 *
 * All pointers in sda_decode_args are DEVICE pointers unless noted.  The
 * caller owns every buffer, including the workspace.  The library allocates
 * nothing; its only state is a per-device cache of the compute-unit count
 * (read once, thread-safe) and, for sda_decode_static alone, a static device
 * scratch array.  Every other entry point is re-entrant; calls that may
 * overlap (other streams, other threads) need workspaces of their own, since
 * each call rewrites its workspace.  sda_decode
 * validates on the host and never reads device memory there; index contents
 * (region ids, block-table entries, positions) are trusted, as on the page.
 * On any error it returns before launching anything.
 */
#ifndef SDA_H_
#define SDA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDA_ABI_VERSION 8
#define SDA_HEAD_DIM 192     /* query / key / value head dim (fixed) */
#define SDA_KV_ROW 384       /* one cache token row: K[0:192] then V[192:384] */
#define SDA_MAX_HEADS 16     /* GQA-packed query heads per KV group */
#define SDA_MAX_R 2048       /* region slots per row */
#define SDA_MAX_SPLITS 256
#define SDA_MAX_ROWS 16777215 /* rows per call: grid limit (rows * 256 threads < 2^32) */

typedef enum {
  SDA_OK = 0,
  SDA_ERR_INVALID = -1,      /* an argument breaks the operation's contract */
  SDA_ERR_UNSUPPORTED = -2,  /* legal, but outside what the library handles */
  SDA_ERR_WORKSPACE = -3,    /* workspace missing (splits > 1), too small or misaligned */
  SDA_ERR_LAUNCH = -4,       /* the HIP launch reported an error */
  SDA_ERR_SCRATCH = -5       /* sda_decode_static: the call needs more than the
                                library's static scratch (SDA_STATIC_SCRATCH_BYTES) */
} sda_status;

typedef enum {
  SDA_KV_BF16 = 0,           /* cache elements are bfloat16 */
  SDA_KV_FP8_E4M3 = 1        /* cache elements are OCP float8 e4m3fn bytes */
} sda_kv_dtype;

/*
 * Arguments of one decode call.  Field meanings follow `sparse_decode_attention`
 * (page "...ops.sparse_decode_attention").  Strides are in ELEMENTS of the
 * pointed-to type.
 *
 *  rows         number of (token, KV group) rows; rows = tokens * groups,
 *               at most SDA_MAX_ROWS.
 *               Row r is group r % groups of token r / groups.  The
 *               groups*query_len consecutive rows of one request share one
 *               block-table row (request = r / (groups*query_len)).
 *               rows == 0 returns SDA_OK without launching anything.
 *  heads        query heads per row, 1..16.
 *  groups       KV groups G (cache dim 1).
 *  query_len    query tokens per request (1 for decode, >1 for MTP verify).
 *  block        tokens per cache page (cache dim 2).
 *  R            region slots per row (regions dim 1), 0..SDA_MAX_R.  R = 0
 *               is accepted (every active row then outputs zeros), where
 *               the page's kernel needs a regions tensor with at least one
 *               column.
 *  region_tokens tokens per region; 0 means one region per page (= block).
 *               It must divide block.  Region id i covers tokens
 *               [i*region_tokens, (i+1)*region_tokens).
 *  query        bf16 [rows, heads, 192]; dim stride 1; 16-byte aligned, with
 *               row and head strides multiples of 8.
 *  output       bf16 [rows, heads, 192], written in place; dim stride 1;
 *               4-byte aligned, with even strides.
 *  cache        [pages, groups, block, 384]: K in [0:192], V in [192:384].
 *               Last-dim stride 1.  16-byte aligned, with the page, group
 *               and token strides multiples of 16 bytes.  Addressing is
 *               64-bit, so caches larger than 4 GiB are fine.
 *  kv_dtype     sda_kv_dtype of the cache.
 *  regions      int32 [rows, R], unit inner stride.  A negative id marks an
 *               unused slot.  Slot order is irrelevant.  A region whose first
 *               token lies past the row's position contributes nothing; its
 *               block-table entry is never read.
 *  block_table  int32 [requests, pages per request].  Token t of a request
 *               lives at page block_table[request, t / block], slot
 *               t % block.
 *  positions    int32 [rows]: 0-based position of the row's query token.
 *               Token t is visible iff t <= position (inclusive causal mask).
 *  active       uint8 [rows]; 0 marks an inactive (padding) row.  Its query,
 *               gate, block-table row and cache pages are never read, and its
 *               output depends on nothing but the flag; its position and
 *               region ids may be loaded (so they must be addressable), but
 *               their values are never used.
 *  scale        softmax scale applied to q.k.
 *  splits       >= 1: the row's visible regions are dealt to `splits`
 *               workgroups, and their partials are merged by log-sum-exp.
 *               Use sda_splits(rows).  The result does not depend on it
 *               beyond rounding.
 *  clear_inactive  nonzero: inactive rows are written as +0.0.  Zero: they
 *               are left untouched.
 *  k_scale, v_scale  device fp32 scalars, required for SDA_KV_FP8_E4M3 and
 *               ignored for bf16.  Dequantized K = e4m3(byte) * k_scale, and
 *               likewise for V.
 *  gate         optional bf16 [tokens, groups*heads] headwise gate logits, or
 *               NULL.  Head h of row r is scaled by the bf16-rounded
 *               sigmoid(gate[r / groups, (r % groups)*heads + h]).  This is
 *               the `_gate` helper on the same page.
 *  workspace    device scratch of at least sda_workspace_bytes(rows, heads,
 *               splits) bytes, 16-byte aligned.  May be NULL when splits == 1;
 *               rows then start in index order.  Given a workspace, a call
 *               whose grid of rows*splits workgroups takes 2 to 4 rounds of
 *               the workgroups the chip holds at once (up to 2048) first
 *               ranks rows by visible tokens and starts the heavy ones first
 *               (the result is the same either way).
 */
typedef struct sda_decode_args {
  int32_t rows, heads, groups, query_len, block, R, region_tokens;
  const void *query;
  int64_t q_row_stride, q_head_stride;
  void *output;
  int64_t o_row_stride, o_head_stride;
  const void *cache;
  int32_t kv_dtype;
  int64_t c_page_stride, c_group_stride, c_token_stride;
  const int32_t *regions;
  int64_t regions_row_stride;
  const int32_t *block_table;
  int64_t table_row_stride;
  const int32_t *positions;
  const uint8_t *active;
  float scale;
  int32_t splits;
  int32_t clear_inactive;
  const float *k_scale;
  const float *v_scale;
  const void *gate;
  int64_t gate_row_stride, gate_head_stride;
  void *workspace;
  size_t workspace_bytes;
} sda_decode_args;

/*
 * Enqueue one sparse decode attention call on `stream`.  The call is
 * asynchronous, performs no host synchronisation and no allocation, and may
 * be captured in a HIP graph.  It launches the split kernel, a (rows, splits)
 * grid.  When splits > 1 it also launches the combine kernel, which merges
 * the partials and then applies the gate and the inactive-row clear.  When
 * splits == 1 the combine is fused into the split kernel.  Two variants of
 * the schedule depend on the device's compute-unit count (the result is the
 * same): a grid of 2 to 4 rounds of resident workgroups with a workspace is
 * preceded by the bin and order kernels (heaviest rows first), and a large
 * batch of short region lists runs the row-stream kernel instead of the
 * split kernel: one 4-wave workgroup per CU whose waves take whole rows
 * back to back (splits == 1, output on 16-byte boundaries, R <= 64, and
 * with w = 4 * CUs waves, 2w <= rows <= 8w and ceil(rows / w) * R <= 256).
 * sda_decode_kernels reports which.
 * Returns an sda_status.
 */
int sda_decode(const sda_decode_args *args, hipStream_t stream);

/*
 * The kernels sda_decode(args, stream) would launch, as SDA_KERNEL_* bits in
 * *kernels (0 when rows == 0).  It validates exactly as sda_decode does and
 * returns the same status, but launches nothing and touches no device
 * memory: only the device's compute-unit count is queried.  *kernels is 0
 * on any error; kernels == NULL gives SDA_ERR_INVALID.  For profilers and
 * benchmarks that name the kernel they measure.
 */
#define SDA_KERNEL_ORDER 1      /* bin + order kernels (row ranking) */
#define SDA_KERNEL_SPLIT 2      /* split kernel, (rows, splits) grid */
#define SDA_KERNEL_ROW_STREAM 4 /* row-stream kernel, one workgroup per CU */
#define SDA_KERNEL_COMBINE 8    /* combine kernel (splits > 1) */
int sda_decode_kernels(const sda_decode_args *args, hipStream_t stream, int *kernels);

/*
 * sda_decode without a caller workspace, for callers that cannot allocate:
 * code under HIP graph capture, serving loops and harnesses that forbid
 * hipMalloc.  It is sda_decode (same arguments, validation, kernels and
 * result) with the library's own static device array of
 * SDA_STATIC_SCRATCH_BYTES as the workspace; the caller still passes every
 * input and output.  args->workspace must be NULL and args->workspace_bytes
 * 0 (else SDA_ERR_INVALID).  A call whose sda_workspace_bytes(rows, heads,
 * splits) exceeds SDA_STATIC_SCRATCH_BYTES returns SDA_ERR_SCRATCH before
 * touching the device; with splits from sda_splits every call up to 2M rows
 * fits.  The call allocates nothing: each GPU holds its own copy of the
 * array from the first call on it until the process ends, and the array
 * keeps the last call's contents (nothing in it has to start at zero).  All
 * calls on one GPU share that GPU's array, so calls that may overlap on one
 * GPU (other streams, other threads) race: serialise them, or use
 * sda_decode with a workspace each.
 */
#define SDA_STATIC_SCRATCH_BYTES (16u << 20)
int sda_decode_static(const sda_decode_args *args, hipStream_t stream);

/*
 * Split count for `rows` rows.  This is the MI355X counterpart of
 * `sparse_decode_splits` on page "...ops.sparse_decode_attention".  It depends
 * on rows only, because graphs are captured per batch size.  Host-only and
 * pure; returns 1 for rows <= 0.
 */
int sda_splits(int rows);

/*
 * Bytes of workspace for sda_decode: the row order and row bins, rows*8
 * bytes rounded up to 256, plus, when splits > 1, the fp32 partial outputs
 * and log-sum-exps, rows*splits*heads*(192+1)*4 bytes rounded up to 256.
 * The partials are the split outputs and log-sum-exps that
 * `sparse_decode_attention` (page "...ops.sparse_decode_attention") allocates
 * with torch.empty for its combine; here the caller owns that memory.
 * Returns 0 for invalid sizes.
 */
size_t sda_workspace_bytes(int rows, int heads, int splits);

/*
 * Gated sliding-window decode: the fused decode of the non-DSA layers, page
 * "vllm.models.step5.nvidia.sparse_attention", section
 * `Step5SplitKVFlashAttentionImpl` (`forward_with_headwise_gate`, which
 * calls `swa_decode_gated`, and `_split_kv_cache`, which views the same
 * packed cache as K and V).  A uniform batch of tokens = requests *
 * query_len query tokens; token j (0-based) of request q has position
 * seq_lens[q] - query_len + j and attends, head by head, over the tokens at
 * positions max(0, pos - window + 1) .. pos of its request (a causal window
 * of `window` tokens, i.e. sliding_window[0] + 1).  The query heads of a KV
 * group are packed into one workgroup (GQA), as in sda_decode, together
 * with up to `pack` consecutive query tokens of the request, whose windows
 * overlap (`swa_decode_plan` returns such a pack), and the headwise sigmoid
 * gate (the `_gate` helper of page "...ops.
 * sparse_decode_attention") scales each head.  A token whose position is
 * negative (seq_len < query_len) outputs zeros.  Strides are in ELEMENTS.
 *
 *  tokens       query tokens, a multiple of query_len; 0 returns SDA_OK.
 *               tokens * groups must not exceed SDA_MAX_ROWS.
 *  heads        query heads per KV group, 1..16.
 *  groups       KV groups G (cache dim 1).
 *  query_len    query tokens per request (1 decode, 2..4 MTP verify; any
 *               value >= 1 is accepted).
 *  block        tokens per page; a multiple of 16 (else UNSUPPORTED).
 *  window       tokens attended, >= 1.  (window + pack + 14) / block + 2
 *               must not exceed SDA_MAX_R (else UNSUPPORTED).
 *  pack         query tokens per workgroup, 1..min(query_len, 16 / heads),
 *               or 0 for that maximum (sda_swa_plan).  Each token's heads
 *               are separate MFMA columns with their own window mask; the
 *               union of the windows is read once.  The result does not
 *               depend on it beyond rounding.
 *  query        bf16 [tokens, groups*heads, 192]; head g*heads + h belongs
 *               to KV group g.  Dim stride 1; 16-byte aligned; token and
 *               head strides multiples of 8.
 *  output       bf16 [tokens, groups*heads, 192], written in place; dim
 *               stride 1; 4-byte aligned; even strides.
 *  cache        bf16 [pages, groups, block, 384], K then V; same alignment
 *               and 32-bit in-page offset rules as sda_decode.
 *  block_table  int32 [requests, pages per request], unit inner stride.
 *               Only the columns covering each window are read.
 *  seq_lens     int32 [requests]: tokens of the request, the new ones
 *               included.
 *  scale        softmax scale applied to q.k.
 *  splits       >= 1 (sda_swa_plan): each row's window is cut into
 *               `splits` contiguous runs whose partials are merged by
 *               log-sum-exp.  The result does not depend on it beyond
 *               rounding.
 *  gate         bf16 [tokens, groups*heads] gate logits, or NULL for none.
 *  workspace    as for sda_decode, sda_workspace_bytes(tokens*groups,
 *               heads, splits) bytes; may be NULL when splits == 1.
 */
typedef struct sda_swa_args {
  int32_t tokens, heads, groups, query_len, block, window, pack;
  const void *query;
  int64_t q_token_stride, q_head_stride;
  void *output;
  int64_t o_token_stride, o_head_stride;
  const void *cache;
  int64_t c_page_stride, c_group_stride, c_token_stride;
  const int32_t *block_table;
  int64_t table_row_stride;
  const int32_t *seq_lens;
  float scale;
  int32_t splits;
  const void *gate;
  int64_t gate_token_stride, gate_head_stride;
  void *workspace;
  size_t workspace_bytes;
} sda_swa_args;

/*
 * Enqueue one gated sliding-window decode call on `stream`: the split kernel
 * of sda_decode in its window mode over a (requests * ceil(query_len / pack)
 * * groups, splits) grid, and the combine kernel (per row) when splits > 1.  Asynchronous, no allocation, no host
 * synchronisation.  Returns an sda_status; on error nothing is launched.
 */
int sda_swa_decode(const sda_swa_args *args, hipStream_t stream);

/*
 * Plan of a sliding-window call, the MI355X counterpart of `swa_decode_plan`
 * (page "vllm.models.step5.nvidia.sparse_attention",
 * `forward_with_headwise_gate`, which passes it the device's SM count before
 * the window): writes the pack (the largest, min(query_len, 16 / heads)) to
 * *pack if pack is not NULL and returns the split count: double while the
 * doubled grid of requests * ceil(query_len / pack) * groups * splits * 2
 * workgroups fits `compute_units` (up to 32 splits), further capped so that
 * every split keeps at least 8 chunks of 16 tokens of the packed tokens'
 * union window.  compute_units <= 0 reads the current device's count
 * (sda_device_compute_units); given a count, the call is host-only and pure.
 * Returns 1 (and pack 1) for invalid sizes.
 */
int sda_swa_plan(int tokens, int groups, int heads, int query_len, int compute_units, int window,
                 int *pack);

/*
 * Compute units of HIP device `device` (the current device when negative),
 * from hipDeviceAttributeMultiprocessorCount, read once per device; 0 if the
 * runtime cannot report it.  sda_decode, sda_swa_decode and
 * sda_select_regions size their residency decisions (waves per workgroup,
 * the row-order pass, two selection workgroups per CU) from the count of the
 * device their stream runs on; they return SDA_ERR_LAUNCH when it cannot be
 * read.  sda_splits does not use it: like the page's
 * `sparse_decode_splits`, it depends on rows only.
 */
int sda_device_compute_units(int device);

/*
 * Region selection: `select_regions` on page "vllm.models.step5.nvidia.
 * flashinfer_sparse" as `select_and_run_decode_attention` calls it before the
 * sparse decode (`sort=False`).  For each row: the candidates are regions
 * 0 .. n_r - 1, n_r = topk_lengths[r] clamped to [0, num_regions] (all
 * num_regions score columns when topk_lengths is NULL).  The current region is
 * selected whenever it is a candidate; the other topk - 1 slots take the
 * highest-scoring remaining candidates.  Equal scores go to the lower region
 * id (-0.0 ranks below +0.0).  The selected ids are written in ascending
 * order, followed by -1 up to topk: exactly the `regions` input of
 * sda_decode (with region_tokens = the indexer's region size).  NaN scores
 * are outside the contract.  All pointers are device pointers; strides in
 * elements.
 *
 *  rows          rows (token, KV group), at most SDA_SELECT_MAX_ROWS; 0 returns
 *                OK.
 *  num_regions   score columns S, 0..SDA_MAX_SCORE_COLUMNS.
 *  topk          output slots per row; 0 returns OK.
 *  scores        fp32 [rows, S], unit inner stride, 4-byte aligned.
 *  current       int32 [rows]: the region holding the row's own token
 *                (position / region_tokens); a value outside [0, n_r) forces
 *                nothing.
 *  topk_lengths  int32 [rows] or NULL.
 *  regions       int32 [rows, topk] output; row stride >= topk.
 */
#define SDA_MAX_SCORE_COLUMNS 32768
#define SDA_SELECT_MAX_ROWS 4194303 /* grid limit: rows * 1024 threads < 2^32 */

typedef struct sda_select_args {
  int32_t rows, num_regions, topk;
  const float *scores;
  int64_t scores_row_stride;
  const int32_t *current;
  const int32_t *topk_lengths;
  int32_t *regions;
  int64_t regions_row_stride;
} sda_select_args;

/*
 * Enqueue one selection call: one 1024-thread workgroup per row (radix select
 * of the threshold score in registers and LDS, then an ordered compaction).
 * Asynchronous, no allocation.  Returns an sda_status; on error nothing is
 * launched.
 */
int sda_select_regions(const sda_select_args *args, hipStream_t stream);

/*
 * Decode indexer logits: the region scores `decode_logits` produces on page
 * "vllm.models.step5.nvidia.flashinfer_sparse" for the selection that follows
 * (its kernels are not shown; this formula is a reading):
 *     scores[r, j] = sum_h weights[r, h] * max(0, s_j * (q[r, h, :] . k_j))
 * for regions j = 0 .. positions[r] / region_tokens of row r, and -inf for
 * the other score columns.  q and k_j are OCP e4m3 (exact products, fp32
 * sums); k_j is region j's 256-byte summary, kept in the page that holds its
 * tokens: page block_table[request, j / regions_per_page], slot
 * j % regions_per_page, with fp32 scale s_j.  Row r is group r % groups of
 * token r / groups; the groups * query_len rows of a request share its
 * block-table row, and its rows x heads query columns (<= 64) are scored
 * together, reading each summary once per request.  Strides: bytes for the
 * e4m3 tensors, elements otherwise.
 *
 *  rows, heads   rows (a multiple of groups * query_len); indexer heads per
 *                row, a power of two <= 16.
 *  regions_per_page  summaries per page (block / region_tokens).
 *  num_regions   score columns S, at most SDA_LOGITS_MAX_REGIONS.
 *  query         e4m3 [rows, heads, 256]; 16-byte aligned rows and heads.
 *  weights       fp32 [rows, heads], unit head stride.
 *  summaries     e4m3 [pages, regions_per_page, 256]; 16-byte aligned.
 *  summary_scales fp32 [pages, regions_per_page], unit region stride.
 *  block_table   int32 [requests, cols], unit inner stride.
 *  table_cols    cols of block_table (>= 0, and <= table_row_stride when
 *                positive), or 0 if unknown.  Every scored region's column
 *                lies below cols.  With cols given, a workgroup requests its
 *                chunk's table entries (columns below cols) together with
 *                the positions, one dependent round trip fewer; with 0 only
 *                the columns of each request's scored regions are read.
 *  positions     int32 [rows].
 *  scores        fp32 [rows, S] output, 4-byte aligned (else INVALID); the row
 *                stride (in floats, any value) must keep rows apart, which is
 *                not checked.
 *  current, topk_lengths  optional int32 [rows] outputs for the selection:
 *                positions / region_tokens (-1 for a negative position) and
 *                the scored region count min(current + 1, S).
 */
#define SDA_LOGITS_MAX_COLUMNS 64
#define SDA_LOGITS_MAX_REGIONS (65535 * 256) /* grid limit: 256 regions per workgroup */

typedef struct sda_logits_args {
  int32_t rows, heads, groups, query_len, regions_per_page, num_regions, region_tokens;
  const void *query;
  int64_t q_row_stride, q_head_stride;
  const float *weights;
  int64_t w_row_stride;
  const void *summaries;
  int64_t s_page_stride, s_region_stride;
  const float *summary_scales;
  int64_t ss_page_stride;
  const int32_t *block_table;
  int64_t table_row_stride;
  const int32_t *positions;
  float *scores;
  int64_t scores_row_stride;
  int32_t *current;
  int32_t *topk_lengths;
  int32_t table_cols;
} sda_logits_args;

/*
 * Enqueue one logits call: a (requests, ceil(S / 256)) grid of 256-thread
 * workgroups.  Asynchronous, no allocation.  Returns an sda_status; on error
 * nothing is launched.
 */
int sda_indexer_logits(const sda_logits_args *args, hipStream_t stream);

/* Static description of a status code (never NULL). */
const char *sda_status_string(int status);

/* SDA_ABI_VERSION of the built library, and the sizes of sda_decode_args,
 * sda_swa_args, sda_select_args and sda_logits_args, so a binding can check
 * that its mirrors of the structs match. */
int sda_abi_version(void);
size_t sda_args_size(void);
size_t sda_swa_args_size(void);
size_t sda_select_args_size(void);
size_t sda_logits_args_size(void);

#ifdef __cplusplus
}
#endif

#endif /* SDA_H_ */
