// C-ABI layer of libsda.so: host-side validation, split heuristic, workspace
// sizing and kernel launch.  Declarations and the full contract are in
// include/sda.h.
#include "sda.h"

#include <hip/hip_runtime_api.h>

#include <atomic>

#include "sda_launch.h"

static_assert(SDA_MAX_R == sda::kMaxRegions, "LDS region list must hold SDA_MAX_R slots");

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// Workspace layout: [row order and row bins: 2*rows int32][partials:
// rows*splits*heads*192 fp32][log-sum-exps: rows*splits*heads fp32], each
// area rounded up to 256 bytes.  Sets the partial and lse pointers when
// splits > 1.
void split_areas(sda::Params& p, void* workspace) {
  char* base = static_cast<char*>(workspace) + round256((size_t)p.rows * 2 * sizeof(int32_t));
  p.partial = reinterpret_cast<float*>(base);
  p.lse = p.partial + (size_t)p.rows * p.splits * p.heads * SDA_HEAD_DIM;
}

// Split count for `rows` rows on MI355X.  The page "vllm.models.step5.nvidia.
// ops.sparse_decode_attention" (`sparse_decode_splits`) doubles the split
// count while rows*splits*2 <= 256, up to 32 splits.  On B300 that sizes the
// grid for about 1.7 waves of programs.  Here a grid of at most 256 split
// workgroups runs them with 4 waves each (~121 KiB of LDS), one per compute
// unit, so the target is one workgroup per CU: double while the doubled grid
// rows*splits*2 still fits the 256 CUs.  That is the page's rule and bound,
// for a different reason.  On the bf16 gated workload (256 rows) 2 splits
// are slower than 1: the merge costs more than the idle CUs of inactive rows.
constexpr int kComputeUnits = 256;  // MI355X; the target of sda_splits, which stays pure
constexpr int kMaxHeuristicSplits = 32;
constexpr int kSwaMinChunksPerSplit = 8;

// Query tokens of one request that share a window workgroup: as many as fit
// the 16 MFMA columns next to the heads of one KV group.
int max_pack(int heads, int query_len) {
  const int fit = SDA_MAX_HEADS / heads;
  return fit < query_len ? fit : query_len;
}

// Compute units of each device, read once (0 = not read yet).  The plans
// and residency decisions size grids from the device the call runs on, as
// the pages size theirs from `multi_processor_count`.
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_cus[kMaxDevices];

int device_cus(int device) {
  if (device < 0) {
    if (hipGetDevice(&device) != hipSuccess) return 0;
  }
  if (device >= kMaxDevices) {
    int n = 0;
    return hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) == hipSuccess
               ? n
               : 0;
  }
  int n = g_device_cus[device].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      n <= 0)
    return 0;
  g_device_cus[device].store(n, std::memory_order_relaxed);
  return n;
}

// The device a launch on `stream` runs on: the stream's own, or the current
// device for the null stream.
int stream_cus(hipStream_t stream) {
  int device = -1;
  if (stream && hipStreamGetDevice(stream, &device) != hipSuccess) return 0;
  return device_cus(device);
}

}  // namespace

extern "C" {

int sda_device_compute_units(int device) { return device_cus(device); }

int sda_abi_version(void) { return SDA_ABI_VERSION; }

size_t sda_args_size(void) { return sizeof(sda_decode_args); }

int sda_splits(int rows) {
  int splits = 1;
  if (rows <= 0) return 1;
  while (splits < kMaxHeuristicSplits && (int64_t)rows * splits * 2 <= kComputeUnits) splits *= 2;
  return splits;
}

size_t sda_workspace_bytes(int rows, int heads, int splits) {
  if (rows < 0 || heads < 1 || heads > SDA_MAX_HEADS || splits < 1 || splits > SDA_MAX_SPLITS)
    return 0;
  const size_t order = round256((size_t)rows * 2 * sizeof(int32_t));
  if (splits == 1) return order;
  size_t n = (size_t)rows * (size_t)splits * (size_t)heads;
  return order + round256(n * (SDA_HEAD_DIM + 1) * sizeof(float));
}

const char* sda_status_string(int status) {
  switch (status) {
    case SDA_OK: return "ok";
    case SDA_ERR_INVALID: return "invalid argument";
    case SDA_ERR_UNSUPPORTED: return "unsupported argument (alignment, stride or size limit)";
    case SDA_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case SDA_ERR_LAUNCH: return "kernel launch failed";
    case SDA_ERR_SCRATCH:
      return "the call needs more workspace than the static scratch (SDA_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"

namespace {

// Validate a decode call and fill the kernel parameters.  Returns SDA_OK with
// *empty set when there is nothing to launch (rows == 0).
int prepare_decode(const sda_decode_args* a, hipStream_t stream, sda::Params& p, bool& fp8,
                   bool& empty) {
  empty = false;
  if (!a) return SDA_ERR_INVALID;
  // Shape contract: the asserts of `sparse_decode_attention` and the
  // `_direct_sparse_decode` eligibility rule (dim 192, <= 16 heads, 384-wide
  // unit-stride cache rows).
  if (a->rows < 0 || a->heads < 1 || a->heads > SDA_MAX_HEADS || a->groups < 1 ||
      a->query_len < 1 || a->block < 1 || a->R < 0 || a->splits < 1 || a->region_tokens < 0)
    return SDA_ERR_INVALID;
  if (a->kv_dtype != SDA_KV_BF16 && a->kv_dtype != SDA_KV_FP8_E4M3) return SDA_ERR_INVALID;
  const int rt = a->region_tokens ? a->region_tokens : a->block;
  if (a->block % rt) return SDA_ERR_INVALID;
  const int64_t rows_per_req = (int64_t)a->groups * a->query_len;
  if (a->rows % rows_per_req) return SDA_ERR_INVALID;
  fp8 = a->kv_dtype == SDA_KV_FP8_E4M3;
  if (fp8 && (!a->k_scale || !a->v_scale)) return SDA_ERR_INVALID;
  if (a->R > SDA_MAX_R || a->splits > SDA_MAX_SPLITS || a->rows > SDA_MAX_ROWS)
    return SDA_ERR_UNSUPPORTED;
  if (a->rows == 0) {  // nothing to do, nothing launched
    empty = true;
    return SDA_OK;
  }

  if (!a->query || !a->output || !a->cache || !a->block_table || !a->positions || !a->active ||
      (a->R > 0 && !a->regions))
    return SDA_ERR_INVALID;

  // Vector-load alignment: 16-byte Q and cache rows, 4-byte output pairs.
  const int64_t esz = fp8 ? 1 : 2;
  if (!aligned(a->query, 16) || a->q_row_stride % 8 || a->q_head_stride % 8)
    return SDA_ERR_UNSUPPORTED;
  if (!aligned(a->cache, 16) || (a->c_page_stride * esz) % 16 || (a->c_group_stride * esz) % 16 ||
      (a->c_token_stride * esz) % 16)
    return SDA_ERR_UNSUPPORTED;
  if (!aligned(a->output, 4) || a->o_row_stride % 2 || a->o_head_stride % 2)
    return SDA_ERR_UNSUPPORTED;
  // Token rows of one page are addressed with 32-bit byte offsets.
  if (a->c_token_stride < 0 || (int64_t)a->block * a->c_token_stride * esz + 2 * SDA_KV_ROW > 0xFFFFFFFFll)
    return SDA_ERR_UNSUPPORTED;

  p = sda::Params{};
  // row r = token r / groups, group r % groups: row stride per group
  p.q = static_cast<const uint16_t*>(a->query);
  p.qts = a->q_row_stride * a->groups;
  p.qgs = a->q_row_stride;
  p.qhs = a->q_head_stride;
  p.out = static_cast<uint16_t*>(a->output);
  p.ots = a->o_row_stride * a->groups;
  p.ogs = a->o_row_stride;
  p.ohs = a->o_head_stride;
  p.cache = static_cast<const uint8_t*>(a->cache);
  p.cps = a->c_page_stride;
  p.cgs = a->c_group_stride;
  p.cts = a->c_token_stride;
  p.regions = a->regions;
  p.rrs = a->regions_row_stride;
  p.table = a->block_table;
  p.trs = a->table_row_stride;
  p.positions = a->positions;
  p.active = a->active;
  p.k_scale = a->k_scale;
  p.v_scale = a->v_scale;
  p.gate = static_cast<const uint16_t*>(a->gate);
  p.grs = a->gate_row_stride;
  p.ghs = a->gate_head_stride;
  p.scale = a->scale;
  p.rows = a->rows;
  p.heads = a->heads;
  p.groups = a->groups;
  p.rows_per_req = (int32_t)rows_per_req;
  p.block = a->block;
  p.R = a->R;
  p.rt = rt;
  p.rt_shift = (rt & (rt - 1)) == 0 ? __builtin_ctz((unsigned)rt) : -1;
  p.splits = a->splits;
  p.clear = a->clear_inactive ? 1 : 0;
  p.gated = a->gate ? 1 : 0;

  // splits == 1 needs no workspace; given one, the launch may use its order
  // area to start heavy rows first.
  if (a->splits > 1 || a->workspace) {
    size_t need = sda_workspace_bytes(a->rows, a->heads, a->splits);
    if (!a->workspace || a->workspace_bytes < need || !aligned(a->workspace, 16))
      return SDA_ERR_WORKSPACE;
    p.order_ws = static_cast<int32_t*>(a->workspace);
    if (a->splits > 1) split_areas(p, a->workspace);
  }
  p.cus = stream_cus(stream);
  if (p.cus <= 0) return SDA_ERR_LAUNCH;
  return SDA_OK;
}

}  // namespace

extern "C" {

int sda_decode(const sda_decode_args* a, hipStream_t stream) {
  sda::Params p;
  bool fp8 = false, empty = false;
  const int rc = prepare_decode(a, stream, p, fp8, empty);
  if (rc != SDA_OK || empty) return rc;
  hipError_t e = sda::launch(p, fp8, stream);
  return e == hipSuccess ? SDA_OK : SDA_ERR_LAUNCH;
}

int sda_decode_kernels(const sda_decode_args* a, hipStream_t stream, int* kernels) {
  if (!kernels) return SDA_ERR_INVALID;
  *kernels = 0;
  sda::Params p;
  bool fp8 = false, empty = false;
  const int rc = prepare_decode(a, stream, p, fp8, empty);
  if (rc != SDA_OK || empty) return rc;
  const int bits = sda::plan(p);
  *kernels = ((bits & sda::kPlanOrder) ? SDA_KERNEL_ORDER : 0) |
             ((bits & sda::kPlanSplit) ? SDA_KERNEL_SPLIT : 0) |
             ((bits & sda::kPlanRowStream) ? SDA_KERNEL_ROW_STREAM : 0) |
             ((bits & sda::kPlanCombine) ? SDA_KERNEL_COMBINE : 0);
  return SDA_OK;
}

size_t sda_swa_args_size(void) { return sizeof(sda_swa_args); }

int sda_swa_plan(int tokens, int groups, int heads, int query_len, int compute_units, int window,
                 int* pack) {
  if (pack) *pack = 1;
  if (tokens <= 0 || groups <= 0 || window <= 0 || heads < 1 || heads > SDA_MAX_HEADS ||
      query_len < 1 || tokens % query_len)
    return 1;
  const int cus = compute_units > 0 ? compute_units : device_cus(-1);
  if (cus <= 0) return 1;
  const int pk = max_pack(heads, query_len);
  if (pack) *pack = pk;
  // The row-count rule of sda_splits on workgroups, for the device's compute
  // units, and at least kSwaMinChunksPerSplit 16-token chunks per split so
  // that each of the 4 waves keeps its pipeline.
  const int64_t wgs = (int64_t)(tokens / query_len) * (((int64_t)query_len + pk - 1) / pk) * groups;
  const int64_t chunks = ((int64_t)window + pk - 1 + 15) / 16;
  int splits = 1;
  while (splits < kMaxHeuristicSplits && wgs * splits * 2 <= cus &&
         chunks >= (int64_t)kSwaMinChunksPerSplit * splits * 2)
    splits *= 2;
  return splits;
}

int sda_swa_decode(const sda_swa_args* a, hipStream_t stream) {
  if (!a) return SDA_ERR_INVALID;
  // Shape contract of the fused path of `forward_with_headwise_gate`: a
  // uniform batch (tokens = requests * query_len), head dim 192, <= 16 query
  // heads per KV group, a causal window of >= 1 token.
  if (a->tokens < 0 || a->heads < 1 || a->heads > SDA_MAX_HEADS || a->groups < 1 ||
      a->query_len < 1 || a->block < 1 || a->window < 1 || a->splits < 1)
    return SDA_ERR_INVALID;
  if (a->tokens % a->query_len) return SDA_ERR_INVALID;
  const int pmax = max_pack(a->heads, a->query_len);
  if (a->pack < 0 || a->pack > pmax) return SDA_ERR_INVALID;
  const int pack = a->pack ? a->pack : pmax;
  if (a->splits > SDA_MAX_SPLITS || a->block % 16) return SDA_ERR_UNSUPPORTED;
  // LDS page list: a split's run of chunks spans at most the union window
  // (window + pack - 1 tokens) plus 15 tokens of alignment.
  if (((int64_t)a->window + pack - 1 + 15) / a->block + 2 > sda::kMaxRegions)
    return SDA_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)a->tokens * a->groups;
  if (rows > SDA_MAX_ROWS) return SDA_ERR_UNSUPPORTED;
  if (a->tokens == 0) return SDA_OK;

  if (!a->query || !a->output || !a->cache || !a->block_table || !a->seq_lens)
    return SDA_ERR_INVALID;
  if (!aligned(a->query, 16) || a->q_token_stride % 8 || a->q_head_stride % 8)
    return SDA_ERR_UNSUPPORTED;
  if (!aligned(a->cache, 16) || (a->c_page_stride * 2) % 16 || (a->c_group_stride * 2) % 16 ||
      (a->c_token_stride * 2) % 16)
    return SDA_ERR_UNSUPPORTED;
  if (!aligned(a->output, 4) || a->o_token_stride % 2 || a->o_head_stride % 2)
    return SDA_ERR_UNSUPPORTED;
  if (a->c_token_stride < 0 || (int64_t)a->block * a->c_token_stride * 2 + 2 * SDA_KV_ROW > 0xFFFFFFFFll)
    return SDA_ERR_UNSUPPORTED;

  sda::Params p{};
  p.q = static_cast<const uint16_t*>(a->query);
  p.qts = a->q_token_stride;
  p.qgs = a->q_head_stride * a->heads;  // group g's heads start at head g*heads
  p.qhs = a->q_head_stride;
  p.out = static_cast<uint16_t*>(a->output);
  p.ots = a->o_token_stride;
  p.ogs = a->o_head_stride * a->heads;
  p.ohs = a->o_head_stride;
  p.cache = static_cast<const uint8_t*>(a->cache);
  p.cps = a->c_page_stride;
  p.cgs = a->c_group_stride;
  p.cts = a->c_token_stride;
  p.table = a->block_table;
  p.trs = a->table_row_stride;
  p.seq_lens = a->seq_lens;
  p.gate = static_cast<const uint16_t*>(a->gate);
  p.grs = a->gate_token_stride;
  p.ghs = a->gate_head_stride;
  p.scale = a->scale;
  p.rows = (int32_t)rows;
  p.heads = a->heads;
  p.groups = a->groups;
  p.rows_per_req = a->groups * a->query_len;
  p.block = a->block;
  p.rt = a->block;
  p.rt_shift = -1;
  p.splits = a->splits;
  p.gated = a->gate ? 1 : 0;
  p.query_len = a->query_len;
  p.window = a->window;
  p.pack = pack;
  p.ntg = (a->query_len + pack - 1) / pack;

  if (a->splits > 1) {
    size_t need = sda_workspace_bytes(p.rows, a->heads, a->splits);
    if (!a->workspace || a->workspace_bytes < need || !aligned(a->workspace, 16))
      return SDA_ERR_WORKSPACE;
    split_areas(p, a->workspace);
  }
  p.cus = stream_cus(stream);
  if (p.cus <= 0) return SDA_ERR_LAUNCH;

  hipError_t e = sda::launch_window(p, stream);
  return e == hipSuccess ? SDA_OK : SDA_ERR_LAUNCH;
}

size_t sda_select_args_size(void) { return sizeof(sda_select_args); }

int sda_select_regions(const sda_select_args* a, hipStream_t stream) {
  if (!a) return SDA_ERR_INVALID;
  if (a->rows < 0 || a->num_regions < 0 || a->topk < 0) return SDA_ERR_INVALID;
  if (a->rows > 1 && a->regions_row_stride < a->topk) return SDA_ERR_INVALID;
  if (a->num_regions > SDA_MAX_SCORE_COLUMNS || a->rows > SDA_SELECT_MAX_ROWS)
    return SDA_ERR_UNSUPPORTED;
  if (a->rows == 0 || a->topk == 0) return SDA_OK;
  if (!a->current || !a->regions || (a->num_regions > 0 && !a->scores)) return SDA_ERR_INVALID;
  if (!aligned(a->scores, 4) || !aligned(a->current, 4) || !aligned(a->topk_lengths, 4) ||
      !aligned(a->regions, 4))
    return SDA_ERR_INVALID;
  sda::SelParams p{};
  p.scores = a->scores;
  p.srs = a->scores_row_stride;
  p.current = a->current;
  p.lengths = a->topk_lengths;
  p.out = a->regions;
  p.ors = a->regions_row_stride;
  p.rows = a->rows;
  p.S = a->num_regions;
  p.topk = a->topk;
  p.cus = stream_cus(stream);
  if (p.cus <= 0) return SDA_ERR_LAUNCH;
  hipError_t e = sda::launch_select(p, stream);
  return e == hipSuccess ? SDA_OK : SDA_ERR_LAUNCH;
}

size_t sda_logits_args_size(void) { return sizeof(sda_logits_args); }

int sda_indexer_logits(const sda_logits_args* a, hipStream_t stream) {
  if (!a) return SDA_ERR_INVALID;
  if (a->rows < 0 || a->heads < 1 || a->heads > SDA_MAX_HEADS || (a->heads & (a->heads - 1)) ||
      a->groups < 1 || a->query_len < 1 || a->regions_per_page < 1 || a->num_regions < 0 ||
      a->region_tokens < 1 || a->table_cols < 0 ||
      (a->table_cols > 0 && a->table_row_stride < a->table_cols))
    return SDA_ERR_INVALID;
  const int64_t rpr = (int64_t)a->groups * a->query_len;
  if (a->rows % rpr) return SDA_ERR_INVALID;
  if (rpr * a->heads > SDA_LOGITS_MAX_COLUMNS || a->rows > SDA_MAX_ROWS ||
      a->num_regions > SDA_LOGITS_MAX_REGIONS)
    return SDA_ERR_UNSUPPORTED;
  if (a->rows == 0 || a->num_regions == 0) return SDA_OK;
  if (!a->query || !a->weights || !a->summaries || !a->summary_scales || !a->block_table ||
      !a->positions || !a->scores)
    return SDA_ERR_INVALID;
  // 16-byte query / summary loads (the scores are stored 4 bytes at a time)
  if (!aligned(a->query, 16) || a->q_row_stride % 16 || a->q_head_stride % 16 ||
      !aligned(a->summaries, 16) || a->s_page_stride % 16 || a->s_region_stride % 16)
    return SDA_ERR_UNSUPPORTED;
  if (!aligned(a->weights, 4) || !aligned(a->summary_scales, 4) || !aligned(a->scores, 4) ||
      !aligned(a->current, 4) || !aligned(a->topk_lengths, 4))
    return SDA_ERR_INVALID;
  sda::LogitsParams p{};
  p.q = static_cast<const uint8_t*>(a->query);
  p.qrs = a->q_row_stride;
  p.qhs = a->q_head_stride;
  p.w = a->weights;
  p.wrs = a->w_row_stride;
  p.sm = static_cast<const uint8_t*>(a->summaries);
  p.sps = a->s_page_stride;
  p.sms = a->s_region_stride;
  p.sc = a->summary_scales;
  p.scps = a->ss_page_stride;
  p.table = a->block_table;
  p.trs = a->table_row_stride;
  p.tcols = a->table_cols;
  p.positions = a->positions;
  p.out = a->scores;
  p.ors = a->scores_row_stride;
  p.current = a->current;
  p.lengths = a->topk_lengths;
  p.rows = a->rows;
  p.heads = a->heads;
  p.hshift = __builtin_ctz((unsigned)a->heads);
  p.rows_per_req = (int32_t)rpr;
  p.rpb = a->regions_per_page;
  p.S = a->num_regions;
  p.rt = a->region_tokens;
  hipError_t e = sda::launch_logits(p, stream);
  return e == hipSuccess ? SDA_OK : SDA_ERR_LAUNCH;
}

}  // extern "C"
