// Host-only check of the C-ABI layer (sda_api.cpp) under AddressSanitizer
// and UndefinedBehaviorSanitizer.  TEST INFRASTRUCTURE: built with g++ by
// tests/test_sanitizers.py (or __graft_entry__.build(sanitize=True)); the
// library never links it.
//
// The kernel launches and the HIP device queries are stubbed here, so the
// validation, the plan functions and the argument marshalling run on the
// CPU.  Every "device" buffer is an inaccessible (PROT_NONE) mapping: the
// layer promises never to read device memory, and any host dereference of one
// would fault.  Each call that returns SDA_OK must have enqueued exactly one
// launch whose parameters stay inside the caller's workspace.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <sys/mman.h>

#include <random>

#include "sda.h"
#include "sda_launch.h"

// ---- stubs -----------------------------------------------------------------
static int g_launches = 0;
static sda::Params g_last{};
static sda::SelParams g_last_sel{};
static sda::LogitsParams g_last_logits{};

namespace sda {
hipError_t launch(const Params& p, bool, hipStream_t) {
  ++g_launches;
  g_last = p;
  return hipSuccess;
}
int plan(const Params& p) {
  g_last = p;
  return kPlanRowStream | kPlanOrder;
}
hipError_t launch_window(const Params& p, hipStream_t) {
  ++g_launches;
  g_last = p;
  return hipSuccess;
}
hipError_t launch_select(const SelParams& p, hipStream_t) {
  ++g_launches;
  g_last_sel = p;
  return hipSuccess;
}
hipError_t launch_logits(const LogitsParams& p, hipStream_t) {
  ++g_launches;
  g_last_logits = p;
  return hipSuccess;
}
}  // namespace sda

extern "C" {
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int device) {
  if (attr != hipDeviceAttributeMultiprocessorCount || device != 0) return hipErrorInvalidDevice;
  *v = 256;
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
}

// ---- helpers ---------------------------------------------------------------
static int g_fail = 0;
#define CHECK(cond, ...)                                              \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond); \
      fprintf(stderr, __VA_ARGS__);                                   \
      fprintf(stderr, "\n");                                          \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

// A large inaccessible region; "device pointers" point into it.
static char* g_dev = nullptr;
static const size_t kDevBytes = size_t(1) << 34;  // address space only

static void* dev(size_t off) { return g_dev + off; }

static bool valid_status(int rc) {
  return rc == SDA_OK || rc == SDA_ERR_INVALID || rc == SDA_ERR_UNSUPPORTED ||
         rc == SDA_ERR_WORKSPACE || rc == SDA_ERR_LAUNCH;
}

static sda_decode_args base_decode(int rows, int heads, int groups, int qlen, int splits) {
  sda_decode_args a;
  memset(&a, 0, sizeof a);
  a.rows = rows;
  a.heads = heads;
  a.groups = groups;
  a.query_len = qlen;
  a.block = 64;
  a.R = 32;
  a.query = dev(0);
  a.q_row_stride = heads * 192;
  a.q_head_stride = 192;
  a.output = dev(size_t(1) << 30);
  a.o_row_stride = heads * 192;
  a.o_head_stride = 192;
  a.cache = dev(size_t(2) << 30);
  a.kv_dtype = SDA_KV_BF16;
  a.c_page_stride = (int64_t)groups * 64 * 384;
  a.c_group_stride = 64 * 384;
  a.c_token_stride = 384;
  a.regions = (const int32_t*)dev(size_t(3) << 30);
  a.regions_row_stride = 32;
  a.block_table = (const int32_t*)dev(size_t(4) << 30);
  a.table_row_stride = 512;
  a.positions = (const int32_t*)dev(size_t(5) << 30);
  a.active = (const uint8_t*)dev(size_t(6) << 30);
  a.scale = 0.072f;
  a.splits = splits;
  a.clear_inactive = 1;
  a.workspace = dev(size_t(7) << 30);
  a.workspace_bytes = sda_workspace_bytes(rows, heads, splits);
  return a;
}

// A successful decode launch keeps its partials and log-sum-exps inside the
// first sda_workspace_bytes() bytes of the workspace, which the caller's size
// covers, and its row-order area in front of them.
static void check_decode_launch(const sda_decode_args& a) {
  const char* ws = (const char*)a.workspace;
  const size_t need = sda_workspace_bytes(a.rows, a.heads, a.splits);
  CHECK(!a.workspace || a.workspace_bytes >= need, "accepted a workspace of %zu < %zu bytes",
        a.workspace_bytes, need);
  const char* end = ws + need;
  if (a.splits > 1) {
    const char* p0 = (const char*)g_last.partial;
    const char* p1 = p0 + (size_t)a.rows * a.splits * a.heads * 192 * sizeof(float);
    const char* l0 = (const char*)g_last.lse;
    const char* l1 = l0 + (size_t)a.rows * a.splits * a.heads * sizeof(float);
    CHECK(p0 >= ws + (size_t)a.rows * 8 && p1 <= l0 && l1 <= end,
          "rows %d heads %d splits %d: partials/lse outside the workspace", a.rows, a.heads,
          a.splits);
    CHECK(((uintptr_t)p0 % 16) == 0 && ((uintptr_t)l0 % 16) == 0, "unaligned partials");
  }
  if (a.workspace) {
    CHECK((const char*)g_last.order_ws == ws, "order area moved");
  }
  CHECK(g_last.rows == a.rows && g_last.heads == a.heads && g_last.splits == a.splits,
        "sizes not passed through");
  CHECK(g_last.qts == a.q_row_stride * a.groups && g_last.qgs == a.q_row_stride,
        "query token/group strides");
  const int rt = a.region_tokens ? a.region_tokens : a.block;
  CHECK(g_last.rt == rt && a.block % rt == 0, "region tokens %d block %d", g_last.rt, a.block);
  CHECK(g_last.rt_shift < 0 ? (rt & (rt - 1)) != 0 : (1 << g_last.rt_shift) == rt,
        "rt_shift %d for rt %d", g_last.rt_shift, rt);
  CHECK(g_last.cus == 256, "compute units %d", g_last.cus);
}

static int call_decode(sda_decode_args a) {
  const int before = g_launches;
  int kernels = -1;
  const int rc_plan = sda_decode_kernels(&a, nullptr, &kernels);
  CHECK(g_launches == before, "sda_decode_kernels launched");
  if (rc_plan == SDA_OK && a.rows > 0) {
    CHECK(kernels == (SDA_KERNEL_ROW_STREAM | SDA_KERNEL_ORDER), "kernel bits %d", kernels);
    check_decode_launch(a);
  } else {
    CHECK(kernels == 0, "kernel bits %d on status %d", kernels, rc_plan);
  }
  const int rc = sda_decode(&a, nullptr);
  CHECK(rc == rc_plan, "sda_decode_kernels status %d, sda_decode %d", rc_plan, rc);
  CHECK(valid_status(rc), "status %d", rc);
  if (rc == SDA_OK && a.rows > 0) {
    CHECK(g_launches == before + 1, "an OK call with rows must launch once");
    check_decode_launch(a);
  } else {
    CHECK(g_launches == before, "a refused or empty call launched (rc %d)", rc);
  }
  return rc;
}

// ---- cases -----------------------------------------------------------------
static void decode_cases() {
  // The five workload shapes.
  const int shapes[][5] = {{4, 8, 1, 1, 1},     {256, 16, 4, 1, 1}, {512, 16, 2, 1, 1},
                           {1024, 8, 4, 2, 1}, {4096, 16, 4, 1, 1}, {256, 16, 4, 1, 2},
                           {16, 16, 4, 1, 16}, {3, 13, 3, 1, 40}};
  for (auto& s : shapes) {
    sda_decode_args a = base_decode(s[0], s[1], s[2], s[3], s[4]);
    CHECK(call_decode(a) == SDA_OK, "shape rows %d", s[0]);
    a.kv_dtype = SDA_KV_FP8_E4M3;
    a.c_page_stride = (int64_t)s[2] * 64 * 384;
    a.k_scale = (const float*)dev(size_t(8) << 30);
    a.v_scale = (const float*)dev((size_t(8) << 30) + 4);
    CHECK(call_decode(a) == SDA_OK, "fp8 shape rows %d", s[0]);
  }
  // Specific refusals.
  sda_decode_args a = base_decode(256, 16, 4, 1, 2);
  a.workspace_bytes -= 1;
  CHECK(call_decode(a) == SDA_ERR_WORKSPACE, "short workspace");
  a = base_decode(256, 16, 4, 1, 2);
  a.workspace = dev((size_t(7) << 30) + 8);
  CHECK(call_decode(a) == SDA_ERR_WORKSPACE, "misaligned workspace");
  a = base_decode(256, 16, 4, 1, 1);
  a.region_tokens = 24;
  CHECK(call_decode(a) == SDA_ERR_INVALID, "rt must divide block");
  a.region_tokens = 8;
  CHECK(call_decode(a) == SDA_OK, "rt 8");
  a = base_decode(256, 17, 4, 1, 1);
  CHECK(call_decode(a) == SDA_ERR_INVALID, "17 heads");
  a = base_decode(255, 16, 4, 1, 1);
  CHECK(call_decode(a) == SDA_ERR_INVALID, "rows must be a multiple of groups * query_len");
  a = base_decode(0, 16, 4, 1, 1);
  CHECK(call_decode(a) == SDA_OK, "zero rows");
  a = base_decode(256, 16, 4, 1, 1);
  a.kv_dtype = SDA_KV_FP8_E4M3;
  CHECK(call_decode(a) == SDA_ERR_INVALID, "fp8 without scales");
  a = base_decode(256, 16, 4, 1, 1);
  a.c_token_stride = 1 << 29;
  CHECK(call_decode(a) == SDA_ERR_UNSUPPORTED, "32-bit in-page offsets");

  // Randomised arguments: every field perturbed, sometimes to extremes.
  std::mt19937_64 rng(12345);
  auto pick = [&](int64_t lo, int64_t hi) {
    return std::uniform_int_distribution<int64_t>(lo, hi)(rng);
  };
  const int64_t extremes[] = {0, 1, -1, 2, 7, 8, 16, 64, 192, 384, 2047, 2048, 2049, 1 << 24,
                              INT32_MAX, INT32_MIN, (int64_t)1 << 40, -((int64_t)1 << 40)};
  auto wild = [&](int64_t typical) {
    switch (pick(0, 3)) {
      case 0: return extremes[pick(0, sizeof extremes / sizeof extremes[0] - 1)];
      case 1: return typical + pick(-3, 3);
      default: return typical;
    }
  };
  for (int it = 0; it < 200000; ++it) {
    const int groups = (int)pick(1, 4), qlen = (int)pick(1, 3);
    sda_decode_args b = base_decode((int)pick(0, 64) * groups * qlen, (int)pick(1, 16), groups,
                                    qlen, (int)pick(1, 8));
    switch (pick(0, 14)) {
      case 0: b.rows = (int32_t)wild(b.rows); break;
      case 1: b.heads = (int32_t)wild(b.heads); break;
      case 2: b.groups = (int32_t)wild(b.groups); break;
      case 3: b.query_len = (int32_t)wild(b.query_len); break;
      case 4: b.block = (int32_t)wild(b.block); break;
      case 5: b.R = (int32_t)wild(b.R); break;
      case 6: b.region_tokens = (int32_t)wild(8); break;
      case 7: b.splits = (int32_t)wild(b.splits); break;
      case 8: b.q_head_stride = wild(b.q_head_stride); break;
      case 9: b.c_token_stride = wild(b.c_token_stride); break;
      case 10: b.workspace_bytes = (size_t)wild((int64_t)b.workspace_bytes); break;
      case 11: b.kv_dtype = (int32_t)wild(1); break;
      case 12: b.query = pick(0, 1) ? nullptr : dev(8); break;
      case 13: b.regions = nullptr; break;
      default: break;
    }
    if (b.splits > 0 && b.splits <= SDA_MAX_SPLITS && b.heads > 0 && b.heads <= 16 &&
        b.rows >= 0 && pick(0, 1))
      b.workspace_bytes = sda_workspace_bytes(b.rows, b.heads, b.splits);
    call_decode(b);
  }
}

static void swa_cases() {
  std::mt19937_64 rng(777);
  auto pick = [&](int64_t lo, int64_t hi) {
    return std::uniform_int_distribution<int64_t>(lo, hi)(rng);
  };
  for (int it = 0; it < 100000; ++it) {
    sda_swa_args a;
    memset(&a, 0, sizeof a);
    a.query_len = (int)pick(1, 4);
    a.tokens = (int)pick(0, 64) * a.query_len;
    a.heads = (int)pick(1, 16);
    a.groups = (int)pick(1, 4);
    a.block = 16 * (int)pick(1, 8);
    a.window = (int)pick(1, 5000);
    a.pack = (int)pick(0, 4);
    a.query = dev(0);
    a.q_token_stride = (int64_t)a.groups * a.heads * 192;
    a.q_head_stride = 192;
    a.output = dev(size_t(1) << 30);
    a.o_token_stride = a.q_token_stride;
    a.o_head_stride = 192;
    a.cache = dev(size_t(2) << 30);
    a.c_page_stride = (int64_t)a.groups * a.block * 384;
    a.c_group_stride = (int64_t)a.block * 384;
    a.c_token_stride = 384;
    a.block_table = (const int32_t*)dev(size_t(4) << 30);
    a.table_row_stride = 64;
    a.seq_lens = (const int32_t*)dev(size_t(5) << 30);
    a.scale = 0.07f;
    int pack = 0;
    a.splits = sda_swa_plan(a.tokens, a.groups, a.heads, a.query_len, 256, a.window, &pack);
    CHECK(a.splits >= 1 && a.splits <= 32 && pack >= 1 && pack <= a.query_len,
          "plan %d pack %d", a.splits, pack);
    if (pick(0, 3) == 0) a.window = (int)pick(INT32_MIN, INT32_MAX);
    if (pick(0, 3) == 0) a.splits = (int)pick(-2, 300);
    a.workspace = dev(size_t(7) << 30);
    a.workspace_bytes = sda_workspace_bytes(a.tokens * a.groups, a.heads, a.splits);
    const int before = g_launches;
    const int rc = sda_swa_decode(&a, nullptr);
    CHECK(valid_status(rc), "swa status %d", rc);
    if (rc == SDA_OK && a.tokens > 0) {
      CHECK(g_launches == before + 1, "swa launch");
      CHECK(g_last.pack >= 1 && g_last.pack * a.heads <= 16, "pack %d", g_last.pack);
      if (a.splits > 1) {
        const char* l1 = (const char*)g_last.lse +
                         (size_t)a.tokens * a.groups * a.splits * a.heads * sizeof(float);
        CHECK(l1 <= (const char*)a.workspace + a.workspace_bytes, "swa lse past workspace");
      }
    } else {
      CHECK(g_launches == before, "swa refused call launched");
    }
  }
  // the plan at extremes: no overflow, sane results
  const int vals[] = {INT32_MIN, -1, 0, 1, 2, 3, 16, 17, 4096, INT32_MAX};
  for (int t : vals)
    for (int g : vals)
      for (int h : vals)
        for (int q : vals)
          for (int w : vals) {
            int pack = -7;
            const int s = sda_swa_plan(t, g, h, q, 256, w, &pack);
            CHECK(s >= 1 && s <= 32 && pack >= 1, "plan(%d,%d,%d,%d,%d) = %d pack %d", t, g, h,
                  q, w, s, pack);
          }
}

static void select_and_logits_cases() {
  std::mt19937_64 rng(99);
  auto pick = [&](int64_t lo, int64_t hi) {
    return std::uniform_int_distribution<int64_t>(lo, hi)(rng);
  };
  for (int it = 0; it < 50000; ++it) {
    sda_select_args a;
    memset(&a, 0, sizeof a);
    a.rows = (int)pick(-2, 5000);
    a.num_regions = (int)pick(-2, 40000);
    a.topk = (int)pick(-2, 600);
    a.scores = (const float*)dev(4 * pick(0, 2));
    a.scores_row_stride = a.num_regions;
    a.current = (const int32_t*)dev(size_t(1) << 30);
    a.topk_lengths = pick(0, 1) ? nullptr : (const int32_t*)dev(size_t(2) << 30);
    a.regions = (int32_t*)dev(size_t(3) << 30);
    a.regions_row_stride = a.topk + pick(-1, 2);
    const int rc = sda_select_regions(&a, nullptr);
    CHECK(valid_status(rc), "select status %d", rc);
  }
  for (int it = 0; it < 50000; ++it) {
    sda_logits_args a;
    memset(&a, 0, sizeof a);
    a.groups = (int)pick(1, 4);
    a.query_len = (int)pick(1, 4);
    a.rows = (int)pick(0, 32) * a.groups * a.query_len + (pick(0, 9) == 0 ? 1 : 0);
    a.heads = 1 << pick(0, 5);
    a.regions_per_page = (int)pick(0, 16);
    a.num_regions = (int)pick(-1, 70000);
    a.region_tokens = (int)pick(0, 16);
    a.query = dev(16 * pick(0, 1) + pick(0, 1));
    a.q_row_stride = a.heads * 256;
    a.q_head_stride = 256;
    a.weights = (const float*)dev(size_t(1) << 30);
    a.w_row_stride = a.heads;
    a.summaries = dev(size_t(2) << 30);
    a.s_page_stride = 256 * a.regions_per_page;
    a.s_region_stride = 256;
    a.summary_scales = (const float*)dev(size_t(3) << 30);
    a.ss_page_stride = a.regions_per_page;
    a.block_table = (const int32_t*)dev(size_t(4) << 30);
    a.table_row_stride = 512;
    a.table_cols = (int)pick(-1, 600);
    a.positions = (const int32_t*)dev(size_t(5) << 30);
    a.scores = (float*)dev(size_t(6) << 30);
    a.scores_row_stride = a.num_regions + (int64_t)pick(0, 3);
    g_last_logits = sda::LogitsParams{};
    const int rc = sda_indexer_logits(&a, nullptr);
    CHECK(valid_status(rc), "logits status %d", rc);
    if (a.table_cols < 0 || a.table_cols > a.table_row_stride)
      CHECK(rc == SDA_ERR_INVALID, "table_cols %d accepted", a.table_cols);
    if (rc == SDA_OK && g_last_logits.table)
      CHECK(g_last_logits.tcols == a.table_cols, "table_cols %d passed as %d", a.table_cols,
            g_last_logits.tcols);
  }
}

static void small_function_cases() {
  for (int r = -5; r < 100000; r += 7) {
    const int s = sda_splits(r);
    CHECK(s >= 1 && s <= 32, "splits(%d) = %d", r, s);
  }
  CHECK(sda_splits(INT32_MAX) == 1 && sda_splits(INT32_MIN) == 1, "splits at extremes");
  const int vals[] = {INT32_MIN, -1, 0, 1, 16, 17, 256, 257, SDA_MAX_ROWS, INT32_MAX};
  for (int r : vals)
    for (int h : vals)
      for (int s : vals) {
        const size_t n = sda_workspace_bytes(r, h, s);
        CHECK(n % 256 == 0, "workspace bytes %zu not a multiple of 256", n);
      }
  for (int st = -10; st <= 10; ++st) CHECK(sda_status_string(st) != nullptr, "status string");
  CHECK(sda_device_compute_units(0) == 256 && sda_device_compute_units(-1) == 256 &&
            sda_device_compute_units(3) == 0,
        "device compute units");
}

int main() {
  void* m = mmap(nullptr, kDevBytes, PROT_NONE, MAP_PRIVATE | MAP_ANONYMOUS | MAP_NORESERVE, -1,
                 0);
  if (m == MAP_FAILED) {
    perror("mmap");
    return 2;
  }
  g_dev = (char*)m;
  small_function_cases();
  decode_cases();
  swa_cases();
  select_and_logits_cases();
  munmap(m, kDevBytes);
  if (g_fail) {
    fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  printf("sda_api_check: ok (%d launches recorded)\n", g_launches);
  return 0;
}
