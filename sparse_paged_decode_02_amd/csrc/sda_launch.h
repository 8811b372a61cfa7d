// Internal interface between the C-ABI layer (sda_api.cpp) and the kernels
// (sda_kernels.hip): the validated, kernel-ready argument block.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace sda {

constexpr int kMaxRegions = 2048;  // LDS region list per workgroup (= SDA_MAX_R)

struct Params {
  // Row r is group r % groups of token r / groups; its head h sits at
  // q + (r / groups) * qts + (r % groups) * qgs + h * qhs (likewise out).
  const uint16_t* q;          // bf16 bits
  int64_t qts, qgs, qhs;      // query token / group / head strides (elements)
  uint16_t* out;              // bf16 bits
  int64_t ots, ogs, ohs;
  const uint8_t* cache;       // byte view of the cache
  int64_t cps, cgs, cts;      // cache page / group / token strides (elements)
  const int32_t* regions;
  int64_t rrs;
  const int32_t* table;
  int64_t trs;
  const int32_t* positions;   // sparse: [rows]
  const uint8_t* active;      // sparse: [rows]; null means every row is active
  const int32_t* seq_lens;    // window: [requests]
  const float* k_scale;
  const float* v_scale;
  const uint16_t* gate;       // bf16 bits or null
  int64_t grs, ghs;
  const int32_t* order;       // sparse: workgroup x serves row order[x]; null: row x
  int32_t* order_ws;          // sparse: [2 * rows] scratch for the order and the row
                              // bins, or null (index order)
  float* partial;             // [rows, splits, heads, 192] fp32 (splits > 1)
  float* lse;                 // [rows, splits, heads] fp32, base-2 (splits > 1)
  float scale;
  int32_t rows, heads, groups, rows_per_req, block, R, rt, splits, clear, gated;
  int32_t rt_shift;           // log2(rt) when rt is a power of two, else -1
  int32_t query_len, window;  // window mode
  int32_t pack, ntg;          // window mode: tokens per workgroup, token groups per request
  int32_t nt_out;             // set by the launch: store the output non-temporally
  int32_t wide_out;           // set by the launch: 16-byte aligned output, 8 dims per store
  int32_t cus;                // compute units of the device the call runs on
};

// Enqueue the split kernel (and the combine kernel when splits > 1) over
// region lists (sparse decode).  When order_ws is set and the grid takes 2 to
// 4 rounds of the workgroups the chip holds at once, two small kernels first
// write a heaviest-first row order there (rows ranked by visible tokens
// within each block of 1024 rows), and the split kernel follows it.
hipError_t launch(const Params& p, bool fp8, hipStream_t stream);

// The kernels `launch` enqueues for these parameters (kPlan* bits), without
// launching anything.  For grids of at least two rows per resident wave and
// short region lists (splits == 1, 16-byte aligned output) the split kernel
// gives way to the row-stream kernel: one workgroup per CU whose waves take
// whole rows back to back.
constexpr int kPlanOrder = 1, kPlanSplit = 2, kPlanRowStream = 4, kPlanCombine = 8;
int plan(const Params& p);

// The same kernels over each row's sliding window (bf16 cache): token j of a
// request of length L sits at position L - query_len + j and attends over
// positions max(0, pos - window + 1) .. pos.  One split workgroup serves
// `pack` consecutive tokens of a request and KV group (pack * heads <= 16).
// Requires block % 16 == 0.
hipError_t launch_window(const Params& p, hipStream_t stream);

// Region selection (sda_select.hip).
struct SelParams {
  const float* scores;        // [rows, S]
  int64_t srs;
  const int32_t* current;     // [rows]
  const int32_t* lengths;     // [rows] or null (all S columns are candidates)
  int32_t* out;               // [rows, topk]
  int64_t ors;
  int32_t rows, S, topk;
  int32_t cus;                // compute units of the device the call runs on
};

hipError_t launch_select(const SelParams& p, hipStream_t stream);

// Decode indexer logits (sda_logits.hip).
struct LogitsParams {
  const uint8_t* q;           // e4m3 [rows, heads, 256]
  int64_t qrs, qhs;           // bytes
  const float* w;             // [rows, heads]
  int64_t wrs;
  const uint8_t* sm;          // e4m3 summaries [pages, rpb, 256]
  int64_t sps, sms;           // page / region strides (bytes)
  const float* sc;            // [pages, rpb]
  int64_t scps;               // page stride (elements)
  const int32_t* table;
  int64_t trs;
  const int32_t* positions;
  float* out;                 // [rows, S]
  int64_t ors;
  int32_t* current;           // [rows] or null
  int32_t* lengths;           // [rows] or null
  int32_t rows, heads, hshift, rows_per_req, rpb, S, rt;
  // Last, so that the fields above keep their kernel-argument offsets (the
  // setup's scalar loads of them batch as they did before this field).
  int32_t tcols;              // table columns (0: unknown, read scored columns only)
};

hipError_t launch_logits(const LogitsParams& p, hipStream_t stream);

}  // namespace sda
