// Decode indexer logits for gfx950 (MI355X): a score for every region of a
// row's request, the input of the region selection.  The operation is
// `decode_logits` on the page "vllm.models.step5.nvidia.flashinfer_sparse";
// its kernels are not shown, and the formula here is the reading
//     score[r, j] = sum_h w[r,h] * max(0, s_j * q[r,h] . k_j)
// with e4m3 queries q [rows, heads, 256], fp32 head weights w, and region
// j's e4m3 summary k_j (256 bytes beside the KV in the page holding the
// region's tokens) with its fp32 scale s_j.  Columns past the row's own
// region (position / region_tokens) are -inf.
//
// One 256-thread workgroup per (request, chunk of 256 regions).  The columns
// of the contraction are the request's rows x heads (<= 64): all its query
// tokens and KV groups score against the same summaries, so each summary is
// read once per request.
//  * Setup: the columns' queries are converted exactly to bf16 (e4m3 is a
//    subset of bf16) into LDS, with their weights; each row's region count.
//  * Each wave takes 16-region tiles round-robin: lane (i, g) loads bytes
//    [64g, 64g+64) of region i's summary (16-byte loads), converts them to
//    bf16, and for every 16-column tile runs 8 v_mfma_f32_16x16x32_bf16 with
//    the query columns (the same 64 dims per lane on both sides, so the dim
//    order inside the MFMA is immaterial).  Products are exact, sums fp32.
//  * Epilogue per tile: max(0, s_j * dot) * w, summed over a row's heads
//    with lane shuffles, masked to -inf past the row's last region, stored as
//    16 bytes per lane.  Regions past the request's last are never read.
// The bytes are the summaries (+ scales) of each request's regions, the
// queries, and the fp32 score matrix written.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sda_launch.h"

namespace sda {
namespace {

constexpr int kLgThreads = 256;
constexpr int kLgWaves = kLgThreads / 64;
constexpr int kLgChunk = 256;     // regions per workgroup
constexpr int kLgTile = 16;       // regions per MFMA tile
constexpr int kLgMaxCols = 64;    // rows x heads per request
constexpr int kLgQPitch = 72;     // bf16 per (column tile, lane) entry in LDS: 64 + 8 pad

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16 e4m3 bytes -> 16 bf16 (exact), as two 8-element MFMA operands.
__device__ __forceinline__ void e4m3x16_to_bf16(const u32x4 w, bf16x8& lo, bf16x8& hi) {
  uint32_t o[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[q], 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[q], 1.0f, true);
    o[2 * q] = __builtin_bit_cast(uint32_t, a);
    o[2 * q + 1] = __builtin_bit_cast(uint32_t, b);
  }
  lo = __builtin_bit_cast(bf16x8, u32x4{o[0], o[1], o[2], o[3]});
  hi = __builtin_bit_cast(bf16x8, u32x4{o[4], o[5], o[6], o[7]});
}

__global__ __launch_bounds__(kLgThreads) void logits_kernel(const LogitsParams p) {
  const int req = blockIdx.x;
  const int chunk = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, g4 = lane >> 4;
  __shared__ __attribute__((aligned(16))) __bf16 s_q[kLgMaxCols / 16][64][kLgQPitch];
  __shared__ float s_w[kLgMaxCols];
  __shared__ int s_len[kLgMaxCols];

  const int rpr = p.rows_per_req;
  const int r0 = req * rpr;
  const int ncols = rpr * p.heads;
  const int ntiles = (ncols + 15) / 16;

  // Region count of each row of the request (and, once, current / lengths).
  for (int t = tid; t < rpr; t += kLgThreads) {
    const int pos = p.positions[r0 + t];
    const int cur = pos < 0 ? -1 : pos / p.rt;
    const int len = cur + 1 < p.S ? cur + 1 : p.S;
    s_len[t] = len;
    if (chunk == 0) {
      if (p.current) p.current[r0 + t] = cur;
      if (p.lengths) p.lengths[r0 + t] = len;
    }
  }
  // Query columns as bf16, in the lane order of the MFMA B operand: entry
  // (tile, lane) holds column 16 tile + (lane & 15), dims [64 (lane >> 4), +64).
  for (int e = tid; e < ntiles * 64; e += kLgThreads) {
    const int t = e >> 6, l = e & 63;
    const int col = 16 * t + (l & 15);
    __bf16* dst = &s_q[t][l][0];
    if (col < ncols) {
      const int row = r0 + (col >> p.hshift);
      const int h = col & (p.heads - 1);
      const uint8_t* src = p.q + (int64_t)row * p.qrs + (int64_t)h * p.qhs + 64 * (l >> 4);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bf16x8 lo, hi;
        e4m3x16_to_bf16(*reinterpret_cast<const u32x4*>(src + 16 * c), lo, hi);
        *reinterpret_cast<bf16x8*>(dst + 16 * c) = lo;
        *reinterpret_cast<bf16x8*>(dst + 16 * c + 8) = hi;
      }
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) *reinterpret_cast<u32x4*>(dst + 8 * c) = u32x4{0, 0, 0, 0};
    }
  }
  for (int c = tid; c < kLgMaxCols; c += kLgThreads)
    s_w[c] = c < ncols ? p.w[(int64_t)(r0 + (c >> p.hshift)) * p.wrs + (c & (p.heads - 1))] : 0.f;
  __syncthreads();

  int max_len = 0;
  for (int t = 0; t < rpr; ++t) max_len = max(max_len, s_len[t]);

  const int j_begin = chunk * kLgChunk;
  for (int tile = wave; tile < kLgChunk / kLgTile; tile += kLgWaves) {
    const int j0 = j_begin + kLgTile * tile;
    if (j0 >= p.S) break;
    if (j0 >= max_len) {
      // Past every row's last region: -inf, and no summary read.
      for (int e = lane; e < rpr * kLgTile; e += 64) {
        const int row = e / kLgTile, j = j0 + (e - row * kLgTile);
        if (j < p.S) p.out[(int64_t)(r0 + row) * p.ors + j] = -INFINITY;
      }
      continue;
    }
    // A operand: region j0 + i16 (clamped into the request's regions for the
    // load; masked below), bytes [64 g4, +64) as 8 bf16x8 k-slices.
    const int ja = min(j0 + i16, max_len - 1);
    const int64_t pa = p.table[(int64_t)req * p.trs + ja / p.rpb];
    const uint8_t* asrc = p.sm + pa * p.sps + (int64_t)(ja % p.rpb) * p.sms + 64 * g4;
    u32x4 raw[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) raw[c] = *reinterpret_cast<const u32x4*>(asrc + 16 * c);
    // scales of this lane's C rows: regions j0 + 4 g4 + v
    float sc[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int jc = min(j0 + 4 * g4 + v, max_len - 1);
      const int64_t pc = p.table[(int64_t)req * p.trs + jc / p.rpb];
      sc[v] = p.sc[pc * p.scps + jc % p.rpb];
    }
    bf16x8 a[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) e4m3x16_to_bf16(raw[c], a[2 * c], a[2 * c + 1]);

    for (int ct = 0; ct < ntiles; ++ct) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const __bf16* bq = &s_q[ct][lane][0];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(bq + 8 * s);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], b, acc, 0, 0, 0);
      }
      // lane holds S[region j0 + 4 g4 + v][column 16 ct + i16]
      const int col = 16 * ct + i16;
      const float wc = s_w[col < kLgMaxCols ? col : 0];
      float x[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) x[v] = fmaxf(0.f, sc[v] * acc[v]) * (col < ncols ? wc : 0.f);
      // sum over the row's heads: `heads` consecutive lanes of the 16-lane group
      for (int d = 1; d < p.heads; d <<= 1)
#pragma unroll
        for (int v = 0; v < 4; ++v) x[v] += __shfl_xor(x[v], d);
      if (col < ncols && (col & (p.heads - 1)) == 0) {
        const int rowi = col >> p.hshift;
        const int len = s_len[rowi];
        const int jb = j0 + 4 * g4;
        float* dst = p.out + (int64_t)(r0 + rowi) * p.ors + jb;
        float y[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) y[v] = jb + v < len ? x[v] : -INFINITY;
        if (jb + 3 < p.S) {
          *reinterpret_cast<float4*>(dst) = make_float4(y[0], y[1], y[2], y[3]);
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (jb + v < p.S) dst[v] = y[v];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_logits(const LogitsParams& p, hipStream_t stream) {
  const unsigned chunks = (unsigned)((p.S + kLgChunk - 1) / kLgChunk);
  hipLaunchKernelGGL(logits_kernel, dim3((unsigned)(p.rows / p.rows_per_req), chunks),
                     dim3(kLgThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sda
