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
//    [64c + 16g, +16), c = 0..3, of region i's summary (16-byte loads: each
//    instruction reads 64 contiguous bytes of 16 regions), converts them to
//    bf16, and for every 16-column tile runs 8 v_mfma_f32_16x16x32_bf16 with
//    the query columns as the A rows and the regions as the B columns (the
//    same 64 dims per lane on both sides, so the dim order inside the MFMA
//    is immaterial).  Products are exact, sums fp32.
//  * Epilogue per tile: a lane holds four consecutive columns (heads) of one
//    region; max(0, s_j * dot) * w, summed over a row's heads in the lane
//    and across lanes 16 and 32 apart (permlane swaps), masked to -inf past
//    the row's last region, stored 4 bytes per lane (16 lanes: 64
//    contiguous bytes of a row).  Regions past the request's last are never
//    read.  The kernel is instantiated per head count (1..16).
// The bytes are the summaries (+ scales) of each request's regions, the
// queries, and the fp32 score matrix written.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sda_launch.h"
#include "sda_wave.h"

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

// x plus x of the lane kDist (16 or 32) away, in every lane: the permlane
// swap exchanges the two halves of each 32-lane (or the 64-lane) group
// between its two operands, so with x in both the two results are x and the
// partner's x in some order, and their sum is the same in both lanes.
template <int kDist>
__device__ __forceinline__ float add_across(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = kDist == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                             : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// kEarly: the table's column count is known (p.tcols > 0).
template <int kHeads, bool kEarly>
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

  // Loads that depend on nothing else go first: the positions, the query
  // columns (entry = thread: column tile tid >> 6, lane tid & 63), the head
  // weights and (below) the block-table entries.  Each is issued by every
  // lane at an index clamped into range and masked afterwards: with no branch
  // around them they all go out in one round trip, behind one batch of
  // kernel-argument loads.
  static_assert(kLgThreads == (kLgMaxCols / 16) * 64, "one query entry per thread");
  const int qt = tid >> 6, ql = tid & 63;
  const int qcol = 16 * qt + (ql & 15);
  const bool qvalid = qt < ntiles && qcol < ncols;
  u32x4 qraw[4];
  {
    const int qc = qvalid ? qcol : 0;
    const int row = r0 + (qc >> p.hshift);
    const int h = qc & (p.heads - 1);
    const uint8_t* src = p.q + (int64_t)row * p.qrs + (int64_t)h * p.qhs + 16 * (ql >> 4);
#pragma unroll
    for (int c = 0; c < 4; ++c) qraw[c] = *reinterpret_cast<const u32x4*>(src + 64 * c);
  }
  static_assert(kLgMaxCols <= kLgThreads, "one weight per thread");
  const int wc = tid < ncols ? tid : 0;
  float wv = p.w[(int64_t)(r0 + (wc >> p.hshift)) * p.wrs + (wc & (p.heads - 1))];

  // With the table's column count known, each lane requests the block-table
  // entry of one region of its wave's tiles now, beside the positions (an
  // entry past the scored regions is read but not used); otherwise only
  // once the positions show which regions are scored.
  const int j_begin = chunk * kLgChunk;
  const int j_end = min(p.S, j_begin + kLgChunk);
  // This wave's tiles start at j_begin + 16 wave + 64 t (t = 0..3).  Lane l
  // resolves region j_begin + 16 wave + 64 (l >> 4) + (l & 15): its summary
  // row offset and scale, shared with the MFMA lanes by shuffles, so the
  // tile loop issues summary loads only.
  const int jl = j_begin + kLgTile * wave + kLgTile * kLgWaves * (lane >> 4) + (lane & 15);
  int pg_raw = 0;
  if (kEarly) {
    // regions whose column lies in the table (below tcols * rpb >= 1)
    const int j_tab = (int)min((int64_t)j_end, (int64_t)p.tcols * p.rpb);
    pg_raw = p.table[(int64_t)req * p.trs + min(jl, j_tab - 1) / p.rpb];
  }

  // Region count of each row (lane t < rpr: row t) and the request's maximum
  // (every wave reduces it itself).
  const int pos = p.positions[r0 + (lane < rpr ? lane : 0)];
  int lenv = 0, cur = -1;
  if (lane < rpr) {
    cur = pos < 0 ? -1 : pos / p.rt;
    lenv = cur + 1 < p.S ? cur + 1 : p.S;
    if (wave == 0) s_len[lane] = lenv;
  }
  const int max_len = wave_max(lenv);
  // The queries and weights were requested before the positions, so they
  // have landed: consume them here, where the wait for the positions
  // covers them, rather than behind the block-table loads below.
  __asm__ __volatile__("" : "+v"(wv), "+v"(qraw[0]), "+v"(qraw[1]), "+v"(qraw[2]), "+v"(qraw[3]));
  if (!qvalid) qraw[0] = qraw[1] = qraw[2] = qraw[3] = u32x4{0u, 0u, 0u, 0u};  // absent columns
  if (tid >= ncols) wv = 0.f;

  const int j_live = min(j_end, max_len);
  if (!kEarly && jl < j_live) pg_raw = p.table[(int64_t)req * p.trs + jl / p.rpb];
  const int64_t pg = jl < j_live ? pg_raw : 0;
  // The query conversion below overlaps the block-table round trip when the
  // entries are requested only now.
  // Query columns converted to bf16 in the lane order of the MFMA B
  // operand: entry (tile, lane) holds column 16 tile + (lane & 15), dims
  // [64 c + 16 (lane >> 4), +16) for c = 0..3, the dims its A lanes hold.
  if (qt < ntiles) {
    __bf16* dst = &s_q[qt][ql][0];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8 lo, hi;
      e4m3x16_to_bf16(qraw[c], lo, hi);  // zeros for absent columns
      *reinterpret_cast<bf16x8*>(dst + 16 * c) = lo;
      *reinterpret_cast<bf16x8*>(dst + 16 * c + 8) = hi;
    }
  }
  if (tid < kLgMaxCols) s_w[tid] = wv;
  int64_t roff_l = 0;
  float scale_l = 0.f;
  if (jl < j_live) {
    roff_l = pg * p.sps + (int64_t)(jl % p.rpb) * p.sms;
    scale_l = p.sc[pg * p.scps + jl % p.rpb];
  }
  // A operand of tile t: region j0 + i16 (a region past j_live is masked;
  // its lane borrows the tile's first region, always live), bytes
  // [64 c + 16 g4, +16) for c = 0..3, so that each load instruction reads
  // 64 contiguous bytes of each of the 16 regions.
  auto load_tile = [&](int t, u32x4 (&raw)[4]) {
    const int src = kLgTile * t + i16;
    const int j = j_begin + kLgTile * wave + kLgTile * kLgWaves * t + i16;
    const int64_t off = __shfl(roff_l, j < j_live ? src : kLgTile * t);
    const uint8_t* a = p.sm + off + 16 * g4;
#pragma unroll
    for (int c = 0; c < 4; ++c) raw[c] = *reinterpret_cast<const u32x4*>(a + 64 * c);
  };
  const int nt = (j_live - (j_begin + kLgTile * wave) + kLgTile * kLgWaves - 1) /
                 (kLgTile * kLgWaves);  // live tiles of this wave (<= 4)
  // The first tile's summaries are requested before the barrier, as soon as
  // their offsets are known.
  u32x4 raw[4];
  if (nt > 0) load_tile(0, raw);

  // The barrier publishes LDS only (queries, weights, region counts): each
  // wave waits for its own LDS writes, not for its global loads in flight,
  // which a full __syncthreads() fence would also drain.
  __asm__ __volatile__("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // The selection's inputs, once per row, stored after the loads above are
  // on their way (a store in flight would hold up the first wait).
  if (chunk == 0 && wave == 0 && lane < rpr) {
    if (p.current) p.current[r0 + lane] = cur;
    if (p.lengths) p.lengths[r0 + lane] = lenv;
  }

  // Tiles at or past the request's last region: -inf, and no summary read.
  for (int j0 = j_begin + kLgTile * wave; j0 < j_end; j0 += kLgTile * kLgWaves) {
    if (j0 < j_live) continue;
    for (int e = lane; e < rpr * kLgTile; e += 64) {
      const int row = e / kLgTile, j = j0 + (e - row * kLgTile);
      if (j < p.S) p.out[(int64_t)(r0 + row) * p.ors + j] = -INFINITY;
    }
  }
  if (nt > 0) {
    // Everything a tile's epilogue needs beyond its accumulators is fixed for
    // the workgroup or known now: the weights of this lane's columns, the
    // lengths of the rows it stores (LDS), and every tile's summary offsets
    // and this lane's region scale (from the lanes that resolved them).
    // Fetched once here, they keep LDS round trips out of the tile loop.
    constexpr int kHpl = kHeads < 4 ? kHeads : 4;  // a row's heads within a lane
    constexpr int kRpl = 4 / kHpl;                  // rows per lane and column tile
    float wq[kLgMaxCols / 16][4];
    int lrow[kLgMaxCols / 16][kRpl];
#pragma unroll
    for (int ct = 0; ct < kLgMaxCols / 16; ++ct) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int col = 16 * ct + 4 * g4 + v;
        wq[ct][v] = col < ncols ? s_w[col] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < kRpl; ++q) {
        const int col = 16 * ct + 4 * g4 + q * kHpl;
        lrow[ct][q] = col < ncols ? s_len[col / kHeads] : 0;
      }
    }
    int64_t toff[4];
    float tsc[4];
#pragma unroll
    for (int t = 1; t < 4; ++t) {
      const int j = j_begin + kLgTile * wave + kLgTile * kLgWaves * t + i16;
      toff[t] = __shfl(roff_l, j < j_live ? kLgTile * t + i16 : kLgTile * t);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) tsc[t] = __shfl(scale_l, kLgTile * t + i16);
    toff[0] = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t >= nt) break;
      const int j0 = j_begin + kLgTile * wave + kLgTile * kLgWaves * t;
      bf16x8 a[8];
#pragma unroll
      for (int c = 0; c < 4; ++c) e4m3x16_to_bf16(raw[c], a[2 * c], a[2 * c + 1]);
      if (t + 1 < nt) {  // next tile in flight
        const uint8_t* an = p.sm + toff[t + 1 < 4 ? t + 1 : 3] + 16 * g4;
#pragma unroll
        for (int c = 0; c < 4; ++c) raw[c] = *reinterpret_cast<const u32x4*>(an + 64 * c);
      }
      const int j = j0 + i16;  // this lane's region

#pragma unroll
      for (int ct = 0; ct < kLgMaxCols / 16; ++ct) {
        if (ct >= ntiles) break;
        // The query columns are the MFMA's A rows and the regions its B
        // columns, so a lane ends up with four consecutive columns (heads)
        // of one region: S[column 16 ct + 4 g4 + v][region j0 + i16].
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const __bf16* bq = &s_q[ct][lane][0];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(bq + 8 * s);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, a[s], acc, 0, 0, 0);
        }
        float x[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) x[v] = fmaxf(0.f, tsc[t] * acc[v]) * wq[ct][v];
        // a row's heads: kHpl in the lane, then the lanes 16 and 32 apart
        float y[kRpl];
#pragma unroll
        for (int q = 0; q < kRpl; ++q) {
          y[q] = x[q * kHpl];
#pragma unroll
          for (int v = 1; v < kHpl; ++v) y[q] += x[q * kHpl + v];
        }
        if (kHeads >= 8) y[0] = add_across<16>(y[0]);
        if (kHeads >= 16) y[0] = add_across<32>(y[0]);
        if (j < p.S && (kHeads < 8 || ((4 * g4) & (kHeads - 1)) == 0)) {
#pragma unroll
          for (int q = 0; q < kRpl; ++q) {
            const int col = 16 * ct + 4 * g4 + q * kHpl;
            if (col < ncols)
              p.out[(int64_t)(r0 + col / kHeads) * p.ors + j] = j < lrow[ct][q] ? y[q] : -INFINITY;
          }
        }
      }
    }
  }
}

template <bool kEarly>
void launch_heads(const LogitsParams& p, dim3 grid, hipStream_t stream) {
  const dim3 block(kLgThreads);
  switch (p.heads) {
    case 1:
      hipLaunchKernelGGL((logits_kernel<1, kEarly>), grid, block, 0, stream, p);
      break;
    case 2:
      hipLaunchKernelGGL((logits_kernel<2, kEarly>), grid, block, 0, stream, p);
      break;
    case 4:
      hipLaunchKernelGGL((logits_kernel<4, kEarly>), grid, block, 0, stream, p);
      break;
    case 8:
      hipLaunchKernelGGL((logits_kernel<8, kEarly>), grid, block, 0, stream, p);
      break;
    default:  // 16 (the call validates a power of two <= 16)
      hipLaunchKernelGGL((logits_kernel<16, kEarly>), grid, block, 0, stream, p);
      break;
  }
}

}  // namespace

hipError_t launch_logits(const LogitsParams& p, hipStream_t stream) {
  const unsigned chunks = (unsigned)((p.S + kLgChunk - 1) / kLgChunk);
  const dim3 grid((unsigned)(p.rows / p.rows_per_req), chunks);
  if (p.tcols > 0)
    launch_heads<true>(p, grid, stream);
  else
    launch_heads<false>(p, grid, stream);
  return hipGetLastError();
}

}  // namespace sda
