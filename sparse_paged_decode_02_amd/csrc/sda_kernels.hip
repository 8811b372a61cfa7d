// DSA sparse decode attention kernels for gfx950 (MI355X).
//
// The operation is the one the page "vllm.models.step5.nvidia.ops.
// sparse_decode_attention" describes in its module docstring and in its
// `sparse_decode_attention` and `_gate` sections.  Each (token, KV group) row
// packs up to 16 query heads of dim 192, and each row attends over the
// tokens of its selected regions.  Those tokens are read in place from a paged
// [pages, G, block, 384] K|V cache, masked causally at the row's position,
// and dequantized from FP8 with per-tensor scales.  Split partials are merged
// by log-sum-exp.  After the merge come the headwise sigmoid gate and the
// inactive-row clear.
//
// Split kernel: one workgroup per (row, split), 4 waves of 64 (one workgroup
// per CU) or, for grids of at least two workgroups per CU, 2 waves (two per
// CU).
//  * Prologue, per wave and without workgroup barriers: rank the row's
//    visible region slots with ballots, take the split's balanced share, and
//    resolve each region to a cache offset through the block table (only the
//    share's entries are read).  The list goes into LDS.  A sliding-window
//    row instead resolves the pages of its contiguous token window.
//  * Addressing: a chunk's 12 DMAs take their rows from per-lane 64-bit
//    addresses when a chunk may straddle regions, from one scalar base when
//    every chunk lies inside one region (or one window page), from two
//    scalar bases when regions of half a chunk (8 bf16 or 16 FP8 tokens)
//    pair up into a chunk, and from four (two DMAs per chunk with per-lane
//    addresses) when FP8 regions of 8 tokens go four to a chunk.
//  * Main loop: every wave runs its own 2-stage pipeline over chunks of token
//    slots (16 tokens for a bf16 cache, 32 for FP8: 6 KiB of K and 6 KiB of
//    V either way).  A chunk is 12 LDS-DMAs (global_load_lds_dwordx4) into a
//    wave-private stage.  They are issued from inline assembly and marked
//    non-temporal (the bytes are read once), and their completion is awaited
//    with an explicit vmcnt.  The next chunk of the wave is in flight while
//    the current one is computed:
//      S^T[tok, head] = K[tok, :] . Q^T[:, head]   v_mfma_f32_16x16x32_bf16
//      online softmax per head, in the exp2 domain, with lazy rescaling
//      O^T[dim, head] += V^T[dim, tok] . P^T[tok, head]
//    V^T comes from transposing LDS reads (ds_read_b64_tr_b16 for bf16,
//    ds_read_b64_tr_b8 for FP8).  P^T is the S^T accumulator itself,
//    because the C layout of S^T is the B-operand layout of the second
//    product.  bf16 uses v_mfma_f32_16x16x16_bf16 for P.V; FP8 uses the x32
//    form.  FP8 K and V are converted exactly to bf16 (e4m3 is a subset of
//    bf16).  k_scale is folded into the logit scale and v_scale into the
//    final normalisation.
//  * Epilogue: the waves' (max, sum, acc) states are merged through LDS:
//    16 lanes turn the per-wave maxima and sums into one weight per (wave,
//    head) that already holds v_scale, 1/sum and, with one split, the gate,
//    and the output is the weighted sum of the wave accumulators, written
//    as bf16 (combine fused).  Otherwise the fp32 partial output and its base-2
//    log-sum-exp go to the workspace.
// Combine kernel (splits > 1): one 64-thread workgroup per (row, head) merges
// the partials, applies the gate and writes bf16, or clears an inactive row.
// Row-stream kernel (one split, large batches of short region lists): one
// 4-wave workgroup per CU, each wave streaming whole rows back to back
// through the same chunk pipeline and arithmetic, with no cross-wave merge.
// Bin and order kernels (grids of 2 to 4 rounds of resident workgroups,
// given a workspace): rank the rows by visible tokens so that the split
// kernel starts the heaviest first.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "sda_dma.h"
#include "sda_launch.h"
#include "sda_wave.h"


namespace sda {
namespace {

// Waves per split workgroup: 4 (one workgroup per CU, ~121 KiB of LDS) when
// the grid is at most one workgroup per CU, else 2 (~72 KiB, two per CU, so
// that one workgroup's prologue and epilogue overlap the other's streaming).
constexpr int kWavesSmallGrid = 4;
constexpr int kWavesLargeGrid = 2;
constexpr int kStages = 2;          // LDS stages per wave: 1 computed, 1 in flight
constexpr int kSlotBatch = 8;       // 64-slot groups of a region list loaded together
constexpr int kAccStride = 196;     // floats per head row in the wave-merge area

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

// How a split finds the cache rows of its token slots.
enum Addr : int {
  kGeneral = 0,  // region list; a chunk may span regions (per-lane 64-bit addresses)
  kUniform = 1,  // region list; every chunk lies inside one region
  kWindow = 2,   // a contiguous sliding window of tokens, 16-token chunks
  kPair = 3,     // region list of half-chunk regions (8 tokens bf16, 16 FP8): two per chunk
  kQuad = 4,     // region list of 8-token regions, FP8: a chunk is four regions
};


__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Headwise sigmoid gate of the `_gate` section: the bf16 logit widened to fp32,
// 1 / (1 + exp(-g)) with a correctly rounded fp32 division (this file is built
// with -fhip-fp32-correctly-rounded-divide-sqrt), rounded to bf16, widened.
__device__ __forceinline__ float gate_sigmoid(uint32_t bits) {
  float g = bf16_bits_to_float(bits);
  float den = 1.0f + expf(-g);
  float sig = 1.0f / den;
  return bf16_bits_to_float(float_to_bf16_bits(sig));
}

__device__ __forceinline__ float gate_value(const uint16_t* gate, int64_t idx) {
  return gate_sigmoid(gate[idx]);
}

// 4 e4m3 bytes -> 4 bf16 (exact), as two packed pairs {bytes 0,1} {bytes 2,3}.
__device__ __forceinline__ u32x2 fp8x4_to_bf16(uint32_t w) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
}

// Where token slot `slot` of a split lives (general addressing: a chunk may
// span regions).  A masked slot is redirected to the first token of a region
// of the split (always visible), so every load stays in bounds and every V
// row in LDS is finite data whose weight is exactly 0.
__device__ __forceinline__ int64_t token_elem(const Params& p, int slot, const int64_t* s_base,
                                              const int* s_n, int nreg, bool& valid) {
  // region_tokens is almost always a power of two: shift, not divide
  const int k = p.rt_shift >= 0 ? slot >> p.rt_shift : slot / p.rt;
  const int off = slot - k * p.rt;
  int kk = k < nreg ? k : nreg - 1;
  valid = k < nreg && off < s_n[kk];
  return s_base[kk] + (int64_t)(valid ? off : 0) * p.cts;
}

// A split's sliding window: w0..pos is the union of the windows of the
// workgroup's query tokens; chunk c starts at token t_base + 16c; s_base[k]
// is the cache offset of block-table column col_lo + k (page and KV group).
struct Win {
  int w0, pos, t_base, col_lo;
};

// Issue chunk c into LDS stage `stage`.  Returns the visibility of this
// lane's S^T rows (bit t: token slot 16t + i16).  Masked slots load a visible
// token of the same chunk instead (in bounds, finite, weight 0): the first
// token of their region, or the nearest window token.
template <bool kFp8, int kAddr>
__device__ __forceinline__ uint32_t issue_chunk(const Params& p, int c, int nreg,
                                                const int64_t* s_base, const int* s_n, int lane,
                                                uint32_t stage, const LaneDma& ld,
                                                uint32_t cts_bytes, const Win& win) {
  using C = Cfg<kFp8>;
  const uint32_t st = (uint32_t)__builtin_amdgcn_readfirstlane(stage);
  uint32_t vbits = 0;
  if (kAddr == kWindow) {
    // 16 consecutive tokens of one page (block is a multiple of 16): uniform
    // base at the chunk's first token, 32-bit lane offsets.
    static_assert(!kFp8 || kAddr != kWindow, "window chunks are 16 bf16 tokens");
    const int t0 = win.t_base + 16 * c;
    const int col = t0 / p.block;
    const int64_t rb = s_base[col - win.col_lo] + (int64_t)(t0 - col * p.block) * p.cts;
    const uint8_t* base = uniform_ptr(p.cache + rb * C::kEsz);
    uint32_t ko[6], vo[6];
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      const int tc = min(max(t0 + ld.row[j], win.w0), win.pos);
      const uint32_t roff = (uint32_t)(tc - t0) * cts_bytes;
      ko[j] = roff + ld.koff[j];
      vo[j] = roff + ld.voff[j];
    }
    dma_chunk_sbase<kFp8>(base, st, ko, vo);
  } else if (kAddr == kPair) {
    // Regions of half a chunk (8 tokens bf16, 16 tokens FP8): chunk c is
    // regions 2c and 2c+1 of the list, each with a uniform base.  Rows past a
    // region's visible count load that region's token 0, and the second half
    // when the list has no region 2c+1 loads token 0 of region 2c (visible,
    // finite, weight 0).
    constexpr int kHalf = C::kTok / 2;
    const int i16 = lane & 15;
    const int k0 = 2 * c;
    const bool has1 = k0 + 1 < nreg;
    const int n0 = __builtin_amdgcn_readfirstlane(s_n[k0]);
    const int n1 = has1 ? __builtin_amdgcn_readfirstlane(s_n[k0 + 1]) : 0;
    const int64_t rb0 = s_base[k0];
    const int64_t rb1 = has1 ? s_base[k0 + 1] : rb0;
    const uint8_t* base0 = uniform_ptr(p.cache + rb0 * C::kEsz);
    const uint8_t* base1 = uniform_ptr(p.cache + rb1 * C::kEsz);
    // S^T slot 16t + i16: region t (FP8), region i16 >> 3 (bf16)
    if (kFp8)
      vbits = (i16 < n0 ? 1u : 0u) | (i16 < n1 ? 2u : 0u);
    else
      vbits = (i16 < 8 ? i16 < n0 : i16 - 8 < n1) ? 1u : 0u;
    uint32_t ko[6], vo[6];
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      // token row within its region: DMAs 0..2 read region 2c, 3..5 region 2c+1
      const int rr = ld.row[j] & (kHalf - 1);
      const int nn = j < 3 ? n0 : n1;
      const uint32_t roff = rr < nn ? (uint32_t)rr * cts_bytes : 0u;
      ko[j] = roff + ld.koff[j];
      vo[j] = roff + ld.voff[j];
    }
    dma_chunk_sbase2<kFp8>(base0, base1, st, ko, vo);
  } else if (kAddr == kQuad) {
    // 8-token regions (FP8): chunk c is list entries 4c .. 4c + 3, token rows
    // 8q .. 8q + 7 of the chunk from entry 4c + q.  Rows past an entry's
    // visible count load its token 0, and entries past the list load token 0
    // of entry 4c (visible, finite, weight 0).  DMAs 0, 2, 3, 5 take one
    // region's uniform base; DMAs 1 and 4 straddle two regions at lane 32
    // (SDA_CHUNK_ASM_QUAD) and take per-lane 64-bit addresses.
    static_assert(kFp8 || kAddr != kQuad, "quad chunks are FP8");
    const int i16 = lane & 15;
    const int k0 = 4 * c;
    // Entry k0 + q's uniform base and visible count (named values, not arrays:
    // an array of pointers here was kept in scratch memory).
    auto entry_base = [&](int q) {
      return uniform_ptr(p.cache + s_base[k0 + q < nreg ? k0 + q : k0] * C::kEsz);
    };
    auto entry_n = [&](int q) {
      return k0 + q < nreg ? __builtin_amdgcn_readfirstlane(s_n[k0 + q]) : 0;
    };
    const uint8_t* const b0 = entry_base(0);
    const uint8_t* const b1 = entry_base(1);
    const uint8_t* const b2 = entry_base(2);
    const uint8_t* const b3 = entry_base(3);
    const int n0 = entry_n(0), n1 = entry_n(1), n2 = entry_n(2), n3 = entry_n(3);
    // slot 16t + i16 is row i16 & 7 of entry 2t + (i16 >> 3)
    const int r7 = i16 & 7;
    vbits = (r7 < (i16 < 8 ? n0 : n1) ? 1u : 0u) | (r7 < (i16 < 8 ? n2 : n3) ? 2u : 0u);
    auto roff = [&](int j, int n) {
      const int r8 = ld.row[j] & 7;
      return r8 < n ? (uint32_t)r8 * cts_bytes : 0u;
    };
    uint32_t ko[6], vo[6];
    // DMAs 0, 2, 3, 5: entries 0, 1, 2, 3 (quad_region)
    const uint32_t o0 = roff(0, n0), o2 = roff(2, n1), o3 = roff(3, n2), o5 = roff(5, n3);
    ko[0] = o0 + ld.koff[0];
    vo[0] = o0 + ld.voff[0];
    ko[2] = o2 + ld.koff[2];
    vo[2] = o2 + ld.voff[2];
    ko[3] = o3 + ld.koff[3];
    vo[3] = o3 + ld.voff[3];
    ko[5] = o5 + ld.koff[5];
    vo[5] = o5 + ld.voff[5];
    ko[1] = vo[1] = ko[4] = vo[4] = 0;  // unused: DMAs 1 and 4 take 64-bit addresses
    // DMAs 1 and 4: lanes 0..31 read entry 0 / 2, lanes 32..63 entry 1 / 3
    const bool hi = lane >= 32;
    const uint8_t* const l1 = (hi ? b1 : b0) + roff(1, hi ? n1 : n0);
    const uint8_t* const l4 = (hi ? b3 : b2) + roff(4, hi ? n3 : n2);
    dma_chunk_quad(b0, b1, b2, b3, st, ko, vo, l1 + ld.koff[1], l1 + ld.voff[1],
                   l4 + ld.koff[4], l4 + ld.voff[4]);
  } else if (kAddr == kUniform) {
    const int i16 = lane & 15;
    // The chunk lies inside one region: uniform base, 32-bit lane offsets.
    const int slot0 = c * C::kTok;
    const int k = slot0 / p.rt;
    const int off0 = slot0 - k * p.rt;
    const int64_t rb = s_base[k];
    const int nval = __builtin_amdgcn_readfirstlane(s_n[k]);
    const uint8_t* base = uniform_ptr(p.cache + rb * C::kEsz);
#pragma unroll
    for (int t = 0; t < (kFp8 ? 2 : 1); ++t) vbits |= (off0 + 16 * t + i16 < nval ? 1u : 0u) << t;
    uint32_t ko[6], vo[6];
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      const int tok = off0 + ld.row[j];
      const uint32_t roff = tok < nval ? (uint32_t)tok * cts_bytes : 0u;
      ko[j] = roff + ld.koff[j];
      vo[j] = roff + ld.voff[j];
    }
    dma_chunk_sbase<kFp8>(base, st, ko, vo);
  } else {
    const int i16 = lane & 15;
    const int slot0 = c * C::kTok;
#pragma unroll
    for (int t = 0; t < (kFp8 ? 2 : 1); ++t) {
      bool valid;
      (void)token_elem(p, slot0 + 16 * t + i16, s_base, s_n, nreg, valid);
      vbits |= (valid ? 1u : 0u) << t;
    }
    const uint8_t* ka[6];
    const uint8_t* va[6];
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      bool valid;
      const int64_t e = token_elem(p, slot0 + ld.row[j], s_base, s_n, nreg, valid);
      const uint8_t* row = p.cache + e * C::kEsz;
      ka[j] = row + ld.koff[j];
      va[j] = row + ld.voff[j];
    }
    dma_chunk_vaddr<kFp8>(st, ka, va);
  }
  return vbits;
}

struct RowState {
  f32x4 acc[12];  // O^T tiles: lane holds head (lane&15), dims 16nt+4*(lane>>4)+v
  float m;        // running max (base-2 logit units), same in the 4 lanes of a head
  float l;        // this lane's part of the running sum
};

// Online-softmax update from this lane's logits x[] (already scaled to base-2
// units and masked to -inf).  The running max is raised only when some head
// of the wave sees a logit more than kLazyRescale above it.  Otherwise the
// stale max is kept, which only means p <= 2^kLazyRescale (exact up to
// rounding), and the rescale of the 48 accumulators is skipped.  p is
// rounded to bf16 for the P.V product, and the running sum adds the rounded
// values.
constexpr float kLazyRescale = 8.0f;

template <int N>
__device__ __forceinline__ void softmax_step(float (&x)[N], RowState& st, uint32_t (&pb)[N / 2]) {
  float mloc = -INFINITY;
#pragma unroll
  for (int i = 0; i < N; ++i) mloc = fmaxf(mloc, x[i]);
  mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
  if (__ballot(mloc > st.m + kLazyRescale) != 0) {
    const float m_new = fmaxf(st.m, mloc);
    // A column that has seen no visible token yet keeps max -inf (its
    // accumulators are 0): scale it by 1, not by exp2(-inf - -inf) = NaN.
    const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(st.m - m_new);
    st.m = m_new;
    st.l *= alpha;
#pragma unroll
    for (int nt = 0; nt < 12; ++nt) st.acc[nt] *= alpha;
  }
  const float m_use = st.m == -INFINITY ? 0.f : st.m;
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < N; i += 2) {
    bf16x2 pk = {(__bf16)__builtin_amdgcn_exp2f(x[i] - m_use),
                 (__bf16)__builtin_amdgcn_exp2f(x[i + 1] - m_use)};
    const uint32_t w = __builtin_bit_cast(uint32_t, pk);
    psum += __uint_as_float(w << 16) + __uint_as_float(w & 0xFFFF0000u);
    pb[i / 2] = w;
  }
  st.l += psum;
}

// Window-mode visibility of this lane's S^T column: token t of the chunk
// starting at t0 is visible iff lo <= t <= hi (an empty range for unused
// columns).
struct ColWin {
  int t0, lo, hi;
};

// Compute one chunk from its LDS stage (K at +0, V at +kStageBytes).
// Visibility comes from the issue's per-token bits (region modes) or from the
// lane's column window (window mode).
template <bool kFp8, bool kWin>
__device__ __forceinline__ void compute_chunk(const uint8_t* stage, uint32_t vbits,
                                              const ColWin& cw, const u32x4 (&qreg)[6],
                                              float qk_scale_log2, int lane, RowState& st) {
  using C = Cfg<kFp8>;
  const int i16 = lane & 15, g4 = lane >> 4;
  const SDA_LDS uint8_t* kl = (const SDA_LDS uint8_t*)stage;
  // S^T: rows = token slots 16t + 4*g4 + v, columns = heads.  Lane (i16, g4)
  // reads K of token slot 16t + i16, pieces 4u + g4 (8 bf16 dims per k-slice,
  // or 16 FP8 dims feeding two k-slices).
  constexpr int kT = kFp8 ? 2 : 1;
  f32x4 s[kT];
#pragma unroll
  for (int t = 0; t < kT; ++t) {
    const int row = 16 * t + i16;
    const int f = swz_k<kFp8>(row);
    const SDA_LDS uint8_t* kr = kl + row * C::kVBytes;
    u32x4 kw[kFp8 ? 3 : 6];
#pragma unroll
    for (int u = 0; u < (kFp8 ? 3 : 6); ++u)
      kw[u] = *(const SDA_LDS u32x4*)(kr + 16 * ((4 * u + g4) ^ f));
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < 6; ++cc) {
      u32x4 k;
      if (kFp8) {
        u32x4 w = kw[cc >> 1];
        u32x2 c0 = fp8x4_to_bf16(w[(cc & 1) * 2 + 0]);
        u32x2 c1 = fp8x4_to_bf16(w[(cc & 1) * 2 + 1]);
        k = u32x4{c0[0], c0[1], c1[0], c1[1]};
      } else {
        k = kw[cc];
      }
      a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k),
                                                  __builtin_bit_cast(bf16x8, qreg[cc]), a, 0, 0,
                                                  0);
    }
    s[t] = a;
  }
  float x[4 * kT];
  if (kWin) {
    static_assert(!kWin || kT == 1, "window chunks are one 16-token tile");
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = cw.t0 + 4 * g4 + v;
      x[v] = (t >= cw.lo && t <= cw.hi) ? s[0][v] * qk_scale_log2 : -INFINITY;
    }
  } else {
    // Validity of token rows: lanes 0..15 loaded rows 0..15 of each tile.
#pragma unroll
    for (int t = 0; t < kT; ++t) {
      const uint64_t vb = __ballot((vbits >> t) & 1u);
#pragma unroll
      for (int v = 0; v < 4; ++v)
        x[4 * t + v] = ((vb >> (4 * g4 + v)) & 1) ? s[t][v] * qk_scale_log2 : -INFINITY;
    }
  }
  uint32_t pb[2 * kT];
  softmax_step<4 * kT>(x, st, pb);

  // O^T += V^T . P^T over the 12 dim tiles.
  const SDA_LDS uint8_t* lds = kl + kStageBytes;
  if (kFp8) {
    // tr8: lane 16*g4 + m reads 8 bytes of token row 16*(y>>2)+4*g4+(y&3), y = m>>1,
    // at V byte 16*nt + 8*(m&1); it receives byte (lane&15) of 8 rows.
    const int m = lane & 15, y = m >> 1, h = m & 1;
    const int row = 16 * (y >> 2) + 4 * g4 + (y & 3);
    const int f = swz<true>(row);
    const SDA_LDS uint8_t* base = lds + row * Cfg<true>::kVBytes + 8 * h;
    const bf16x8 pv = __builtin_bit_cast(bf16x8, u32x4{pb[0], pb[1], pb[2], pb[3]});
#pragma unroll
    for (int nt = 0; nt < 12; ++nt) {
      const int piece = (nt & ~3) | ((nt & 3) ^ f);
      i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SDA_LDS i32x2*)(base + 16 * piece));
      u32x2 c0 = fp8x4_to_bf16((uint32_t)raw[0]);
      u32x2 c1 = fp8x4_to_bf16((uint32_t)raw[1]);
      u32x4 a = u32x4{c0[0], c0[1], c1[0], c1[1]};
      st.acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), pv,
                                                           st.acc[nt], 0, 0, 0);
    }
  } else {
    // tr16: lane 16*g4 + 4y + q reads 4 bf16 of token row 4*g4 + y at dims
    // 16*nt + 4q; it receives dim 16*nt + (lane&15) of the 4 rows.
    const int y = (lane >> 2) & 3, q = lane & 3;
    const int row = 4 * g4 + y;
    const int f = swz<false>(row) ^ (q >> 1);
    const SDA_LDS uint8_t* base = lds + row * Cfg<false>::kVBytes + 8 * (q & 1);
    const bf16x4 pv = __builtin_bit_cast(bf16x4, u32x2{pb[0], pb[1]});
#pragma unroll
    for (int nt = 0; nt < 12; ++nt) {
      const int piece = ((2 * nt) & ~7) | (((2 * nt) & 7) ^ f);
      bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SDA_LDS bf16x4*)(base + 16 * piece));
      st.acc[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pv, st.acc[nt], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ uint16_t* out_row(const Params& p, int r) {
  const int t = r / p.groups;
  return p.out + (int64_t)t * p.ots + (int64_t)(r - t * p.groups) * p.ogs;
}

// The output is written once and read by the next kernel.  A large output
// (p.nt_out, see kNtOutputBytes) is stored non-temporally: cacheable stores
// left dirty lines whose write-back landed in later calls' streaming.  The
// policy is a template argument of the whole output loop: a branch around
// the store alone is merged by the compiler into one plain store.
template <bool kNt>
__device__ __forceinline__ void store_row_oct(uint16_t* orow, const Params& p, int h, int d,
                                              const f32x4& lo, const f32x4& hi) {
  const u32x4 v = {float_to_bf16_bits(lo[0]) | (float_to_bf16_bits(lo[1]) << 16),
                   float_to_bf16_bits(lo[2]) | (float_to_bf16_bits(lo[3]) << 16),
                   float_to_bf16_bits(hi[0]) | (float_to_bf16_bits(hi[1]) << 16),
                   float_to_bf16_bits(hi[2]) | (float_to_bf16_bits(hi[3]) << 16)};
  u32x4* dst = reinterpret_cast<u32x4*>(orow + (int64_t)h * p.ohs + d);
  if constexpr (kNt)
    __builtin_nontemporal_store(v, dst);
  else
    *dst = v;
}

template <bool kNt>
__device__ __forceinline__ void store_row_pair(uint16_t* orow, const Params& p, int h, int d,
                                               float o0, float o1) {
  uint32_t v = float_to_bf16_bits(o0) | (float_to_bf16_bits(o1) << 16);
  uint32_t* dst = reinterpret_cast<uint32_t*>(orow + (int64_t)h * p.ohs + d);
  if constexpr (kNt)
    __builtin_nontemporal_store(v, dst);
  else
    *dst = v;
}

__device__ __forceinline__ void clear_row(const Params& p, int r, int tid, int nthreads) {
  uint16_t* orow = out_row(p, r);
  for (int e = tid; e < p.heads * (kDim / 2); e += nthreads) {
    int h = e / (kDim / 2), d = 2 * (e - h * (kDim / 2));
    *reinterpret_cast<uint32_t*>(orow + (int64_t)h * p.ohs + d) = 0u;
  }
}

// Runs step(i0, 0), step(i0, 1), ... with compile-time stage indices while
// they return true.
template <typename F, int... Ss>
__device__ __forceinline__ bool run_steps(F& step, int i0, std::integer_sequence<int, Ss...>) {
  return (step(i0, std::integral_constant<int, Ss>{}) && ...);
}

// LDS use (stages + region list) allows one 4-wave or two 2-wave workgroups
// per CU, i.e. one wave per SIMD.
template <bool kFp8, bool kFused, int kAddr, int kWaves>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(1, 1))) void
split_kernel(const Params p) {
  using C = Cfg<kFp8>;
  constexpr int kThreads = 64 * kWaves;
  const int split = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, g4 = lane >> 4;

  __shared__ int64_t s_base[kMaxRegions];
  __shared__ int s_n[kMaxRegions];
  __shared__ __attribute__((aligned(1024))) uint8_t s_stage[kWaves][kStages][kChunkBytes];
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  __shared__ float s_fac[kWaves][16];
  // block-table entries of slot groups 1 .. kSlotBatch - 1 in the deferred
  // list mode (below), one per slot, landed by LDS-DMA
  __shared__ int32_t s_pages[kSlotBatch - 1][64];

  // The workgroup's query columns (the 16 columns of the MFMA tiles).
  //  * region modes: row r = blockIdx.x, or order[blockIdx.x] when the rows
  //    run heaviest first (token r / groups, group r % groups);
  //    column = head.
  //  * window mode: blockIdx.x = (request, token group, KV group), group
  //    fastest.  A token group is `pack` consecutive query tokens of the
  //    request (GQA and token packing: column = token-in-group * heads + head).
  int r = 0, tok0, g, req, pos, ncols, id_first = -1;
  int col_token, col_head;  // this lane's column
  ColWin cw{0, 1, 0};
  const uint16_t* qcol;
  if (kAddr == kWindow) {
    const int wg = blockIdx.x;
    const int rest = wg / p.groups;
    g = wg - rest * p.groups;
    req = rest / p.ntg;
    const int jj0 = (rest - req * p.ntg) * p.pack;
    const int np = min(p.pack, p.query_len - jj0);
    tok0 = req * p.query_len + jj0;
    ncols = np * p.heads;
    // Token j of a request of length L sits at L - query_len + j; `pos` is
    // the last token of the group, and the group's windows span
    // [max(0, pos_first - window + 1), pos].
    const int pos_first = p.seq_lens[req] - p.query_len + jj0;
    pos = pos_first + np - 1;
    const int jl = i16 / p.heads;
    const int h = i16 - jl * p.heads;
    col_token = tok0 + jl;
    col_head = h;
    qcol = p.q + (int64_t)(tok0 + jl) * p.qts + (int64_t)g * p.qgs + (int64_t)h * p.qhs;
    if (i16 < ncols) {
      cw.hi = pos_first + jl;
      cw.lo = (int)max((int64_t)0, (int64_t)cw.hi - p.window + 1);
    }
  } else {
    r = p.order ? p.order[blockIdx.x] : (int)blockIdx.x;
    // The active flag, the position and the first 64 region ids do not
    // depend on each other: one round trip for all three.
    const int act = p.active[r];
    pos = p.positions[r];
    id_first = lane < p.R ? p.regions[(int64_t)r * p.rrs + lane] : -1;
    __asm__ __volatile__("" : "+v"(pos), "+v"(id_first));
    if (!act) {
      // An inactive row reads nothing further (the position and ids loaded
      // with its flag go unused).  With splits > 1 the combine clears.
      if (kFused && p.clear) clear_row(p, r, tid, kThreads);
      return;
    }
    tok0 = r / p.groups;
    g = r - tok0 * p.groups;
    req = r / p.rows_per_req;
    ncols = p.heads;
    col_token = tok0;
    col_head = i16;
    qcol = p.q + (int64_t)tok0 * p.qts + (int64_t)g * p.qgs + (int64_t)i16 * p.qhs;
  }

  // Q^T B-operand: lane holds column (lane & 15), 8 dims per k-slice, in the
  // same dim order as the K loads.  Issued first so that its latency overlaps
  // the region resolution below.
  u32x4 qreg[6];
#pragma unroll
  for (int cc = 0; cc < 6; ++cc) {
    int d = kFp8 ? 64 * (cc >> 1) + 16 * g4 + 8 * (cc & 1) : 32 * cc + 8 * g4;
    qreg[cc] = i16 < ncols ? *reinterpret_cast<const u32x4*>(qcol + d) : u32x4{0, 0, 0, 0};
  }
  // The column's gate logit travels with Q, so that the epilogue does no
  // dependent global load.
  uint32_t gbits = 0;
  if (kFused && p.gated && i16 < ncols)
    gbits = p.gate[(int64_t)col_token * p.grs + (int64_t)(g * p.heads + col_head) * p.ghs];

  // Row extent, resolved by every wave on its own with no workgroup barrier.
  // All waves write identical values to the shared LDS list, and a wave only
  // ever reads entries after its own writes (LDS executes a wave's
  // operations in order), so the list is consistent without synchronisation.
  int nreg = 0, nchunks = 0;
  Win win{0, 0, 0, 0};
  // Deferred list mode (one split, 65..512 region slots): group 0's entries
  // are written before the pipeline starts; the block-table entries of
  // groups 1..7 are requested by LDS-DMA behind the first chunk and turned
  // into list entries after the first wait.  ids_d / kk_d: slot 64b + lane's
  // region id and list entry (-1: not visible); n0: group 0's entries.
  bool pending = false;
  int n0 = 0;
  int ids_d[kSlotBatch], kk_d[kSlotBatch];
  if (kAddr == kWindow) {
    // The union window's 16-token chunks, aligned down to a multiple of 16
    // so that a chunk never straddles a page, are dealt to the splits in
    // balanced contiguous runs.  s_base gets the pages this split's run
    // touches.
    const int w0 = (int)max((int64_t)0, (int64_t)pos - (ncols / p.heads - 1) - p.window + 1);
    const int a = w0 & ~15;
    const int total = pos < 0 ? 0 : (pos + 1 - a + 15) >> 4;
    const int clo = (int)(((int64_t)split * total + p.splits - 1) / p.splits);
    const int chi = (int)(((int64_t)(split + 1) * total + p.splits - 1) / p.splits);
    nchunks = chi - clo;
    win.w0 = w0;
    win.pos = pos;
    win.t_base = a + 16 * clo;
    if (nchunks > 0) {
      const int tb = min(a + 16 * chi, pos + 1) - 1;
      win.col_lo = win.t_base / p.block;
      const int npages = tb / p.block - win.col_lo + 1;
      const int32_t* trow = p.table + (int64_t)req * p.trs + win.col_lo;
      for (int k = lane; k < npages; k += 64)
        s_base[k] = (int64_t)trow[k] * p.cps + (int64_t)g * p.cgs;
    }
  } else {
    const int rt = p.rt;
    const int32_t* reg = p.regions + (int64_t)r * p.rrs;
    // Each wave ranks the visible slots (id >= 0, first token <= pos) in
    // slot order, 64 at a time.  It takes this split's balanced share, ranks
    // [ceil(s*V/S), ceil((s+1)*V/S)), and writes the share's cache offsets
    // and visible counts to the LDS list.  With one split every visible slot
    // is in the share, so the count pass is skipped.  Up to kSlotBatch
    // groups of 64 slots are loaded together (their ids, then their
    // block-table entries): two round trips per 512 slots.
    // The first 64 slots (id_first) were loaded with the row's flag.
    const int ngroups = (p.R + 63) / 64;
    if (ngroups <= 1) {
      // At most 64 slots: the ids loaded with the flag are the whole list.
      const bool vis = id_first >= 0 && (int64_t)id_first * rt <= pos;
      const uint64_t m = __ballot(vis);
      const int nvis = __popcll(m);
      const int lo1 = (int)(((int64_t)split * nvis + p.splits - 1) / p.splits);
      const int hi1 = (int)(((int64_t)(split + 1) * nvis + p.splits - 1) / p.splits);
      const int k = __popcll(m & ((1ull << lane) - 1ull));
      if (vis && k >= lo1 && k < hi1) {
        const int64_t t0 = (int64_t)id_first * rt;
        const int64_t col = t0 / p.block;
        const int off0 = (int)(t0 - col * p.block);
        const int64_t page = p.table[(int64_t)req * p.trs + col];
        s_base[k - lo1] = page * p.cps + (int64_t)g * p.cgs + (int64_t)off0 * p.cts;
        s_n[k - lo1] = (int)min((int64_t)rt, (int64_t)pos - t0 + 1);
      }
      nreg = hi1 - lo1;
    } else {
      bool deferred = p.splits == 1 && ngroups <= kSlotBatch;
      if (deferred) {
        // Deferred list mode.  Group 0's block-table entries and the ids of
        // groups 1..7 share one round trip; every slot's rank is known after
        // it.
        const bool vis0 = id_first >= 0 && (int64_t)id_first * rt <= pos;
        int64_t page0 = 0;
        if (vis0) page0 = p.table[(int64_t)req * p.trs + (int64_t)id_first * rt / p.block];
        ids_d[0] = id_first;
#pragma unroll
        for (int b = 1; b < kSlotBatch; ++b) {
          const int j = 64 * b + lane;
          ids_d[b] = b < ngroups && j < p.R ? reg[j] : -1;
        }
        int base_rank = 0;
#pragma unroll
        for (int b = 0; b < kSlotBatch; ++b) {
          const bool vis = ids_d[b] >= 0 && (int64_t)ids_d[b] * rt <= pos;
          const uint64_t m = __ballot(vis);
          kk_d[b] = vis ? base_rank + __popcll(m & ((1ull << lane) - 1ull)) : -1;
          base_rank += __popcll(m);
          if (b == 0) n0 = base_rank;
        }
        // The first two chunks of every wave are issued before the first
        // wait: group 0 must cover them, or the row takes the path below.
        const int cover = (int)(((int64_t)2 * kWaves * C::kTok - 1) / rt) + 1;
        if (n0 < cover && base_rank > n0) {
          deferred = false;
        } else {
          if (vis0) {
            const int64_t t0 = (int64_t)id_first * rt;
            s_base[kk_d[0]] = page0 * p.cps + (int64_t)g * p.cgs + (t0 % p.block) * p.cts;
            s_n[kk_d[0]] = (int)min((int64_t)rt, (int64_t)pos - t0 + 1);
          }
          nreg = base_rank;
          pending = nreg > n0;
        }
      }
      if (!deferred) {
        auto load_ids = [&](int k0, int (&idb)[kSlotBatch]) {
#pragma unroll
          for (int b = 0; b < kSlotBatch; ++b) {
            const int j = 64 * (k0 + b) + lane;
            idb[b] = k0 + b == 0 ? id_first : (k0 + b < ngroups && j < p.R ? reg[j] : -1);
          }
        };
        int lo = 0, hi = 0x7FFFFFFF;
        if (p.splits > 1) {
          int nvis = 0;
          for (int k0 = 0; k0 < ngroups; k0 += kSlotBatch) {
            int idb[kSlotBatch];
            load_ids(k0, idb);
#pragma unroll
            for (int b = 0; b < kSlotBatch; ++b)
              nvis += __popcll(__ballot(idb[b] >= 0 && (int64_t)idb[b] * rt <= pos));
          }
          lo = (int)(((int64_t)split * nvis + p.splits - 1) / p.splits);
          hi = (int)(((int64_t)(split + 1) * nvis + p.splits - 1) / p.splits);
        }
        int base_rank = 0;
        for (int k0 = 0; k0 < ngroups; k0 += kSlotBatch) {
          int idb[kSlotBatch];
          load_ids(k0, idb);
          int64_t pg[kSlotBatch];
          int kk[kSlotBatch];
#pragma unroll
          for (int b = 0; b < kSlotBatch; ++b) {
            const bool vis = idb[b] >= 0 && (int64_t)idb[b] * rt <= pos;
            const uint64_t m = __ballot(vis);
            const int k = base_rank + __popcll(m & ((1ull << lane) - 1ull));
            const bool mine = vis && k >= lo && k < hi;
            kk[b] = mine ? k - lo : -1;
            pg[b] = mine ? p.table[(int64_t)req * p.trs + (int64_t)idb[b] * rt / p.block] : 0;
            base_rank += __popcll(m);
          }
#pragma unroll
          for (int b = 0; b < kSlotBatch; ++b) {
            if (kk[b] >= 0) {
              const int64_t t0 = (int64_t)idb[b] * rt;
              const int off0 = (int)(t0 % p.block);
              s_base[kk[b]] = pg[b] * p.cps + (int64_t)g * p.cgs + (int64_t)off0 * p.cts;
              s_n[kk[b]] = (int)min((int64_t)rt, (int64_t)pos - t0 + 1);
            }
          }
        }
        nreg = p.splits > 1 ? hi - lo : base_rank;
      }
    }
    nchunks = (int)(((int64_t)nreg * rt + C::kTok - 1) / C::kTok);
  }
  // The list reads below must follow this wave's own list writes.
  __asm__ __volatile__("" ::: "memory");
  // Consume Q here, so the compiler's wait for these loads sits before the
  // pipeline rather than inside it.
#pragma unroll
  for (int cc = 0; cc < 6; ++cc) __asm__ __volatile__("" : "+v"(qreg[cc]));
  __asm__ __volatile__("" : "+v"(gbits));

  const float kscale = kFp8 ? *p.k_scale : 1.0f;
  const float qk_scale_log2 = p.scale * kscale * 1.4426950408889634f;

  RowState st;
#pragma unroll
  for (int nt = 0; nt < 12; ++nt) st.acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;

  const uint8_t* my_stage = &s_stage[wave][0][0];
  const uint32_t my_stage_lds = lds_addr(my_stage);

  // kStages-deep per-wave pipeline over LDS stages: iteration i (chunk
  // c = wave + kWaves*i) computes stage i % kStages while the next chunk is
  // in flight.  An iteration with a next chunk issues it (12 DMA
  // instructions) and waits until at most those 12 are outstanding, i.e.
  // chunk c has landed; the last iteration issues nothing and waits for
  // everything, so no load is left in flight past the loop.
  static_assert(kStages == 2, "the tail wait assumes one chunk in flight");
  if (wave < nchunks) {
    const LaneDma ld = lane_dma<kFp8>(lane);
    const uint32_t cts_bytes = (uint32_t)(p.cts * C::kEsz);
    uint32_t vb[kStages];
    vb[0] = issue_chunk<kFp8, kAddr>(p, wave, nreg, s_base, s_n, lane, my_stage_lds, ld, cts_bytes,
                                     win);
    // Deferred list mode: the block-table entries of groups 1..7 go to
    // s_pages by LDS-DMA (one dword per lane; slots that are not visible
    // read the row's first entry); the first wait below covers them.
    if (kAddr != kWindow && pending) {
      const int32_t* trow = p.table + (int64_t)req * p.trs;
#pragma unroll
      for (int b = 1; b < kSlotBatch; ++b) {
        if (64 * b >= p.R) break;
        const int32_t* a = kk_d[b] >= 0 ? trow + (int64_t)ids_d[b] * p.rt / p.block : trow;
        dma_dword((uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(&s_pages[b - 1][0])), a);
      }
    }
    // List entries of groups 1..7 from the landed block-table entries.
    auto convert = [&]() {
#pragma unroll
      for (int b = 1; b < kSlotBatch; ++b) {
        if (kk_d[b] >= 0) {
          const int64_t page = s_pages[b - 1][lane];
          const int64_t t0 = (int64_t)ids_d[b] * p.rt;
          s_base[kk_d[b]] = page * p.cps + (int64_t)g * p.cgs + (t0 % p.block) * p.cts;
          s_n[kk_d[b]] = (int)min((int64_t)p.rt, (int64_t)pos - t0 + 1);
        }
      }
      // later list reads follow these writes (a wave's LDS operations run
      // in order)
      __asm__ __volatile__("" ::: "memory");
      pending = false;
    };
    auto step = [&](int i0, auto stage_c) -> bool {
      constexpr int S = decltype(stage_c)::value;
      constexpr int SN = (S + kStages - 1) % kStages;
      const int c = wave + kWaves * (i0 + S);
      if (c >= nchunks) return false;
      // Stage SN was last read by the previous iteration, whose reads all
      // completed before its MFMAs; the asm below keeps them above the DMA.
      const int cn = c + kWaves * (kStages - 1);
      if (kAddr != kWindow && pending && cn < nchunks &&
          (int)(((int64_t)(cn + 1) * C::kTok - 1) / p.rt) >= n0) {
        // the next chunk reaches past group 0 before the entries were
        // converted: wait for everything in flight and convert now
        wait_vmcnt<0>();
        convert();
      }
      if (cn < nchunks) {
        vb[SN] = issue_chunk<kFp8, kAddr>(p, cn, nreg, s_base, s_n, lane,
                                          my_stage_lds + SN * kChunkBytes, ld, cts_bytes, win);
        wait_vmcnt<kOpsPerChunk * (kStages - 1)>();
      } else {
        wait_vmcnt<0>();
      }
      if (kAddr != kWindow && pending) convert();
      if (kAddr == kWindow) cw.t0 = win.t_base + 16 * c;
      compute_chunk<kFp8, kAddr == kWindow>(my_stage + S * kChunkBytes, vb[S], cw, qreg,
                                            qk_scale_log2, lane, st);
      return true;
    };
    for (int i0 = 0;; i0 += kStages)
      if (!run_steps(step, i0, std::make_integer_sequence<int, kStages>{})) break;
  }

  // Merge the 4 waves.  The per-lane sums of a head live in its 4 lane groups.
  // Each wave parks its state in its own (drained) stage memory, so a single
  // barrier separates the writes from the cross-wave reads.
  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  constexpr int kWaveStride = kStages * kChunkBytes / sizeof(float);  // floats between waves
  static_assert(16 * kAccStride <= kWaveStride, "merge area fits a wave's stages");
  float* s_acc = reinterpret_cast<float*>(&s_stage[0][0][0]);
#pragma unroll
  for (int nt = 0; nt < 12; ++nt) {
    float* dst = s_acc + (size_t)wave * kWaveStride + i16 * kAccStride + 16 * nt + 4 * g4;
    *reinterpret_cast<f32x4*>(dst) = st.acc[nt];
  }
  if (g4 == 0) {
    s_m[wave][i16] = st.m;
    s_l[wave][i16] = l;
  }
  __syncthreads();

  // Per column, once: the merged max and sum, the weight of each wave's
  // partial state, 1/L, v_scale and (combine fused) the gate, folded into one
  // factor per wave.  Lanes 0..15 of wave 0 hold columns 0..15.
  if (tid < 16) {
    const int c = tid;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][c]);
    float f[kWaves];
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      f[w] = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_m[w][c] - M);
      L += s_l[w][c] * f[w];
    }
    float scale = M == -INFINITY ? 0.f : (kFp8 ? *p.v_scale : 1.0f) / L;
    if (kFused && p.gated) scale *= gate_sigmoid(gbits);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s_fac[w][c] = f[w] * scale;
    if (!kFused && c < ncols) {
      const int row = kAddr == kWindow ? col_token * p.groups + g : r;
      p.lse[((int64_t)row * p.splits + split) * p.heads + col_head] =
          M == -INFINITY ? -INFINITY : M + __log2f(L);
    }
  }
  __syncthreads();

  auto output_loop = [&](auto nt) {
  if (kFused && p.wide_out) {
    // 16-byte aligned output: 8 dims per thread, one 16-byte store (the same
    // sums in the same order as the pair loop below).
    for (int e = tid; e < ncols * (kDim / 8); e += kThreads) {
      const int c = e / (kDim / 8), d = 8 * (e - c * (kDim / 8));
      int token = tok0, h = c;
      if (kAddr == kWindow) {
        const int jl = c / p.heads;
        token += jl;
        h = c - jl * p.heads;
      }
      f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float fw = s_fac[w][c];
        const f32x4* src =
            reinterpret_cast<const f32x4*>(s_acc + (size_t)w * kWaveStride + c * kAccStride + d);
        lo += src[0] * fw;
        hi += src[1] * fw;
      }
      uint16_t* orow = p.out + (int64_t)token * p.ots + (int64_t)g * p.ogs;
      store_row_oct<decltype(nt)::value>(orow, p, h, d, lo, hi);
    }
    return;
  }
  for (int e = tid; e < ncols * (kDim / 2); e += kThreads) {
    const int c = e / (kDim / 2), d = 2 * (e - c * (kDim / 2));
    // column c -> (token, head) and its output row
    int token = tok0, h = c;
    if (kAddr == kWindow) {
      const int jl = c / p.heads;
      token += jl;
      h = c - jl * p.heads;
    }
    float o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float fw = s_fac[w][c];
      const float* src = s_acc + (size_t)w * kWaveStride + c * kAccStride + d;
      o0 += src[0] * fw;
      o1 += src[1] * fw;
    }
    if (kFused) {
      uint16_t* orow = p.out + (int64_t)token * p.ots + (int64_t)g * p.ogs;
      store_row_pair<decltype(nt)::value>(orow, p, h, d, o0, o1);
    } else {
      const int row = kAddr == kWindow ? token * p.groups + g : r;
      int64_t ph = ((int64_t)row * p.splits + split) * p.heads + h;
      *reinterpret_cast<float2*>(p.partial + ph * kDim + d) = make_float2(o0, o1);
    }
  }
  };
  if (kFused && p.nt_out)
    output_loop(std::true_type{});
  else
    output_loop(std::false_type{});
}

// Row-stream kernel, for batches of at least two rows per wave of the chip:
// every wave owns whole rows (rows w, w + W, w + 2W, ... for wave w of W)
// and streams them back to back through its own two-stage chunk pipeline, so
// the pipeline never drains between rows.
//  * Up front, each wave resolves the region lists of all its rows at once:
//    their flags, positions, region ids and gate logits in one round trip,
//    their block-table entries in a second.  The lists go to the wave's part
//    of LDS; no workgroup barrier is ever taken.
//  * A row's query (16 columns x 192 bf16) moves to one of two per-wave LDS
//    buffers by LDS-DMA, issued together with the row's first chunk, and is
//    read into the MFMA B-operand registers when that chunk is computed.
//  * After a row's last chunk, the wave folds its running sums, v_scale and
//    the gate into one factor per column, rounds the output to bf16 through
//    the chunk's just-computed LDS stage and writes it with 16-byte stores,
//    while the next row's first chunk is already in flight.
// The arithmetic per chunk is the split kernel's (issue_chunk,
// compute_chunk); one wave sums a row's chunks in order.
constexpr int kStreamWaves = 4;
constexpr int kStreamMaxRows = 8;   // rows per wave
constexpr int kStreamList = 256;    // region-list entries per wave (all its rows)
constexpr int kStreamMaxR = 64;     // region slots per row (one id per lane)
constexpr int kQueryBytes = 16 * kDim * 2;
static_assert(kQueryBytes == 6 * 1024, "a query is six 1 KiB LDS-DMAs");
static_assert(kStreamMaxRows <= 64 && kStreamMaxR <= 64, "one lane per row / slot");

// The six LDS-DMAs of one row's query: piece P = 64k + lane of 16 bytes
// (column P / 24, dims 8 (P % 24) ..) lands at buffer byte 16 P, i.e. the
// buffer is [16 columns][192] bf16.  Per-lane 64-bit addresses.
__device__ __forceinline__ void dma_query(uint32_t buf, const uint8_t* const (&a)[6]) {
  uint32_t saved;
  __asm__ __volatile__(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[st]\n\t" SDA_LDDMA("a0", "off", "") SDA_NEXT SDA_LDDMA("a1", "off", "")
          SDA_NEXT SDA_LDDMA("a2", "off", "") SDA_NEXT SDA_LDDMA("a3", "off", "") SDA_NEXT
              SDA_LDDMA("a4", "off", "") SDA_NEXT SDA_LDDMA("a5", "off", "")
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [st] "s"(buf), [a0] "v"(a[0]), [a1] "v"(a[1]), [a2] "v"(a[2]), [a3] "v"(a[3]),
        [a4] "v"(a[4]), [a5] "v"(a[5])
      : "memory");
}

template <bool kFp8, int kAddr, bool kNt>
__global__ __launch_bounds__(64 * kStreamWaves) __attribute__((amdgpu_waves_per_eu(1, 1))) void
row_stream_kernel(const Params p) {
  using C = Cfg<kFp8>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g4 = lane >> 4;

  __shared__ __attribute__((aligned(1024))) uint8_t s_stage[kStreamWaves][2][kChunkBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_query[kStreamWaves][2][kQueryBytes];
  __shared__ int64_t s_base[kStreamWaves][kStreamList];
  __shared__ int s_n[kStreamWaves][kStreamList];

  // This wave's rows: r_j = gw + j * W, j < nrows (the launch guarantees
  // 1 <= nrows <= kStreamMaxRows and nrows * R <= kStreamList).
  const int W = gridDim.x * kStreamWaves;
  const int gw = blockIdx.x * kStreamWaves + wave;
  const int nrows = (p.rows - gw + W - 1) / W;

  // Round trip 1: lane j holds row j's flag and position; ids[j] holds slot
  // `lane` of row j; gl[j] the gate logit of column i16 of row j.  Loads are
  // unconditional at clamped indices (one round trip), masked afterwards.
  const int rl = gw + min(lane, nrows - 1) * W;
  const int act_l = p.active[rl];
  const int pos_l = p.positions[rl];
  int ids[kStreamMaxRows];
  uint32_t gl[kStreamMaxRows];
  const int slot = min(lane, max(p.R - 1, 0));
#pragma unroll
  for (int j = 0; j < kStreamMaxRows; ++j) {
    const int r = gw + min(j, nrows - 1) * W;
    ids[j] = -1;
    gl[j] = 0;
    if (j >= nrows) continue;  // wave-uniform: no requests for absent rows
    if (p.R > 0) ids[j] = p.regions[(int64_t)r * p.rrs + slot];
    if (p.gated) {
      const int t = r / p.groups;
      const int col = min(i16, p.heads - 1);
      gl[j] = p.gate[(int64_t)t * p.grs + (int64_t)((r - t * p.groups) * p.heads + col) * p.ghs];
    }
  }
  const float kscale = kFp8 ? *p.k_scale : 1.0f;
  const float vscale = kFp8 ? *p.v_scale : 1.0f;
  const float qk_scale_log2 = p.scale * kscale * 1.4426950408889634f;

  // Round trip 2: the block-table entries of every visible slot of every row.
  const int rt = p.rt;
  int64_t pages[kStreamMaxRows];
  uint64_t vis[kStreamMaxRows];
#pragma unroll
  for (int j = 0; j < kStreamMaxRows; ++j) {
    const int r = gw + min(j, nrows - 1) * W;
    const int act = __builtin_amdgcn_readlane(act_l, min(j, nrows - 1));
    const int pos = __builtin_amdgcn_readlane(pos_l, min(j, nrows - 1));
    const int id = lane < p.R ? ids[j] : -1;
    const bool v = j < nrows && act && id >= 0 && (int64_t)id * rt <= pos;
    vis[j] = __ballot(v);
    const int64_t t0 = v ? (int64_t)id * rt : 0;
    const int req = r / p.rows_per_req;
    pages[j] = v ? p.table[(int64_t)req * p.trs + t0 / p.block] : 0;
  }
  // Lists: row j's visible slots in slot order at entries off_j .. off_j +
  // nreg_j.  Lane j keeps nreg_j and off_j (read back with readlane: row
  // indices are wave-uniform, and register arrays are never indexed at run
  // time).
  int off = 0, nreg_l = 0, off_l = 0;
  int64_t* lb = s_base[wave];
  int* ln = s_n[wave];
#pragma unroll
  for (int j = 0; j < kStreamMaxRows; ++j) {
    const int r = gw + min(j, nrows - 1) * W;
    const int pos = __builtin_amdgcn_readlane(pos_l, min(j, nrows - 1));
    const int g = r % p.groups;
    const uint64_t m = vis[j];
    if ((m >> lane) & 1) {
      const int k = off + __popcll(m & ((1ull << lane) - 1ull));
      const int64_t t0 = (int64_t)ids[j] * rt;
      lb[k] = pages[j] * p.cps + (int64_t)g * p.cgs + (t0 % p.block) * p.cts;
      ln[k] = (int)min((int64_t)rt, (int64_t)pos - t0 + 1);
    }
    if (lane == j) {
      nreg_l = __popcll(m);
      off_l = off;
    }
    off += __popcll(m);
  }
  // the list reads below follow this wave's own list writes
  __asm__ __volatile__("" ::: "memory");
  // rows with visible tokens, one bit per row
  const uint64_t live = __ballot(lane < nrows && nreg_l > 0);

  // Rows with nothing to stream (inactive, or no visible token): zeros,
  // unless inactive and not cleared.
  for (int j = 0; j < nrows; ++j) {
    if ((live >> j) & 1) continue;
    const int act = __builtin_amdgcn_readlane(act_l, j);
    if (!act && !p.clear) continue;
    uint16_t* orow = out_row(p, gw + j * W);
    for (int e = lane; e < p.heads * (kDim / 8); e += 64) {
      const int h = e / (kDim / 8), d = 8 * (e - h * (kDim / 8));
      *reinterpret_cast<u32x4*>(orow + (int64_t)h * p.ohs + d) = u32x4{0, 0, 0, 0};
    }
  }

  // The stream of (row j, chunk c) items over the rows with visible tokens.
  auto row_nreg = [&](int j) { return __builtin_amdgcn_readlane(nreg_l, j); };
  auto row_chunks = [&](int j) {
    return (int)(((int64_t)row_nreg(j) * rt + C::kTok - 1) / C::kTok);
  };
  auto next_row = [&](int j) {  // first row after j with visible tokens, or nrows
    const uint64_t after = live & ~((2ull << j) - 1ull);
    return after ? (int)__builtin_ctzll(after) : nrows;
  };

  const uint8_t* my_stage = &s_stage[wave][0][0];
  const uint32_t my_stage_lds = lds_addr(my_stage);
  const uint32_t my_query_lds = lds_addr(&s_query[wave][0][0]);
  const LaneDma ld = lane_dma<kFp8>(lane);
  const uint32_t cts_bytes = (uint32_t)(p.cts * C::kEsz);
  const Win win{0, 0, 0, 0};

  // Query DMA of row r into buffer qb.
  auto issue_query = [&](int r, int qb) {
    const int t = r / p.groups;
    const uint16_t* qrow = p.q + (int64_t)t * p.qts + (int64_t)(r - t * p.groups) * p.qgs;
    const uint8_t* a[6];
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      const int P = 64 * k + lane;
      const int col = P / 24;
      const int c = col < p.heads ? col : 0;
      a[k] = reinterpret_cast<const uint8_t*>(qrow + (int64_t)c * p.qhs + 8 * (P - 24 * col));
    }
    dma_query((uint32_t)__builtin_amdgcn_readfirstlane(my_query_lds + qb * kQueryBytes), a);
  };
  auto issue_item = [&](int j, int c, int stage) {
    const int o = __builtin_amdgcn_readlane(off_l, j);
    return issue_chunk<kFp8, kAddr>(p, c, row_nreg(j), lb + o, ln + o, lane,
                                    my_stage_lds + stage * kChunkBytes, ld, cts_bytes, win);
  };

  int j = live ? (int)__builtin_ctzll(live) : nrows;
  if (j >= nrows) return;
  int qb = 0;
  issue_query(gw + j * W, qb);
  uint32_t vb[2];
  vb[0] = issue_item(j, 0, 0);
  int c = 0, nch = row_chunks(j);
  int s = 0;

  RowState st;
#pragma unroll
  for (int nt = 0; nt < 12; ++nt) st.acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
  u32x4 qreg[6];
  const ColWin cw{0, 1, 0};

  for (;;) {
    // the next item: chunk c + 1 of this row, or the first chunk of the next
    // row with visible tokens (its query DMA goes first)
    int jn = j, cn = c + 1;
    if (cn >= nch) {
      jn = next_row(j);
      cn = 0;
    }
    if (jn < nrows) {
      if (cn == 0) {
        issue_query(gw + jn * W, qb ^ 1);
        vb[s ^ 1] = issue_item(jn, 0, s ^ 1);
        wait_vmcnt<kOpsPerChunk + 6>();
      } else {
        vb[s ^ 1] = issue_item(jn, cn, s ^ 1);
        wait_vmcnt<kOpsPerChunk>();
      }
    } else {
      wait_vmcnt<0>();
    }
    if (c == 0) {
      // this row's query has landed with its first chunk: B operand, column i16
      const SDA_LDS uint8_t* qcol =
          (const SDA_LDS uint8_t*)&s_query[wave][qb][0] + i16 * (kDim * 2);
#pragma unroll
      for (int cc = 0; cc < 6; ++cc) {
        const int d = kFp8 ? 64 * (cc >> 1) + 16 * g4 + 8 * (cc & 1) : 32 * cc + 8 * g4;
        qreg[cc] = i16 < p.heads ? *(const SDA_LDS u32x4*)(qcol + 2 * d) : u32x4{0, 0, 0, 0};
      }
    }
    compute_chunk<kFp8, false>(my_stage + s * kChunkBytes, vb[s], cw, qreg, qk_scale_log2, lane,
                               st);
    if (c + 1 == nch) {
      // Row j is complete: fold the sums, v_scale and the gate into one
      // factor per column and write the row through the computed stage.
      float l = st.l;
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
      float f = st.m == -INFINITY ? 0.f : vscale / l;
      if (p.gated) {
        uint32_t gj = gl[0];
#pragma unroll
        for (int i = 1; i < kStreamMaxRows; ++i) gj = i == j ? gl[i] : gj;  // no run-time index
        f *= gate_sigmoid(gj);
      }
      uint8_t* stg = const_cast<uint8_t*>(my_stage) + s * kChunkBytes;
#pragma unroll
      for (int nt = 0; nt < 12; ++nt) {
        const f32x4 v = st.acc[nt] * f;
        const u32x2 w = {float_to_bf16_bits(v[0]) | (float_to_bf16_bits(v[1]) << 16),
                         float_to_bf16_bits(v[2]) | (float_to_bf16_bits(v[3]) << 16)};
        *(SDA_LDS u32x2*)((SDA_LDS uint8_t*)stg + (i16 * kDim + 16 * nt + 4 * g4) * 2) = w;
      }
      __asm__ __volatile__("" ::: "memory");  // a wave's LDS operations run in order
      uint16_t* orow = out_row(p, gw + j * W);
#pragma unroll
      for (int k = 0; k < 6; ++k) {
        const int P = 64 * k + lane;
        const int col = P / 24;
        if (col < p.heads) {
          const u32x4 v = *(const SDA_LDS u32x4*)((SDA_LDS uint8_t*)stg + 16 * P);
          u32x4* dst = reinterpret_cast<u32x4*>(orow + (int64_t)col * p.ohs + 8 * (P - 24 * col));
          if constexpr (kNt)
            __builtin_nontemporal_store(v, dst);
          else
            *dst = v;
        }
      }
      // the next DMA into this stage (next iteration) follows these reads
      __asm__ __volatile__("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int nt = 0; nt < 12; ++nt) st.acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      st.m = -INFINITY;
      st.l = 0.f;
    }
    if (jn >= nrows) break;
    if (jn != j) {
      j = jn;
      nch = row_chunks(j);
      qb ^= 1;
    }
    c = cn;
    s ^= 1;
  }
}

// One 64-thread workgroup per (row, head), a (rows, heads) grid: 3 dims per
// thread.
__global__ __launch_bounds__(64) void combine_kernel(const Params p) {
  const int r = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  uint16_t* orow = out_row(p, r) + (int64_t)h * p.ohs;
  if (p.active && !p.active[r]) {
    if (p.clear)
      for (int d = tid; d < kDim; d += 64) orow[d] = 0;
    return;
  }
  const int64_t ph0 = (int64_t)r * p.splits * p.heads + h;
  float M = -INFINITY;
  for (int s = 0; s < p.splits; ++s) M = fmaxf(M, p.lse[ph0 + (int64_t)s * p.heads]);
  float o[3] = {0.f, 0.f, 0.f};
  if (M != -INFINITY) {
    float W = 0.f;
    for (int s = 0; s < p.splits; ++s) {
      const int64_t ph = ph0 + (int64_t)s * p.heads;
      const float w = __builtin_amdgcn_exp2f(p.lse[ph] - M);
      const float* src = p.partial + ph * kDim;
      W += w;
#pragma unroll
      for (int u = 0; u < 3; ++u) o[u] += w * src[tid + 64 * u];
    }
#pragma unroll
    for (int u = 0; u < 3; ++u) o[u] /= W;
  }
  float gv = 1.0f;
  if (p.gated)
    gv = gate_value(p.gate, (int64_t)(r / p.groups) * p.grs +
                                (int64_t)((r % p.groups) * p.heads + h) * p.ghs);
#pragma unroll
  for (int u = 0; u < 3; ++u) orow[tid + 64 * u] = (uint16_t)float_to_bf16_bits(o[u] * gv);
}

// Row order for grids a few times larger than the chip holds at once.
// Workgroups start in index order as earlier ones retire, so a heavy row that
// starts late stretches the tail of the launch.  Two small kernels rank the
// rows by visible tokens (0 for an inactive row) and write them heaviest
// first within each block of 1024 rows:
//  * bin_kernel: one wave per row, spread over the chip; writes each
//    row's bin, 0 (heaviest) .. kOrderBins - 1, of width
//    (R * region tokens + 1) / kOrderBins;
//  * order_kernel: one 1024-thread workgroup per block of 1024 rows; a stable
//    counting sort on the bins.
// Rows of nearly equal work share a bin and keep index order: neighbouring
// rows are the KV groups of one token, which read neighbouring slices of the
// same pages.  Blocks of 1024 rows are at least as large as the resident grid
// (512 workgroups), which is what keeps light rows at the end.  A row's
// result does not depend on which workgroup computes it.
constexpr int kOrderBlock = 1024;
constexpr int kOrderWaves = kOrderBlock / 64;
constexpr int kOrderBins = 32;
constexpr int kOrderMaxRounds = 4;  // order grids of up to 4x the resident workgroups
static_assert(kOrderBins * kOrderWaves == 8 * 64, "the scan: 8 entries per lane of one wave");

template <int kLoads>
__global__ __launch_bounds__(256) void bin_kernel(Params p, int64_t max_tokens, int32_t* bins) {
  const int lane = threadIdx.x & 63;
  // One wave per row: lane l holds slots l, l + 64, ... (kLoads >= R / 64
  // of them) of the row's region ids, all requested at once with the flag
  // and the position (one round trip), at indices clamped into the row and
  // masked afterwards.
  const int r = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (r >= p.rows) return;
  const int act = p.active[r];
  const int pos_raw = p.positions[r];
  const int32_t* row = p.regions + (int64_t)r * p.rrs;
  int ids[kLoads];
#pragma unroll
  for (int k = 0; k < kLoads; ++k) ids[k] = row[min(64 * k + lane, p.R - 1)];
  // Region id i is visible in part or whole iff 0 <= i <= pq, wholly iff
  // 0 <= i < pf; the one partial region shows pos % rt + 1 tokens.
  const int pos = act ? pos_raw : -1;
  const int pq = pos >= 0 ? pos / p.rt : -1;
  const int pf = pos >= 0 ? (pos + 1) / p.rt : 0;
  const int part = pos >= 0 ? pos - pq * p.rt + 1 : 0;
  int64_t tokens = 0;
#pragma unroll
  for (int k = 0; k < kLoads; ++k) {
    const int id = 64 * k + lane < p.R ? ids[k] : -1;
    const uint64_t ba = __ballot(id >= 0 && id <= pq);
    const uint64_t bf = __ballot(id >= 0 && id < pf);
    tokens += (int64_t)__popcll(bf) * p.rt + (int64_t)__popcll(ba & ~bf) * part;
  }
  if (lane == 0) bins[r] = kOrderBins - 1 - (int)(tokens * kOrderBins / (max_tokens + 1));
}

__global__ __launch_bounds__(kOrderBlock) void order_kernel(Params p, const int32_t* bins) {
  // s_cnt[bin][wave]: rows of the wave in the bin, then their first slot.
  __shared__ __attribute__((aligned(16))) int s_cnt[kOrderBins * kOrderWaves];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int r = blockIdx.x * kOrderBlock + t;
  const int bin_raw = bins[min(r, p.rows - 1)];
  // The counts are cleared while the bins are in flight (an LDS-only
  // barrier: a __syncthreads() fence would wait for the load).
  if (t < kOrderBins * kOrderWaves) s_cnt[t] = 0;
  __asm__ __volatile__("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  const int bin = r < p.rows ? bin_raw : -1;
  // Lanes of the wave in the same bin, and this lane's rank among them.
  uint64_t same = __ballot(bin >= 0);
#pragma unroll
  for (int b = 1; b < kOrderBins; b <<= 1) {
    const uint64_t m = __ballot((bin & b) != 0);
    same &= (bin & b) ? m : ~m;
  }
  const uint64_t below = lane ? ~0ull >> (64 - lane) : 0ull;
  const int rank = __popcll(same & below);
  if (bin >= 0 && rank == 0) s_cnt[bin * kOrderWaves + wave] = __popcll(same);
  __syncthreads();
  // Exclusive scan of s_cnt in (bin, wave) order, the first slot of each
  // wave's rows of each bin, by wave 0 alone: lane l takes the 8 entries
  // [8 l, 8 l + 8), scans them, and one wave scan adds the lanes before.
  if (wave == 0) {
    int4* c4 = reinterpret_cast<int4*>(s_cnt) + 2 * lane;
    const int4 a = c4[0], b = c4[1];
    const int e[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    int run = 0, ex[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      ex[q] = run;
      run += e[q];
    }
    const int base = wave_inclusive_scan(run) - run;
    c4[0] = make_int4(base + ex[0], base + ex[1], base + ex[2], base + ex[3]);
    c4[1] = make_int4(base + ex[4], base + ex[5], base + ex[6], base + ex[7]);
  }
  __syncthreads();
  if (bin >= 0) p.order_ws[blockIdx.x * kOrderBlock + s_cnt[bin * kOrderWaves + wave] + rank] = r;
}

// Workgroups resident at once for a grid of `wgs` workgroups on `cus`
// compute units (the wave count, and with it the workgroups per CU, follows
// from the grid size).
int64_t resident_workgroups(int64_t wgs, int cus) {
  return wgs >= 2 * (int64_t)cus ? 2 * (int64_t)cus : (int64_t)cus;
}

bool two_per_cu(int64_t wgs, int cus) { return wgs >= 2 * (int64_t)cus; }

// Whether the split kernel's grid is worth ranking first: a workspace is
// given and the grid takes 2 to kOrderMaxRounds rounds of resident
// workgroups.  With one round every row starts at once, and with many the
// tail is a small part of the launch.
bool wants_order(const Params& p) {
  const int64_t wgs = (int64_t)p.rows * p.splits;
  const int64_t resident = resident_workgroups(wgs, p.cus);
  return p.order_ws && wgs > resident && wgs <= kOrderMaxRounds * resident;
}

// Enqueue the bin and order kernels (the caller has checked wants_order);
// returns the order to follow.
const int32_t* launch_order(const Params& p, hipStream_t stream) {
  // The workspace's order area holds the bins ([rows] after the order).
  int32_t* bins = p.order_ws + p.rows;
  const int64_t max_tokens = (int64_t)p.R * p.rt;
  const dim3 bin_grid((unsigned)((p.rows + 3) / 4));  // one wave per row
  static_assert(kMaxRegions <= 64 * 32, "at most 32 region-id loads per lane");
  if (p.R <= 64)
    hipLaunchKernelGGL(bin_kernel<1>, bin_grid, dim3(256), 0, stream, p, max_tokens, bins);
  else if (p.R <= 64 * 2)
    hipLaunchKernelGGL(bin_kernel<2>, bin_grid, dim3(256), 0, stream, p, max_tokens, bins);
  else if (p.R <= 64 * 4)
    hipLaunchKernelGGL(bin_kernel<4>, bin_grid, dim3(256), 0, stream, p, max_tokens, bins);
  else if (p.R <= 64 * 8)
    hipLaunchKernelGGL(bin_kernel<8>, bin_grid, dim3(256), 0, stream, p, max_tokens, bins);
  else if (p.R <= 64 * 16)
    hipLaunchKernelGGL(bin_kernel<16>, bin_grid, dim3(256), 0, stream, p, max_tokens, bins);
  else
    hipLaunchKernelGGL(bin_kernel<32>, bin_grid, dim3(256), 0, stream, p, max_tokens, bins);
  hipLaunchKernelGGL(order_kernel, dim3((unsigned)((p.rows + kOrderBlock - 1) / kOrderBlock)),
                     dim3(kOrderBlock), 0, stream, p, (const int32_t*)bins);
  return p.order_ws;
}

template <bool kFp8, bool kFused, int kAddr>
void launch_split(const Params& p, unsigned wgs, hipStream_t stream) {
  const dim3 grid(wgs, (unsigned)p.splits);
  if (two_per_cu((int64_t)wgs * p.splits, p.cus))
    hipLaunchKernelGGL((split_kernel<kFp8, kFused, kAddr, kWavesLargeGrid>), grid,
                       dim3(64 * kWavesLargeGrid), 0, stream, p);
  else
    hipLaunchKernelGGL((split_kernel<kFp8, kFused, kAddr, kWavesSmallGrid>), grid,
                       dim3(64 * kWavesSmallGrid), 0, stream, p);
}

template <bool kFp8, bool kFused>
void launch_region_list(const Params& p, hipStream_t stream) {
  const unsigned wgs = (unsigned)p.rows;
  if (p.rt % Cfg<kFp8>::kTok == 0)
    launch_split<kFp8, kFused, kUniform>(p, wgs, stream);
  else if (2 * p.rt == Cfg<kFp8>::kTok)
    launch_split<kFp8, kFused, kPair>(p, wgs, stream);
  else if (kFp8 && p.rt == 8)
    launch_split<kFp8, kFused, kFp8 ? kQuad : kGeneral>(p, wgs, stream);
  else
    launch_split<kFp8, kFused, kGeneral>(p, wgs, stream);
}

// The row-stream kernel serves fused calls with at least two rows per wave
// of the chip (one 4-wave workgroup per CU), at most kStreamMaxRows rows per
// wave whose lists fit the wave's kStreamList entries, and an output on
// 16-byte boundaries.
bool use_row_stream(const Params& p) {
  if (p.splits != 1 || !p.wide_out || p.R > kStreamMaxR || p.cus <= 0) return false;
  const int64_t waves = (int64_t)kStreamWaves * p.cus;
  const int64_t per_wave = (p.rows + waves - 1) / waves;
  return p.rows >= 2 * waves && per_wave <= kStreamMaxRows && per_wave * p.R <= kStreamList;
}

template <bool kFp8, int kAddr>
void launch_row_stream_addr(const Params& p, hipStream_t stream) {
  const dim3 grid((unsigned)p.cus), block(64 * kStreamWaves);
  if (p.nt_out)
    hipLaunchKernelGGL((row_stream_kernel<kFp8, kAddr, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((row_stream_kernel<kFp8, kAddr, false>), grid, block, 0, stream, p);
}

template <bool kFp8>
void launch_row_stream(const Params& p, hipStream_t stream) {
  if (p.rt % Cfg<kFp8>::kTok == 0)
    launch_row_stream_addr<kFp8, kUniform>(p, stream);
  else if (2 * p.rt == Cfg<kFp8>::kTok)
    launch_row_stream_addr<kFp8, kPair>(p, stream);
  else if (kFp8 && p.rt == 8)
    launch_row_stream_addr<kFp8, kFp8 ? kQuad : kGeneral>(p, stream);
  else
    launch_row_stream_addr<kFp8, kGeneral>(p, stream);
}

template <bool kFp8>
void launch_dtype(const Params& p, hipStream_t stream) {
  if (use_row_stream(p))
    launch_row_stream<kFp8>(p, stream);
  else if (p.splits == 1)
    launch_region_list<kFp8, true>(p, stream);
  else
    launch_region_list<kFp8, false>(p, stream);
}

hipError_t launch_combine(const Params& p, hipStream_t stream) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)p.rows, (unsigned)p.heads), dim3(64), 0, stream,
                     p);
  return hipGetLastError();
}

}  // namespace

// Output bytes per call from which the fused output is stored non-temporally
// (0.5 MiB per XCD, against its 4 MiB L2).  Measured on MI355X, back to
// back, non-temporal vs cacheable stores: 25 MB (large-batch FP8) 534 ->
// 503 us and 6.3 MB (sliding-window gated) 134.4 -> 130.4 us; 1.5 and 3 MB
// (bf16 gated, FP8 cache) unchanged; 3 MB (multi-token) 133.4 -> 135.9 us.
static constexpr int64_t kNtOutputBytes = int64_t(4) << 20;

static bool large_output(const Params& p) {
  return (int64_t)p.rows * p.heads * kDim * 2 >= kNtOutputBytes;
}

// Output rows and heads on 16-byte boundaries: the fused epilogue stores 8
// dims per thread.
static bool wide_output(const Params& p) {
  return (reinterpret_cast<uintptr_t>(p.out) & 15) == 0 && p.ots % 8 == 0 && p.ogs % 8 == 0 &&
         p.ohs % 8 == 0;
}

static Params with_output_policy(const Params& p0) {
  Params p = p0;
  p.nt_out = large_output(p) ? 1 : 0;
  p.wide_out = wide_output(p) ? 1 : 0;
  return p;
}

int plan(const Params& p0) {
  const Params p = with_output_policy(p0);
  if (use_row_stream(p)) return kPlanRowStream;
  return (wants_order(p) ? kPlanOrder : 0) | kPlanSplit | (p.splits > 1 ? kPlanCombine : 0);
}

hipError_t launch(const Params& p0, bool fp8, hipStream_t stream) {
  Params p = with_output_policy(p0);
  p.order = !use_row_stream(p) && wants_order(p) ? launch_order(p, stream) : nullptr;
  if (fp8)
    launch_dtype<true>(p, stream);
  else
    launch_dtype<false>(p, stream);
  return launch_combine(p, stream);
}

hipError_t launch_window(const Params& p0, hipStream_t stream) {
  Params p = p0;
  p.nt_out = large_output(p) ? 1 : 0;
  p.wide_out = wide_output(p) ? 1 : 0;
  // grid.x = requests * token groups * KV groups; the combine runs per row.
  const unsigned wgs = (unsigned)(p.rows / p.rows_per_req * p.ntg * p.groups);
  if (p.splits == 1)
    launch_split<false, true, kWindow>(p, wgs, stream);
  else
    launch_split<false, false, kWindow>(p, wgs, stream);
  return launch_combine(p, stream);
}

}  // namespace sda
