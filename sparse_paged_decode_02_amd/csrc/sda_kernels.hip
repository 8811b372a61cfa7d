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
// Split kernel: one 256-thread workgroup (4 waves of 64) per (row, split).
//  * Prologue: the workgroup ranks the row's visible region slots, takes its
//    balanced share of them, and resolves each region to a cache offset
//    through the block table.  Only that share's block-table entries are
//    read.  The offsets go into LDS.
//  * Main loop: each wave owns chunks of 32 token slots.  For every chunk it
//    issues the next chunk's K|V loads before computing on the current one.
//    The loads are 16-byte global loads into registers, in MFMA operand
//    layout, so K never touches LDS.
//      S^T[tok, head] = K[tok, :] . Q^T[:, head]
//          12 x v_mfma_f32_16x16x32_bf16 (2 token tiles x 6 dim slices)
//      online softmax per head, in the exp2 domain
//      O^T[dim, head] += V^T[dim, tok] . P^T[tok, head]
//          12 x MFMA (12 dim tiles).  V^T is read from a wave-private,
//          padded LDS tile, and P^T comes straight from the S^T accumulators:
//          the S^T tile already has the B-operand layout.
//    FP8 K and V are converted exactly to bf16 (e4m3 is a subset of bf16).
//    k_scale is folded into the logit scale and v_scale into the final
//    normalisation.
//  * Epilogue: the 4 waves' (max, sum, acc) states are merged through LDS.
//    With one split, the gate is applied and the result is written as bf16
//    (combine fused).  Otherwise the fp32 partial output and its base-2
//    log-sum-exp go to the workspace.
// Combine kernel (splits > 1): one workgroup per row merges the partials,
// applies the gate and writes bf16, or clears an inactive row.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sda_launch.h"

namespace sda {
namespace {

constexpr int kDim = 192;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 32;       // token slots per wave iteration (2 MFMA tiles)
constexpr int kVStride = 208;    // bf16 per LDS V row: 192 + 16 pad; 104 dwords,
                                 // so the 4 token rows one V^T read touches
                                 // land 8 banks apart
constexpr int kAccStride = 196;  // floats per head row in the wave-merge area

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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
__device__ __forceinline__ float gate_value(const uint16_t* gate, int64_t idx) {
  float g = bf16_bits_to_float(gate[idx]);
  float den = 1.0f + expf(-g);
  float sig = 1.0f / den;
  return bf16_bits_to_float(float_to_bf16_bits(sig));
}

__device__ __forceinline__ u32x4 load16(const uint8_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// 4 e4m3 bytes -> 4 bf16 (exact): {bytes 0,1 ; bytes 2,3} as two packed pairs.
__device__ __forceinline__ u32x2 fp8x4_to_bf16(uint32_t w) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
}

// Dim offset of the 8 elements lane group g4 supplies to MFMA k-slice cc.
// bf16 loads 8 elements per 16-byte load: slice cc covers [32cc, 32cc+32).
// FP8 loads 16 elements per load, feeding slices 2pp and 2pp+1.
template <bool kFp8>
__device__ __forceinline__ int slice_dim(int cc, int g4) {
  return kFp8 ? 64 * (cc >> 1) + 16 * g4 + 8 * (cc & 1) : 32 * cc + 8 * g4;
}

template <bool kFp8>
struct ChunkRegs {
  static constexpr int kLoads = kFp8 ? 3 : 6;  // 16-byte loads per token half-row
  u32x4 k[2][kLoads];
  u32x4 v[2][kLoads];
  bool valid[2];
};

struct RowState {
  f32x4 acc[12];   // O^T tiles: lane holds head (lane&15), dims 16nt+4*(lane>>4)+v
  float m;         // running max (base-2 logit units), same in the 4 lanes of a head
  float l;         // this lane's part of the running sum
};

// Token slot of MFMA row i of tile t within a chunk.  The interleave makes the
// 4 tokens that one V^T read touches (fixed t and v, lane groups g4 = 0..3)
// consecutive LDS rows.
__device__ __forceinline__ int chunk_token(int t, int i) { return 16 * t + 4 * (i & 3) + (i >> 2); }

template <bool kFp8>
__device__ __forceinline__ void issue_chunk(const Params& p, int c, int nreg,
                                            const int64_t* s_base, const int* s_n,
                                            int lane, ChunkRegs<kFp8>& cr) {
  const int i16 = lane & 15, g4 = lane >> 4;
  constexpr int kEsz = kFp8 ? 1 : 2;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    int slot = c * kChunk + chunk_token(t, i16);
    int k = slot / p.rt;
    int off = slot - k * p.rt;
    bool valid = k < nreg && off < s_n[k < nreg ? k : 0];
    cr.valid[t] = valid;
    if (valid) {
      const uint8_t* row = p.cache + (s_base[k] + (int64_t)off * p.cts) * kEsz;
#pragma unroll
      for (int u = 0; u < ChunkRegs<kFp8>::kLoads; ++u) {
        int d = kFp8 ? 64 * u + 16 * g4 : 32 * u + 8 * g4;
        cr.k[t][u] = load16(row + d * kEsz);
        cr.v[t][u] = load16(row + (kDim + d) * kEsz);
      }
    } else {
#pragma unroll
      for (int u = 0; u < ChunkRegs<kFp8>::kLoads; ++u) {
        cr.k[t][u] = u32x4{0, 0, 0, 0};
        cr.v[t][u] = u32x4{0, 0, 0, 0};
      }
    }
  }
}

template <bool kFp8>
__device__ __forceinline__ void compute_chunk(const ChunkRegs<kFp8>& cr, const u32x4 (&qreg)[6],
                                              float qk_scale_log2, uint16_t (*s_vw)[kVStride],
                                              int lane, RowState& st) {
  const int i16 = lane & 15, g4 = lane >> 4;

  // V rows of this lane's two tokens -> wave-private LDS tile (bf16, row = token slot).
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    uint16_t* vrow = s_vw[chunk_token(t, i16)];
#pragma unroll
    for (int u = 0; u < ChunkRegs<kFp8>::kLoads; ++u) {
      if (kFp8) {
        u32x4 w = cr.v[t][u];
        u32x2 w0 = fp8x4_to_bf16(w[0]), w1 = fp8x4_to_bf16(w[1]);
        u32x2 w2 = fp8x4_to_bf16(w[2]), w3 = fp8x4_to_bf16(w[3]);
        u32x4 a = {w0[0], w0[1], w1[0], w1[1]};
        u32x4 b = {w2[0], w2[1], w3[0], w3[1]};
        int d = 64 * u + 16 * g4;
        *reinterpret_cast<u32x4*>(vrow + d) = a;
        *reinterpret_cast<u32x4*>(vrow + d + 8) = b;
      } else {
        *reinterpret_cast<u32x4*>(vrow + 32 * u + 8 * g4) = cr.v[t][u];
      }
    }
  }

  // S^T tiles: rows = token slots chunk_token(t, 4*g4 + v), columns = heads.
  f32x4 s[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < 6; ++cc) {
      u32x4 kb;
      if (kFp8) {
        uint32_t w0 = cr.k[t][cc >> 1][(cc & 1) * 2 + 0];
        uint32_t w1 = cr.k[t][cc >> 1][(cc & 1) * 2 + 1];
        u32x2 c0 = fp8x4_to_bf16(w0), c1 = fp8x4_to_bf16(w1);
        kb = u32x4{c0[0], c0[1], c1[0], c1[1]};
      } else {
        kb = cr.k[t][cc];
      }
      a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb),
                                                  __builtin_bit_cast(bf16x8, qreg[cc]), a, 0, 0, 0);
    }
    s[t] = a;
  }

  // Which token rows are real: lanes 0..15 loaded rows 0..15 of each tile.
  uint64_t vb0 = __ballot(cr.valid[0]);
  uint64_t vb1 = __ballot(cr.valid[1]);

  float x[2][4];
  float mloc = -INFINITY;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    int bit = 4 * g4 + v;
    x[0][v] = ((vb0 >> bit) & 1) ? s[0][v] * qk_scale_log2 : -INFINITY;
    x[1][v] = ((vb1 >> bit) & 1) ? s[1][v] * qk_scale_log2 : -INFINITY;
    mloc = fmaxf(mloc, fmaxf(x[0][v], x[1][v]));
  }
  mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
  float m_new = fmaxf(st.m, mloc);
  float m_use = m_new == -INFINITY ? 0.f : m_new;
  float alpha = __builtin_amdgcn_exp2f(st.m - m_use);
  st.m = m_new;

  // P^T B-operand: element e = 4t + v <-> token chunk_token(t, 4*g4 + v).
  u32x4 pb;
  float psum = 0.f;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int v = 0; v < 4; v += 2) {
      float p0 = __builtin_amdgcn_exp2f(x[t][v] - m_use);
      float p1 = __builtin_amdgcn_exp2f(x[t][v + 1] - m_use);
      uint32_t b0 = float_to_bf16_bits(p0), b1 = float_to_bf16_bits(p1);
      psum += bf16_bits_to_float(b0) + bf16_bits_to_float(b1);
      pb[2 * t + v / 2] = b0 | (b1 << 16);
    }
  }
  st.l = st.l * alpha + psum;
#pragma unroll
  for (int nt = 0; nt < 12; ++nt) st.acc[nt] *= alpha;

  // LDS writes above are from other lanes of this wave; LDS executes a wave's
  // operations in order, so only compiler reordering must be prevented.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const bf16x8 pbv = __builtin_bit_cast(bf16x8, pb);
#pragma unroll
  for (int nt = 0; nt < 12; ++nt) {
    const uint16_t* col = &s_vw[0][16 * nt + i16];
    u32x4 a;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      int t = e >> 2, v = e & 3;
      uint32_t lo = col[(size_t)(16 * t + 4 * v + g4) * kVStride];
      uint32_t hi = col[(size_t)(16 * t + 4 * (v + 1) + g4) * kVStride];
      a[e >> 1] = lo | (hi << 16);
    }
    st.acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), pbv,
                                                         st.acc[nt], 0, 0, 0);
  }

  // The next chunk's LDS writes must not move above these reads.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ void store_row_pair(const Params& p, int r, int h, int d, float o0,
                                               float o1) {
  uint32_t v = float_to_bf16_bits(o0) | (float_to_bf16_bits(o1) << 16);
  *reinterpret_cast<uint32_t*>(p.out + (int64_t)r * p.ors + (int64_t)h * p.ohs + d) = v;
}

__device__ __forceinline__ void clear_row(const Params& p, int r) {
  for (int e = threadIdx.x; e < p.heads * (kDim / 2); e += kThreads) {
    int h = e / (kDim / 2), d = 2 * (e - h * (kDim / 2));
    *reinterpret_cast<uint32_t*>(p.out + (int64_t)r * p.ors + (int64_t)h * p.ohs + d) = 0u;
  }
}

template <bool kFp8, bool kFused>
__global__ __launch_bounds__(kThreads) void split_kernel(const Params p) {
  const int r = blockIdx.x;
  const int split = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  __shared__ int64_t s_base[kMaxRegions];
  __shared__ int s_n[kMaxRegions];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[kWaves][kChunk][kVStride];
  __shared__ int s_cnt[kWaves];
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];

  if (!p.active[r]) {
    // Inactive rows read nothing else.  With splits > 1 the combine clears.
    if (kFused && p.clear) clear_row(p, r);
    return;
  }

  const int pos = p.positions[r];
  const int g = r % p.groups;
  const int req = r / p.rows_per_req;
  const int rt = p.rt;
  const int32_t* reg = p.regions + (int64_t)r * p.rrs;

  // Pass 1: how many slots are visible (id >= 0 and first token <= pos).
  int nvis = 0;
  for (int j0 = 0; j0 < p.R; j0 += kThreads) {
    int j = j0 + tid;
    bool vis = false;
    if (j < p.R) {
      int id = reg[j];
      vis = id >= 0 && (int64_t)id * rt <= pos;
    }
    nvis += __syncthreads_count(vis);
  }
  // Balanced share: split s takes visible ranks [ceil(s*V/S), ceil((s+1)*V/S)).
  const int lo = (int)(((int64_t)split * nvis + p.splits - 1) / p.splits);
  const int hi = (int)(((int64_t)(split + 1) * nvis + p.splits - 1) / p.splits);
  const int nreg = hi - lo;

  // Pass 2: rank the visible slots in slot order; resolve this split's share.
  int base_rank = 0;
  for (int j0 = 0; j0 < p.R; j0 += kThreads) {
    int j = j0 + tid;
    int id = -1;
    bool vis = false;
    if (j < p.R) {
      id = reg[j];
      vis = id >= 0 && (int64_t)id * rt <= pos;
    }
    uint64_t m = __ballot(vis);
    __syncthreads();
    if (lane == 0) s_cnt[wave] = __popcll(m);
    __syncthreads();
    int before = base_rank, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      int cw = s_cnt[w];
      before += w < wave ? cw : 0;
      total += cw;
    }
    int k = before + __popcll(m & ((1ull << lane) - 1ull));
    if (vis && k >= lo && k < hi) {
      int64_t t0 = (int64_t)id * rt;
      int64_t col = t0 / p.block;
      int off0 = (int)(t0 - col * p.block);
      int64_t page = p.table[(int64_t)req * p.trs + col];
      s_base[k - lo] = page * p.cps + (int64_t)g * p.cgs + (int64_t)off0 * p.cts;
      s_n[k - lo] = (int)min((int64_t)rt, (int64_t)pos - t0 + 1);
    }
    base_rank += total;
  }
  __syncthreads();

  // Q^T B-operand: lane holds head (lane & 15), 8 dims per k-slice.
  const int i16 = lane & 15, g4 = lane >> 4;
  u32x4 qreg[6];
  {
    const uint16_t* qrow = p.q + (int64_t)r * p.qrs + (int64_t)i16 * p.qhs;
#pragma unroll
    for (int cc = 0; cc < 6; ++cc) {
      if (i16 < p.heads)
        qreg[cc] = *reinterpret_cast<const u32x4*>(qrow + slice_dim<kFp8>(cc, g4));
      else
        qreg[cc] = u32x4{0, 0, 0, 0};
    }
  }
  const float kscale = kFp8 ? *p.k_scale : 1.0f;
  const float qk_scale_log2 = p.scale * kscale * 1.4426950408889634f;

  RowState st;
#pragma unroll
  for (int nt = 0; nt < 12; ++nt) st.acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;

  const int nchunks = (int)(((int64_t)nreg * rt + kChunk - 1) / kChunk);
  uint16_t(*s_vw)[kVStride] = s_v[wave];

  // Software pipeline: chunk c+kWaves is in flight while chunk c is computed.
  ChunkRegs<kFp8> ra, rb;
  int c = wave;
  if (c < nchunks) issue_chunk<kFp8>(p, c, nreg, s_base, s_n, lane, ra);
  while (c < nchunks) {
    int cn = c + kWaves;
    if (cn < nchunks) issue_chunk<kFp8>(p, cn, nreg, s_base, s_n, lane, rb);
    compute_chunk<kFp8>(ra, qreg, qk_scale_log2, s_vw, lane, st);
    c = cn;
    if (c >= nchunks) break;
    cn = c + kWaves;
    if (cn < nchunks) issue_chunk<kFp8>(p, cn, nreg, s_base, s_n, lane, ra);
    compute_chunk<kFp8>(rb, qreg, qk_scale_log2, s_vw, lane, st);
    c = cn;
  }

  // Merge the 4 waves.  The per-lane sums of a head live in its 4 lane groups.
  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  __syncthreads();  // every wave is done with s_v
  float* s_acc = reinterpret_cast<float*>(&s_v[0][0][0]);  // [kWaves][16][kAccStride]
  static_assert(sizeof(s_v) >= sizeof(float) * kWaves * 16 * kAccStride, "merge area");
#pragma unroll
  for (int nt = 0; nt < 12; ++nt) {
    float* dst = s_acc + ((size_t)wave * 16 + i16) * kAccStride + 16 * nt + 4 * g4;
    *reinterpret_cast<f32x4*>(dst) = st.acc[nt];
  }
  if (g4 == 0) {
    s_m[wave][i16] = st.m;
    s_l[wave][i16] = l;
  }
  __syncthreads();

  const float vscale = kFp8 ? *p.v_scale : 1.0f;
  for (int e = tid; e < p.heads * (kDim / 2); e += kThreads) {
    int h = e / (kDim / 2), d = 2 * (e - h * (kDim / 2));
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
    float o0 = 0.f, o1 = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        float f = __builtin_amdgcn_exp2f(s_m[w][h] - M);
        const float* src = s_acc + ((size_t)w * 16 + h) * kAccStride + d;
        L += s_l[w][h] * f;
        o0 += src[0] * f;
        o1 += src[1] * f;
      }
      float inv = vscale / L;
      o0 *= inv;
      o1 *= inv;
    }
    if (kFused) {
      if (p.gated) {
        float gv = gate_value(p.gate, (int64_t)(r / p.groups) * p.grs +
                                          (int64_t)(g * p.heads + h) * p.ghs);
        o0 *= gv;
        o1 *= gv;
      }
      store_row_pair(p, r, h, d, o0, o1);
    } else {
      int64_t ph = ((int64_t)r * p.splits + split) * p.heads + h;
      *reinterpret_cast<float2*>(p.partial + ph * kDim + d) = make_float2(o0, o1);
      if (d == 0) p.lse[ph] = M == -INFINITY ? -INFINITY : M + __log2f(L);
    }
  }
}

__global__ __launch_bounds__(kThreads) void combine_kernel(const Params p) {
  const int r = blockIdx.x;
  if (!p.active[r]) {
    if (p.clear) clear_row(p, r);
    return;
  }
  const int g = r % p.groups;
  for (int e = threadIdx.x; e < p.heads * (kDim / 2); e += kThreads) {
    int h = e / (kDim / 2), d = 2 * (e - h * (kDim / 2));
    const int64_t ph0 = (int64_t)r * p.splits * p.heads + h;
    float M = -INFINITY;
    for (int s = 0; s < p.splits; ++s) M = fmaxf(M, p.lse[ph0 + (int64_t)s * p.heads]);
    float o0 = 0.f, o1 = 0.f;
    if (M != -INFINITY) {
      float W = 0.f;
      for (int s = 0; s < p.splits; ++s) {
        int64_t ph = ph0 + (int64_t)s * p.heads;
        float w = __builtin_amdgcn_exp2f(p.lse[ph] - M);
        float2 v = *reinterpret_cast<const float2*>(p.partial + ph * kDim + d);
        W += w;
        o0 += w * v.x;
        o1 += w * v.y;
      }
      o0 /= W;
      o1 /= W;
    }
    if (p.gated) {
      float gv = gate_value(p.gate, (int64_t)(r / p.groups) * p.grs +
                                        (int64_t)(g * p.heads + h) * p.ghs);
      o0 *= gv;
      o1 *= gv;
    }
    store_row_pair(p, r, h, d, o0, o1);
  }
}

}  // namespace

hipError_t launch(const Params& p, bool fp8, hipStream_t stream) {
  dim3 grid((unsigned)p.rows, (unsigned)p.splits);
  dim3 block(kThreads);
  const bool fused = p.splits == 1;
  if (fp8) {
    if (fused)
      hipLaunchKernelGGL((split_kernel<true, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((split_kernel<true, false>), grid, block, 0, stream, p);
  } else {
    if (fused)
      hipLaunchKernelGGL((split_kernel<false, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((split_kernel<false, false>), grid, block, 0, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || fused) return e;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)p.rows), block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace sda
