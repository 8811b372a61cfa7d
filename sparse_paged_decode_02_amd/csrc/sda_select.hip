// Region selection for gfx950 (MI355X): per row, the `topk` regions that the
// sparse decode attends.  The operation is `select_regions` on the page
// "vllm.models.step5.nvidia.flashinfer_sparse" as `select_and_run_decode_
// attention` calls it (`sort=False`): an unsorted top-k over the row's region
// scores, limited to the row's first topk_lengths[r] regions, with the current
// region always selected.  Equal scores go to the lower region id (-0.0 ranks
// below +0.0), and the ids are written in ascending order, then -1.
//
// One 1024-thread workgroup (16 waves) per row; wave w owns the contiguous
// ids [w L, (w+1) L), L = 256 I, and lane l holds ids w L + 4 l + 256 i + c.
//  1. Keys: 16-byte loads (4-byte ones when the row is not 16-byte aligned)
//     of the scores as order-preserving 32-bit keys, held in registers.
//     Non-candidates get key 0, which no score maps to (NaN aside).
//  2. Threshold key T.  A 12-bit MSB-first radix pass histograms the keys
//     (LDS atomics), and a block scan from the top bin finds the bin where
//     the count of larger keys reaches the number still needed.  That bin's
//     keys (typically 1-3% of the row) go to an LDS list.  With at most
//     kRankCap of them, each listed key is ranked against the whole list
//     (how many are greater, how many equal) by a group of lanes, and the key
//     of the needed rank is T.  Larger bins take two more radix passes (12 and 8 bits) over
//     the list, or over the registers when the bin exceeds the list.  Either
//     way T is exact, together with how many keys equal to T are taken.
//  3. Compaction in id order: keys > T, the forced region and the first
//     needed keys == T are selected.  Each wave counts its selections, one
//     barrier gives every wave its output offset, and each wave then writes
//     its range in order with in-wave scans (no further barriers).
// The bytes are the row's candidate scores (read once) and the output; the
// work is LDS-atomic and scan bound for long rows, latency bound for short
// ones.  The 1024-thread workgroup waits at each of its barriers, so beyond
// one row per CU a second resident workgroup is what hides the waits.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sda.h"
#include "sda_launch.h"
#include "sda_wave.h"

namespace sda {
namespace {

constexpr int kSelThreads = 1024;
static_assert((int64_t)SDA_SELECT_MAX_ROWS * kSelThreads < (int64_t(1) << 32),
              "a grid of SDA_SELECT_MAX_ROWS workgroups fits 2^32 work-items");
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kHistBins = 4096;
constexpr int kCandCap = 4096;  // keys of the first pass's threshold bin kept in LDS
constexpr int kRankCap = 1024;  // listed keys ranked directly (at least one lane each)
static_assert(kRankCap <= kSelThreads && kRankCap + 3 <= kCandCap, "rank list fits");

// Keys that order like the floats: flip all bits of negatives, set the sign
// bit of non-negatives.  -0.0 -> 0x7FFFFFFF < +0.0 -> 0x80000000.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Sums of the 16 per-wave counts cnt[0..15] over waves < upto (uniform) and
// over all: lane w reads wave w's count, one scan, two lane reads.
__device__ __forceinline__ void wave_counts(const int* cnt, int upto, int lane, int& before,
                                            int& all) {
  const int x = wave_inclusive_scan(lane < kSelWaves ? cnt[lane] : 0);
  all = __builtin_amdgcn_readlane(x, kSelWaves - 1);
  before = upto > 0 ? __builtin_amdgcn_readlane(x, upto - 1) : 0;
}

// Lanes below this one whose bit is set in mask.
__device__ __forceinline__ int mbcnt(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Digit d of a histogram with nb bins (nb a multiple of 64, at most 4096)
// such that the count of keys in bins above d is < need <= the count in bins
// >= d.  Wave 0 searches in two levels: lane l sums the per = nb / 64 bins
// [nb - per (l+1), nb - per l); a wave scan from the top finds the lane L
// where the count reaches `need`; then lane l takes bin nb - per L - 1 - l
// of L's range and a second scan finds the bin.  One barrier publishes the
// result through s_pick.  kAllLoads: all of a lane's bins are read at once
// (one LDS round trip, up to 64 VGPRs); otherwise 16 at a time.
template <int NB, bool kAllLoads>
__device__ __forceinline__ int find_digit(const int* hist, int need, int* s_pick, int wave,
                                          int lane, int& above) {
  static_assert(NB % 256 == 0 && NB <= 4096, "bins: a multiple of 256, at most 4096");
  constexpr int nb = NB;
  if (wave == 0) {
    constexpr int per = nb / 64;
    const int hi = nb - per * lane;  // exclusive top of this lane's bins
    int local = 0;
    if (kAllLoads) {
      int4 v4[per / 4];
#pragma unroll
      for (int q = 0; q < per / 4; ++q)
        v4[q] = *reinterpret_cast<const int4*>(hist + hi - per + 4 * q);
#pragma unroll
      for (int q = 0; q < per / 4; ++q) local += v4[q].x + v4[q].y + v4[q].z + v4[q].w;
    } else {
#pragma unroll 4
      for (int q = 0; q < per / 4; ++q) {
        const int4 v = *reinterpret_cast<const int4*>(hist + hi - per + 4 * q);
        local += v.x + v.y + v.z + v.w;
      }
    }
    int total;
    const int excl = wave_exclusive_scan(local, total);
    const uint64_t m1 = __ballot(excl < need && need <= excl + local);
    const int L = (int)__builtin_ctzll(m1);
    const int base = __shfl(excl, L);
    const int top = nb - per * L - 1;  // L's highest bin
    const int v = lane < per ? hist[top - lane] : 0;
    int tot2;
    const int ex2 = base + wave_exclusive_scan(v, tot2);
    const uint64_t m2 = __ballot(lane < per && ex2 < need && need <= ex2 + v);
    const int L2 = (int)__builtin_ctzll(m2);
    if (lane == L2) {
      s_pick[0] = top - L2;
      s_pick[1] = ex2;
    }
  }
  __syncthreads();
  above = s_pick[1];
  return s_pick[0];
}

// kShared: up to 16 keys per lane the kernel fits 64 VGPRs, so two
// workgroups share a CU (8 waves per SIMD).  Otherwise (one workgroup per
// CU: few rows, or 32 keys per lane) registers buy latency instead.
template <int I, bool kShared>
__global__ __launch_bounds__(kSelThreads) __attribute__((amdgpu_waves_per_eu(kShared ? 8 : 4)))
void select_kernel(const SelParams p) {
  static_assert(!kShared || I <= 4, "32 keys per lane do not fit 64 VGPRs");
  constexpr bool kAllLoads = !kShared && I <= 4;  // find_digit's bins in one round trip
  constexpr int K4 = 4 * I;  // keys per lane
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // 64 padding bins past the histogram take the invalid keys of pass 1
  // (one per lane, so they never contend), which keeps that pass branch-free.
  __shared__ __attribute__((aligned(16))) int hist[kHistBins + 64];
  __shared__ int s_pick[3];
  __shared__ int s_cnt[2][kSelWaves];  // [taken outright | eq][wave]
  __shared__ __attribute__((aligned(16))) uint32_t s_ckey[kCandCap + 4];

  int n = p.lengths ? p.lengths[r] : p.S;
  n = n < 0 ? 0 : (n > p.S ? p.S : n);
  const int cur = p.current[r];
  const bool forced = cur >= 0 && cur < n && p.topk > 0;
  const int curx = forced ? cur : -1;
  const int pool = n - (forced ? 1 : 0);
  const int want = p.topk - (forced ? 1 : 0);
  const int need0 = want < pool ? want : pool;  // pool keys to take
  int32_t* o = p.out + (int64_t)r * p.ors;
  const int id0 = wave * (256 * I) + 4 * lane;  // id of key[4 i + c] = id0 + 256 i + c

  // 1. keys of the pool (0 elsewhere)
  const float* srow = p.scores + (int64_t)r * p.srs;
  // 16-byte loads when every 4-id group below n lies in the row (the row is
  // 16-byte aligned and n is a multiple of 4); 4-byte loads otherwise.  The
  // choice is per row, so each path issues all its loads back to back.
  const bool vec = ((uintptr_t)srow & 15u) == 0 && (n & 3) == 0;
  float sc[K4];
  if (vec) {
#pragma unroll
    for (int i = 0; i < I; ++i) {
      const int j = id0 + 256 * i;
      float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j < n) f = *reinterpret_cast<const float4*>(srow + j);
      sc[4 * i + 0] = f.x;
      sc[4 * i + 1] = f.y;
      sc[4 * i + 2] = f.z;
      sc[4 * i + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < I; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = id0 + 256 * i + c;
        sc[4 * i + c] = j < n ? srow[j] : 0.f;
      }
  }
  // The histogram is cleared while the scores are in flight: the barrier
  // publishes LDS only (a full __syncthreads() fence would wait for the
  // loads), and the keys are formed after it.
  const bool take_all = need0 == pool;
  const bool radix = !take_all && need0 > 0;
  if (radix) {
    for (int b = tid; b < kHistBins; b += kSelThreads) hist[b] = 0;
    __asm__ __volatile__("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  uint32_t key[K4];
#pragma unroll
  for (int i = 0; i < I; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = id0 + 256 * i + c;
      key[4 * i + c] = (j < n && j != curx) ? order_key(sc[4 * i + c]) : 0u;
    }

  // 2. threshold: every pool key > T is taken, plus need_eq keys == T
  uint32_t T = 0;
  int need_eq = 0, eq_total = 0;
  if (radix) {
    // pass 1 (bits 31..20) over the registers (histogram cleared above)
#pragma unroll
    for (int k = 0; k < K4; ++k)
      atomicAdd(&hist[key[k] != 0u ? (int)(key[k] >> 20) : kHistBins + lane], 1);
    __syncthreads();
    int above;
    const int d1 = find_digit<kHistBins, kAllLoads>(hist, need0, s_pick, wave, lane, above);
    int need = need0 - above;
    uint32_t prefix = (uint32_t)d1 << 20, pmask = 0xFFF00000u;
    const int inbin = hist[d1];
    const bool listed = inbin <= kCandCap;
    const bool ranked = inbin <= kRankCap;
    if (listed) {
      // The keys of bin d1 (typically a few percent) go to an LDS list; the
      // other two passes run over it.  Per-wave counts, one barrier, then
      // each wave writes at its offset.
      uint32_t cbits = 0;
#pragma unroll
      for (int k = 0; k < K4; ++k)
        cbits |= (key[k] != 0u && (key[k] >> 20) == (uint32_t)d1 ? 1u : 0u) << k;
      int cw;
      int off = wave_exclusive_scan(__popc(cbits), cw);
      if (lane == 0) s_cnt[0][wave] = cw;
      __syncthreads();
      int before, all;
      wave_counts(s_cnt[0], wave, lane, before, all);
      off += before;
      while (cbits) {  // a lane has ~0.1-1 candidates: order within the list is free
        const int k = __builtin_ctz(cbits);
        cbits &= cbits - 1u;
        uint32_t kk = 0;
#pragma unroll
        for (int q = 0; q < K4; ++q) kk = q == k ? key[q] : kk;
        s_ckey[off++] = kk;
      }
      // Key 0 (never a candidate: neither greater nor equal) pads the list
      // to whole 16-byte reads.
      if (ranked && tid < 3) s_ckey[inbin + tid] = 0u;
    }
    __syncthreads();
    if (ranked) {
      // T is the need-th largest listed key: the one with fewer than `need`
      // keys above it and at least `need` at or above it.  A group of P
      // consecutive lanes (P a power of two, inbin * P <= kSelThreads, at
      // most a wave) ranks one listed key, each lane over every P-th 16-byte
      // piece of the list, and the group sums its counts.  Every group
      // holding a key equal to T writes the same three values.
      int P = 1;
      while (P < 64 && inbin * P * 2 <= kSelThreads) P *= 2;
      const int ci = tid / P, part = tid & (P - 1);
      int gt = 0, eq = 0;
      uint32_t kt = 0;
      if (ci < inbin) {
        kt = s_ckey[ci];
        const uint4* l4 = reinterpret_cast<const uint4*>(s_ckey);
#pragma unroll 1
        for (int e = part; e < (inbin + 3) >> 2; e += P) {
          const uint4 v = l4[e];
          gt += (v.x > kt) + (v.y > kt) + (v.z > kt) + (v.w > kt);
          eq += (v.x == kt) + (v.y == kt) + (v.z == kt) + (v.w == kt);
        }
      }
      for (int o = 1; o < P; o <<= 1) {
        gt += __shfl_xor(gt, o);
        eq += __shfl_xor(eq, o);
      }
      if (ci < inbin && part == 0 && gt < need && need <= gt + eq) {
        s_pick[0] = (int)kt;
        s_pick[1] = gt;
        s_pick[2] = eq;
      }
      __syncthreads();
      T = (uint32_t)s_pick[0];
      need_eq = need - s_pick[1];
      eq_total = s_pick[2];
    } else {
#pragma unroll
      for (int pass = 1; pass < 3; ++pass) {
        const int shift = pass == 1 ? 8 : 0;
        const int nb = pass == 2 ? 256 : kHistBins;
        const uint32_t dmask = (uint32_t)nb - 1u;
        for (int b = tid; b < nb; b += kSelThreads) hist[b] = 0;
        __syncthreads();
        if (listed) {
          for (int e = tid; e < inbin; e += kSelThreads) {
            const uint32_t k = s_ckey[e];
            if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1);
          }
        } else {
#pragma unroll
          for (int k = 0; k < K4; ++k)
            if (key[k] != 0u && (key[k] & pmask) == prefix)
              atomicAdd(&hist[(key[k] >> shift) & dmask], 1);
        }
        __syncthreads();
        const int d = pass == 2 ? find_digit<256, kAllLoads>(hist, need, s_pick, wave, lane, above)
                                : find_digit<kHistBins, kAllLoads>(hist, need, s_pick, wave, lane,
                                                                  above);
        need -= above;
        prefix |= (uint32_t)d << shift;
        pmask |= dmask << shift;
        if (pass == 2) eq_total = hist[d];  // pool keys == T
      }
      T = prefix;
      need_eq = need;
    }
  }
  // Without ties at T (all keys == T taken) the selection is key >= T.
  const bool ties = radix && eq_total > need_eq;
  const uint64_t t_take = (uint64_t)T + (ties ? 1u : 0u);  // taken outright: key >= t_take

  // 3. compaction in id order.  gtf: taken outright (key >= t_take, every
  // pool key when all are taken, or the forced region); eq (ties only):
  // key == T, the first need_eq of which in id order are taken.
  auto gtf_of = [&](int k, int id) -> bool {
    return (key[k] != 0u && (take_all || (radix && (uint64_t)key[k] >= t_take))) || id == curx;
  };
  auto eq_of = [&](int k) -> bool { return ties && key[k] == T; };
  // Bit k of tbits: key k is taken outright; of ebits (ties only): key == T.
  uint32_t tbits = 0, ebits = 0;
#pragma unroll
  for (int i = 0; i < I; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      tbits |= (gtf_of(4 * i + c, id0 + 256 * i + c) ? 1u : 0u) << (4 * i + c);
      if (ties) ebits |= (eq_of(4 * i + c) ? 1u : 0u) << (4 * i + c);
    }
  const int g_wave = wave_sum(__popc(tbits));
  const int e_wave = ties ? wave_sum(__popc(ebits)) : 0;
  if (lane == 0) {
    s_cnt[0][wave] = g_wave;
    s_cnt[1][wave] = e_wave;
  }
  __syncthreads();
  int g_prev, g_all, e_prev = 0, e_all = 0;
  wave_counts(s_cnt[0], wave, lane, g_prev, g_all);
  if (ties) wave_counts(s_cnt[1], wave, lane, e_prev, e_all);
  if (!ties) need_eq = 0;
  // output slot of the wave's first selection; eq keys still to take there
  int run = g_prev + min(need_eq, e_prev);
  int eq_left = need_eq - e_prev;
  if (!ties) {
    if (g_wave > 0) {
#pragma unroll
      for (int i = 0; i < I; ++i) {
        // In id order a 256-id group is lane-major: lane l holds ids 4l .. 4l+3.
        const uint32_t nib = (tbits >> (4 * i)) & 15u;
        if (__ballot(nib != 0u) == 0) continue;
        const int c4 = __popc(nib);
        const uint64_t b0 = __ballot(c4 & 1), b1 = __ballot(c4 & 2), b2 = __ballot(c4 & 4);
        int slot = run + mbcnt(b0) + 2 * mbcnt(b1) + 4 * mbcnt(b2);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if ((nib >> c) & 1u) {
            if (slot < p.topk) o[slot] = id0 + 256 * i + c;
            ++slot;
          }
        }
        run += __popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2);
      }
    }
  } else if (g_wave + (eq_left > 0 ? e_wave : 0) > 0) {
#pragma unroll
    for (int i = 0; i < I; ++i) {
      bool gt[4], eq[4];
      int e_lanes = 0, e_tot = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        gt[c] = (tbits >> (4 * i + c)) & 1u;
        eq[c] = eq_left > 0 && ((ebits >> (4 * i + c)) & 1u);
        const uint64_t em = __ballot(eq[c]);
        e_lanes += mbcnt(em);
        e_tot += __popcll(em);
      }
      bool sel[4];
      int eseen = e_lanes;
      int s_lanes = 0, s_tot = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        sel[c] = gt[c] || (eq[c] && eseen < eq_left);
        eseen += eq[c] ? 1 : 0;
        const uint64_t sm = __ballot(sel[c]);
        s_lanes += mbcnt(sm);
        s_tot += __popcll(sm);
      }
      int slot = run + s_lanes;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (sel[c]) {
          if (slot < p.topk) o[slot] = id0 + 256 * i + c;
          ++slot;
        }
      }
      run += s_tot;
      eq_left -= e_tot;
    }
  }
  const int total = g_all + min(need_eq, e_all);  // == (forced ? 1 : 0) + need0
  for (int s = total + tid; s < p.topk; s += kSelThreads) o[s] = -1;
}

// Rows beyond one per CU run two workgroups per CU where the keys fit.
template <int I>
void launch_select(const SelParams& p, hipStream_t stream) {
  if (I <= 4 && p.rows > p.cus)
    hipLaunchKernelGGL((select_kernel<I, I <= 4>), dim3((unsigned)p.rows), dim3(kSelThreads), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((select_kernel<I, false>), dim3((unsigned)p.rows), dim3(kSelThreads), 0,
                       stream, p);
}

}  // namespace

hipError_t launch_select(const SelParams& p, hipStream_t stream) {
  // I groups of 4 keys per lane: 4096 I ids per row
  const int groups = (p.S + 4 * kSelThreads - 1) / (4 * kSelThreads);
  if (groups <= 1)
    launch_select<1>(p, stream);
  else if (groups <= 2)
    launch_select<2>(p, stream);
  else if (groups <= 4)
    launch_select<4>(p, stream);
  else
    launch_select<8>(p, stream);
  return hipGetLastError();
}

}  // namespace sda
