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
// The 256-id groups below the row's length are the live ones; every other
// group holds no candidate, and each phase skips it for the whole wave.
//  1. Keys: 16-byte loads (4-byte ones when the row is not 16-byte aligned)
//     of the scores as order-preserving 32-bit keys, held in registers.
//     Ids past the length read the bit pattern 0xFFFFFFFF, whose key is 0,
//     and the one wave holding the current region clears its key, so key 0
//     marks a non-candidate (no finite score maps to it).
//  2. Threshold key T.  A 12- or 13-bit MSB-first radix pass histograms
//     the keys (LDS atomics; non-candidates land in bin 0, below every
//     finite score).  All threads then read 4 or 8 bins each from the top,
//     one barrier publishes the per-wave totals, and the wave whose range
//     reaches the count still needed finds the bin and publishes it.  That
//     bin's keys (typically under 1% of the row) go to an LDS list, each
//     wave taking its slots from a shared counter.  With at most kRankCap of
//     them, each listed key is ranked against the whole list (how many are
//     greater, how many equal) by a group of lanes, and the key of the
//     needed rank is T.  Larger bins take two more radix passes (down to
//     bit 8, then 8 bits) over the list, or over the registers when the bin
//     exceeds the list.  Either way T is exact, together with how many keys
//     equal to T are taken.
//  3. Compaction in id order.  Without ties at T the selection is key >= T
//     (the current region's key raised to the maximum): per-lane counts of
//     each live group, packed two groups to a word, one wave scan per word,
//     and one barrier for the per-wave offsets; each lane then writes its
//     ids at its own slots.  With ties, keys > T, the current region and
//     the first needed keys == T are selected with ballots per 4-id column.
// The bytes are the row's candidate scores (read once) and the output; the
// work is a chain of barrier-separated phases per row, so beyond one row per
// CU a second resident workgroup is what hides the waits.

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
// Pass 1 takes the top 12 key bits, or 13 (8192 bins, 32 KiB: two
// workgroups still share a CU) for rows of 16 keys per lane: there the
// threshold bin, which the ranking compares pairwise, then holds about half
// the keys.  Passes 2 and 3 (tied or crowded bins) take the bits below down
// to bit 8, then bits 7..0.
template <int I>
struct Pass1 {
  static constexpr int kShift = I >= 4 ? 19 : 20;
  static constexpr int kBins = 1 << (32 - kShift);
  static constexpr int kBinsPerThread = kBins / kSelThreads;
  static constexpr int kP2Bins = 1 << (kShift - 8);
};
constexpr int kCandCap = 4096;  // keys of the first pass's threshold bin kept in LDS
constexpr int kRankCap = 1024;  // listed keys ranked directly (at least one lane each)
constexpr int kRankPad = 4;     // list slots past kCandCap
// The ranking reads 16-byte pieces up to 3 P past the list's last piece
// (P <= 64 lanes per listed key), all zero-padded.
static_assert(kRankCap <= kSelThreads && kRankCap + 3 + 12 * 64 <= kCandCap + kRankPad,
              "rank list fits");

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
// >= d, for the later radix passes (crowded or tied threshold bins).  Wave 0
// searches in two levels: lane l sums the per = nb / 64 bins
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
  constexpr int K4 = 4 * I;                       // keys per lane
  constexpr int kWaveIdsLog2 = I == 1 ? 8 : I == 2 ? 9 : I == 4 ? 10 : 11;
  static_assert((1 << kWaveIdsLog2) == 256 * I, "a wave owns 256 I ids");
  using P1 = Pass1<I>;
  constexpr int kP1Shift = P1::kShift, kHistBins = P1::kBins, kP2Bins = P1::kP2Bins;
  constexpr int kBPT = P1::kBinsPerThread;  // pass-1 bins per thread: 4 or 8
  static_assert(kHistBins == kBPT * kSelThreads && kBPT % 4 == 0, "whole int4 reads");
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __shared__ __attribute__((aligned(16))) int hist[kHistBins];
  __shared__ int s_pick[3];
  __shared__ int s_tot[kSelWaves];      // pass 1: keys per wave's bin range
  __shared__ int s_cnt[2][kSelWaves];   // [taken outright | eq][wave]
  __shared__ int s_fill;                // candidate-list entries handed out
  __shared__ __attribute__((aligned(16))) uint32_t s_ckey[kCandCap + kRankPad];

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
  // 256-id groups holding candidates: group i of wave w is [256 (w I + i), +256)
  const int nlive = (n + 255) >> 8;

  // 1. keys of the pool (0 elsewhere)
  const float* srow = p.scores + (int64_t)r * p.srs;
  // 16-byte loads when every 4-id group below n lies in the row (the row is
  // 16-byte aligned and n is a multiple of 4); 4-byte loads otherwise.  The
  // choice is per row, so each path issues all its loads back to back.
  const bool vec = ((uintptr_t)srow & 15u) == 0 && (n & 3) == 0;
  // Ids at or past n read as the bit pattern 0xFFFFFFFF, whose key is 0.
  const float kNoKey = __uint_as_float(0xFFFFFFFFu);
  float sc[K4];
  if (vec) {
#pragma unroll
    for (int i = 0; i < I; ++i) {
      const int j = id0 + 256 * i;
      float4 f = make_float4(kNoKey, kNoKey, kNoKey, kNoKey);
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
        sc[4 * i + c] = j < n ? srow[j] : kNoKey;
      }
  }
  // The histogram is cleared while the scores are in flight: the barrier
  // publishes LDS only (a full __syncthreads() fence would wait for the
  // loads), and the keys are formed after it.
  const bool take_all = need0 == pool;
  const bool radix = !take_all && need0 > 0;
  if (radix) {
#pragma unroll
    for (int q = 0; q < kBPT / 4; ++q)
      reinterpret_cast<int4*>(hist)[tid + q * kSelThreads] = make_int4(0, 0, 0, 0);
    if (tid == 0) s_fill = 0;
    __asm__ __volatile__("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  // The current region's key is cleared by the one wave that holds it.
  uint32_t key[K4];
#pragma unroll
  for (int k = 0; k < K4; ++k) key[k] = order_key(sc[k]);
  if (forced && (curx >> kWaveIdsLog2) == wave) {
    const int d = curx - id0;
#pragma unroll
    for (int k = 0; k < K4; ++k) key[k] = d == 256 * (k >> 2) + (k & 3) ? 0u : key[k];
  }

  // 2. threshold: every pool key > T is taken, plus need_eq keys == T
  uint32_t T = 0;
  int need_eq = 0, eq_total = 0;
  if (radix) {
    // Pass 1 (bits 31..kP1Shift) over the live groups' keys.  Key 0 (not a
    // candidate) lands in bin 0, which only NaN scores share, so the
    // search below never reaches bin 0 on finite scores.
#pragma unroll
    for (int i = 0; i < I; ++i)
      if (wave * I + i < nlive)
#pragma unroll
        for (int c = 0; c < 4; ++c) atomicAdd(&hist[key[4 * i + c] >> kP1Shift], 1);
    __syncthreads();
    // Digit search by all threads: thread t holds bins kBPT (1023 - t) ..
    // + kBPT - 1, so wave 0 holds the top bins.  Per-wave totals, one
    // barrier, then the wave whose range reaches need0 finds the lane and the
    // bin.
    int hb[kBPT];  // this thread's bins, ascending
    {
      const int4* hist4 = reinterpret_cast<const int4*>(hist);
#pragma unroll
      for (int q = 0; q < kBPT / 4; ++q) {
        const int4 v = hist4[(kBPT / 4) * (kSelThreads - 1 - tid) + q];
        hb[4 * q + 0] = v.x;
        hb[4 * q + 1] = v.y;
        hb[4 * q + 2] = v.z;
        hb[4 * q + 3] = v.w;
      }
    }
    int local = 0;
#pragma unroll
    for (int q = 0; q < kBPT; ++q) local += hb[q];
    int wtot;
    const int excl = wave_exclusive_scan(local, wtot);
    if (lane == 0) s_tot[wave] = wtot;
    __syncthreads();
    {
      const int wx = wave_inclusive_scan(lane < kSelWaves ? s_tot[lane] : 0);
      // the histogram holds 256 nlive >= pool >= need0 keys: W exists
      const int W = (int)__builtin_ctzll(__ballot(lane < kSelWaves && wx >= need0));
      if (wave == W) {
        const int wbase = W > 0 ? __builtin_amdgcn_readlane(wx, W - 1) : 0;
        const int c0 = wbase + excl;
        if (c0 < need0 && need0 <= c0 + local) {  // exactly one lane
          // its bins from the top: j steps down to the first where the count
          // reaches need0
          int c = c0, j = 0;
#pragma unroll
          for (int q = 0; q < kBPT - 1; ++q)
            if (j == q && need0 > c + hb[kBPT - 1 - q]) {
              c += hb[kBPT - 1 - q];
              j = q + 1;
            }
          int cnt = hb[kBPT - 1];
#pragma unroll
          for (int q = 1; q < kBPT; ++q) cnt = j == q ? hb[kBPT - 1 - q] : cnt;
          s_pick[0] = kBPT * (kSelThreads - 1 - tid) + kBPT - 1 - j;
          s_pick[1] = c;
          s_pick[2] = cnt;
        }
      }
    }
    __syncthreads();
    const int d1 = s_pick[0];
    int need = need0 - s_pick[1];
    const int inbin = s_pick[2];
    uint32_t prefix = (uint32_t)d1 << kP1Shift, pmask = ~((1u << kP1Shift) - 1u);
    const bool listed = inbin <= kCandCap;
    const bool ranked = inbin <= kRankCap;
    // ranking: a group of P lanes per listed key (P a power of two, at most a
    // wave, inbin * P <= kSelThreads), each lane over 16-byte pieces part,
    // part + P, ... of the list, four at a time
    int P = 1;
    while (P < 64 && inbin * P * 2 <= kSelThreads) P *= 2;
    const int pieces = (inbin + 3) >> 2;
    if (listed) {
      // The keys of bin d1 (typically a few percent) go to an LDS list.  Each
      // wave takes its slots from a shared counter (list order is free).
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < I; ++i)
        if (wave * I + i < nlive)
#pragma unroll
          for (int c = 0; c < 4; ++c) cnt += (key[4 * i + c] - prefix) < (1u << kP1Shift) ? 1 : 0;
      int cw;
      int off = wave_exclusive_scan(cnt, cw);
      if (cw > 0) {
        int base = 0;
        if (lane == 0) base = atomicAdd(&s_fill, cw);
        off += __builtin_amdgcn_readlane(base, 0);
#pragma unroll
        for (int i = 0; i < I; ++i)
          if (wave * I + i < nlive)
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if ((key[4 * i + c] - prefix) < (1u << kP1Shift)) s_ckey[off++] = key[4 * i + c];
      }
      // Key 0 (never a candidate: neither greater nor equal) pads the list
      // to every piece the unrolled ranking reads.
      if (ranked && tid < 4 * (pieces + 3 * P) - inbin) s_ckey[inbin + tid] = 0u;
    }
    __syncthreads();
    if (ranked) {
      // T is the need-th largest listed key: the one with fewer than `need`
      // keys above it and at least `need` at or above it.  Every group
      // holding a key equal to T writes the same three values.
      const int ci = tid / P, part = tid & (P - 1);
      int gt = 0, eq = 0;
      uint32_t kt = 0;
      if (ci < inbin) {
        kt = s_ckey[ci];
        const uint4* l4 = reinterpret_cast<const uint4*>(s_ckey);
#pragma unroll 1
        for (int e = part; e < pieces; e += 4 * P) {
          uint4 v[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = l4[e + u * P];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            gt += (v[u].x > kt) + (v[u].y > kt) + (v[u].z > kt) + (v[u].w > kt);
            eq += (v[u].x == kt) + (v[u].y == kt) + (v[u].z == kt) + (v[u].w == kt);
          }
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
        const int nb = pass == 2 ? 256 : kP2Bins;
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
          for (int i = 0; i < I; ++i)
            if (wave * I + i < nlive)
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                const uint32_t k = key[4 * i + c];
                if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1);
              }
        }
        __syncthreads();
        int above;
        const int d = pass == 2 ? find_digit<256, kAllLoads>(hist, need, s_pick, wave, lane, above)
                                : find_digit<kP2Bins, kAllLoads>(hist, need, s_pick, wave, lane,
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

  // 3. compaction in id order
  if (!ties) {
    // Selected: key >= t_sel.  Key 0 marks a non-candidate, so t_sel >= 1;
    // the current region's key becomes the largest key, which every t_sel
    // takes (with nothing else to take, t_sel is that key alone).
    const uint32_t t_sel = take_all ? 1u : !radix ? 0xFFFFFFFFu : (T > 1u ? T : 1u);
    if (forced && (curx >> kWaveIdsLog2) == wave) {
      const int d = curx - id0;
#pragma unroll
      for (int k = 0; k < K4; ++k) key[k] = d == 256 * (k >> 2) + (k & 3) ? 0xFFFFFFFFu : key[k];
    }
    // Per-lane counts of each live group, two groups per 32-bit word (a
    // group's total over the wave is at most 256), one wave scan per word.
    constexpr int W2 = (I + 1) / 2;
    int pre[W2], tot[W2];
    int g_wave = 0;
#pragma unroll
    for (int h = 0; h < W2; ++h) {
      int v = 0;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int i = 2 * h + s;
        if (i < I && wave * I + i < nlive) {
          int c4 = 0;
#pragma unroll
          for (int c = 0; c < 4; ++c) c4 += key[4 * i + c] >= t_sel ? 1 : 0;
          v += c4 << (16 * s);
        }
      }
      pre[h] = wave_exclusive_scan(v, tot[h]);
      g_wave += (tot[h] & 0xFFFF) + ((uint32_t)tot[h] >> 16);
    }
    if (lane == 0) s_cnt[0][wave] = g_wave;
    __syncthreads();
    int g_prev, g_all;
    wave_counts(s_cnt[0], wave, lane, g_prev, g_all);
    int run = g_prev;  // output slot of this wave's first selection
#pragma unroll
    for (int i = 0; i < I; ++i) {
      if (wave * I + i >= nlive) break;
      const int h = i >> 1, s = 16 * (i & 1);
      const int gtot = (int)(((uint32_t)tot[h] >> s) & 0xFFFFu);
      if (gtot > 0) {
        int slot = run + (int)(((uint32_t)pre[h] >> s) & 0xFFFFu);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (key[4 * i + c] >= t_sel) {
            if (slot < p.topk) o[slot] = id0 + 256 * i + c;
            ++slot;
          }
        }
      }
      run += gtot;
    }
    for (int s = g_all + tid; s < p.topk; s += kSelThreads) o[s] = -1;
    return;
  }

  // Ties at T: keys > T and the current region are taken outright; of the
  // keys == T, the first need_eq in id order.
  auto gtf_of = [&](int k, int id) -> bool { return key[k] > T || id == curx; };
  auto eq_of = [&](int k) -> bool { return key[k] == T && T != 0u; };
  uint32_t tbits = 0, ebits = 0;
#pragma unroll
  for (int i = 0; i < I; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      tbits |= (gtf_of(4 * i + c, id0 + 256 * i + c) ? 1u : 0u) << (4 * i + c);
      ebits |= (eq_of(4 * i + c) ? 1u : 0u) << (4 * i + c);
    }
  const int g_wave = wave_sum(__popc(tbits));
  const int e_wave = wave_sum(__popc(ebits));
  if (lane == 0) {
    s_cnt[0][wave] = g_wave;
    s_cnt[1][wave] = e_wave;
  }
  __syncthreads();
  int g_prev, g_all, e_prev, e_all;
  wave_counts(s_cnt[0], wave, lane, g_prev, g_all);
  wave_counts(s_cnt[1], wave, lane, e_prev, e_all);
  // output slot of the wave's first selection; eq keys still to take there
  int run = g_prev + min(need_eq, e_prev);
  int eq_left = need_eq - e_prev;
  if (g_wave + (eq_left > 0 ? e_wave : 0) > 0) {
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
