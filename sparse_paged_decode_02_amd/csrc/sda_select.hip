// Region selection for gfx950 (MI355X): per row, the `topk` regions that the
// sparse decode attends.  The operation is `select_regions` on the page
// "vllm.models.step5.nvidia.flashinfer_sparse" as `select_and_run_decode_
// attention` calls it (`sort=False`): an unsorted top-k over the row's region
// scores, limited to the row's first topk_lengths[r] regions, with the current
// region always selected.  Equal scores go to the lower region id (-0.0 ranks
// below +0.0), and the ids are written in ascending order, then -1.
//
// One 256-thread workgroup per row.
//  1. Each thread loads its scores (ids tid + 256 i) as order-preserving
//     32-bit keys into registers.
//  2. Radix select of the threshold key T: three MSB-first passes of 12, 12
//     and 8 bits.  Each pass histograms the keys that match the prefix found
//     so far (LDS atomics), and a block scan from the top bin finds the digit
//     where the count of larger keys reaches the number still needed.  After
//     the last pass T is exact, together with how many keys equal to T are
//     taken.
//  3. Ordered compaction over blocks of 256 ids: keys > T, the forced region,
//     and the first needed keys == T in id order are selected.  Wave ballots
//     and one barrier per block give each selected id its output slot, so the
//     output is ascending and deterministic.
// The bytes are the row's scores (read once) and the output; the work is
// LDS-atomic and scan bound for long rows, latency bound for short ones.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sda_launch.h"

namespace sda {
namespace {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kHistBins = 4096;

// Keys that order like the floats: flip all bits of negatives, set the sign
// bit of non-negatives.  -0.0 -> 0x7FFFFFFF < +0.0 -> 0x80000000.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lanes_below(uint64_t mask, int lane) {
  return __popcll(mask & ((1ull << lane) - 1ull));
}

// Inclusive scan of v over the workgroup in thread order; `total` gets the sum.
__device__ __forceinline__ int block_inclusive_scan(int v, int* s_w, int tid, int& total) {
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d);
    if (lane >= d) v += u;
  }
  if (lane == 63) s_w[wave] = v;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int t = s_w[w];
    before += w < wave ? t : 0;
    total += t;
  }
  __syncthreads();
  return v + before;
}

// Digit d of a histogram with nb bins such that the count of keys in bins
// above d is < need <= the count in bins >= d.  Returns d; `above` gets the
// count in bins above d.  Thread t scans bins [nb - bpt (t+1), nb - bpt t).
__device__ __forceinline__ int find_digit(const int* hist, int nb, int need, int* s_w,
                                          int* s_pick, int tid, int& above) {
  const int bpt = nb / kSelThreads;
  const int hi = nb - bpt * tid;  // exclusive top of this thread's bins
  int local = 0;
  for (int b = hi - 1; b >= hi - bpt; --b) local += hist[b];
  int total;
  const int incl = block_inclusive_scan(local, s_w, tid, total);
  const int excl = incl - local;
  if (excl < need && need <= incl) {
    int run = excl;
    for (int b = hi - 1; b >= hi - bpt; --b) {
      if (run + hist[b] >= need) {
        s_pick[0] = b;
        s_pick[1] = run;
        break;
      }
      run += hist[b];
    }
  }
  __syncthreads();
  above = s_pick[1];
  const int d = s_pick[0];
  __syncthreads();
  return d;
}

template <int KPT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(const SelParams p) {
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int hist[kHistBins];
  __shared__ int s_w[kSelWaves];
  __shared__ int s_pick[2];
  __shared__ int s_cnt[2][kSelWaves][2];  // per block (double-buffered): gt-or-forced, eq

  int n = p.lengths ? p.lengths[r] : p.S;
  n = n < 0 ? 0 : (n > p.S ? p.S : n);
  const int cur = p.current[r];
  const bool forced = cur >= 0 && cur < n && p.topk > 0;
  const int curx = forced ? cur : -1;
  const int pool = n - (forced ? 1 : 0);
  const int want = p.topk - (forced ? 1 : 0);
  const int need0 = want < pool ? want : pool;  // pool keys to take
  int32_t* o = p.out + (int64_t)r * p.ors;

  // 1. keys of the pool (0 elsewhere; no float maps to 0 but a NaN)
  const float* srow = p.scores + (int64_t)r * p.srs;
  uint32_t key[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int j = tid + kSelThreads * i;
    key[i] = (j < n && j != curx) ? order_key(srow[j]) : 0u;
  }

  // 2. threshold: every pool key > T is taken, plus need_eq keys == T
  const bool take_all = need0 == pool;
  uint32_t T = 0;
  int need_eq = 0;
  if (!take_all && need0 > 0) {
    uint32_t prefix = 0, pmask = 0;
    int need = need0;
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
      const int nb = pass == 2 ? 256 : kHistBins;
      const uint32_t dmask = (uint32_t)nb - 1u;
      for (int b = tid; b < nb; b += kSelThreads) hist[b] = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int j = tid + kSelThreads * i;
        if (j < n && j != curx && (key[i] & pmask) == prefix)
          atomicAdd(&hist[(key[i] >> shift) & dmask], 1);
      }
      __syncthreads();
      int above;
      const int d = find_digit(hist, nb, need, s_w, s_pick, tid, above);
      need -= above;
      prefix |= (uint32_t)d << shift;
      pmask |= dmask << shift;
    }
    T = prefix;
    need_eq = need;
  }

  // 3. ordered compaction
  int base = 0, eqbase = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int j = tid + kSelThreads * i;
    const bool v = j < n && j != curx;
    const bool gtf = (v && (take_all || (need0 > 0 && key[i] > T))) || j == curx;
    const bool eq = v && !take_all && need0 > 0 && key[i] == T;
    const uint64_t gm = __ballot(gtf), em = __ballot(eq);
    int(*cnt)[2] = s_cnt[i & 1];
    if (lane == 0) {
      cnt[wave][0] = __popcll(gm);
      cnt[wave][1] = __popcll(em);
    }
    __syncthreads();
    int gtf_prev = 0, eq_prev = 0, gtf_blk = 0, eq_blk = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
      const int g = cnt[w][0], e = cnt[w][1];
      gtf_prev += w < wave ? g : 0;
      eq_prev += w < wave ? e : 0;
      gtf_blk += g;
      eq_blk += e;
    }
    // The first need_eq keys == T in id order are taken.
    const int eq_left = need_eq - eqbase;  // still to take at the start of the block
    const int eq_before = eq_prev + lanes_below(em, lane);
    const bool sel = gtf || (eq && eq_before < eq_left);
    const int eq_sel_prev = min(max(eq_left, 0), eq_prev);
    const int eq_sel_lane = min(max(eq_left - eq_prev, 0), lanes_below(em, lane));
    const int slot = base + gtf_prev + eq_sel_prev + lanes_below(gm, lane) + eq_sel_lane;
    if (sel && slot < p.topk) o[slot] = j;
    base += gtf_blk + min(max(eq_left, 0), eq_blk);
    eqbase += eq_blk;
  }
  // base == (forced ? 1 : 0) + need0 here
  for (int s = base + tid; s < p.topk; s += kSelThreads) o[s] = -1;
}

template <int KPT>
void launch_select(const SelParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(select_kernel<KPT>, dim3((unsigned)p.rows), dim3(kSelThreads), 0, stream,
                     p);
}

}  // namespace

hipError_t launch_select(const SelParams& p, hipStream_t stream) {
  const int kpt = (p.S + kSelThreads - 1) / kSelThreads;
  if (kpt <= 1)
    launch_select<1>(p, stream);
  else if (kpt <= 2)
    launch_select<2>(p, stream);
  else if (kpt <= 4)
    launch_select<4>(p, stream);
  else if (kpt <= 8)
    launch_select<8>(p, stream);
  else if (kpt <= 16)
    launch_select<16>(p, stream);
  else if (kpt <= 32)
    launch_select<32>(p, stream);
  else if (kpt <= 64)
    launch_select<64>(p, stream);
  else
    launch_select<128>(p, stream);
  return hipGetLastError();
}

}  // namespace sda
