// Gather-ceiling probe (libsda_probe.so, include/sda_probe.h): the split
// kernel's chunk loop with nothing but the loads.  Each workgroup streams its
// list of token blocks through per-wave two-stage LDS pipelines: chunk c of
// the workgroup's concatenated token rows goes to wave c % waves, its 12
// LDS-DMAs are issued while the previous chunk is read back, and the wait is
// the split kernel's vmcnt.  Chunks inside one block take a scalar base plus
// 32-bit lane offsets, blocks of half a chunk pair up (8 bf16 or 16 FP8
// tokens) and FP8 blocks of 8 tokens go four to a chunk under scalar bases,
// and anything else uses per-lane 64-bit addresses, as in the split kernel.  Rows past the end of a workgroup's list load its first token row
// (the split kernel's masked rows load a visible row of their region).
// The library also holds a VALU issue-rate probe (sda_probe_valu): waves of
// independent instructions of one kind, timed to give the SIMD cycles a
// wave64 instruction of that kind occupies.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sda.h"
#include "sda_dma.h"
#include "sda_probe.h"

namespace sda {
namespace {

constexpr int kProbeStages = 2;
constexpr int kValuThreads = 256;

struct ProbeParams {
  const uint8_t* base;
  int64_t ts;  // token stride (bytes)
  const int64_t* offsets;
  const int32_t* start;
  int32_t* sink;
  int32_t tpb;  // token rows per block
};

enum ProbeAddr : int { kProbeGeneral = 0, kProbeUniform = 1, kProbePair = 3, kProbeQuad = 4 };

template <bool kFp8, int kAddr, int kWaves>
__global__ __launch_bounds__(64 * kWaves) void gather_kernel(const ProbeParams p) {
  using C = Cfg<kFp8>;
  constexpr int kThreads = 64 * kWaves;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int64_t s_off[SDA_PROBE_MAX_BLOCKS];
  __shared__ __attribute__((aligned(1024))) uint8_t s_stage[kWaves][kProbeStages][kChunkBytes];

  const int b0 = p.start[blockIdx.x];
  // the LDS list holds SDA_PROBE_MAX_BLOCKS offsets
  const int nb = min(max(p.start[blockIdx.x + 1] - b0, 0), SDA_PROBE_MAX_BLOCKS);
  for (int k = tid; k < nb; k += kThreads) s_off[k] = p.offsets[b0 + k];
  __syncthreads();

  const int total = nb * p.tpb;
  const int nchunks = (total + C::kTok - 1) / C::kTok;
  const uint32_t ts = (uint32_t)p.ts;
  uint32_t seen = 0;
  const uint8_t* my_stage = &s_stage[wave][0][0];
  const uint32_t my_stage_lds = lds_addr(my_stage);
  const LaneDma ld = lane_dma<kFp8>(lane);

  auto issue = [&](int c, uint32_t stage) {
    const uint32_t st = (uint32_t)__builtin_amdgcn_readfirstlane(stage);
    const int slot0 = c * C::kTok;
    uint32_t ko[6], vo[6];
    if (kAddr == kProbeUniform) {
      const int k = slot0 / p.tpb;
      const int off0 = slot0 - k * p.tpb;
      const uint8_t* base = uniform_ptr(p.base + s_off[k] + (int64_t)off0 * p.ts);
#pragma unroll
      for (int j = 0; j < 6; ++j) {
        ko[j] = (uint32_t)ld.row[j] * ts + ld.koff[j];
        vo[j] = (uint32_t)ld.row[j] * ts + ld.voff[j];
      }
      dma_chunk_sbase<kFp8>(base, st, ko, vo);
    } else if (kAddr == kProbePair) {
      // blocks of half a chunk (8 bf16 or 16 FP8 tokens), two to a chunk
      constexpr int kHalf = C::kTok / 2;
      const int k0 = slot0 / kHalf;
      const bool has1 = k0 + 1 < nb;
      const uint8_t* base0 = uniform_ptr(p.base + s_off[k0]);
      const uint8_t* base1 = uniform_ptr(p.base + s_off[has1 ? k0 + 1 : k0]);
#pragma unroll
      for (int j = 0; j < 6; ++j) {
        const uint32_t roff = (uint32_t)(ld.row[j] & (kHalf - 1)) * ts;
        ko[j] = roff + ld.koff[j];
        vo[j] = roff + ld.voff[j];
      }
      dma_chunk_sbase2<kFp8>(base0, base1, st, ko, vo);
    } else if (kAddr == kProbeQuad) {
      // FP8 blocks of 8 tokens, four to a chunk (the split kernel's
      // SDA_CHUNK_ASM_QUAD); blocks past the list load block 4c again.
      const int k0 = slot0 / 8;
      auto blk = [&](int q) { return uniform_ptr(p.base + s_off[k0 + q < nb ? k0 + q : k0]); };
      const uint8_t* const q0 = blk(0);
      const uint8_t* const q1 = blk(1);
      const uint8_t* const q2 = blk(2);
      const uint8_t* const q3 = blk(3);
#pragma unroll
      for (int j = 0; j < 6; ++j) {
        const uint32_t roff = (uint32_t)(ld.row[j] & 7) * ts;
        ko[j] = roff + ld.koff[j];
        vo[j] = roff + ld.voff[j];
      }
      const bool hi = lane >= 32;
      const uint8_t* const l1 = hi ? q1 : q0;
      const uint8_t* const l4 = hi ? q3 : q2;
      dma_chunk_quad(q0, q1, q2, q3, st, ko, vo, l1 + ko[1], l1 + vo[1], l4 + ko[4], l4 + vo[4]);
    } else {
      const uint8_t* ka[6];
      const uint8_t* va[6];
#pragma unroll
      for (int j = 0; j < 6; ++j) {
        int slot = slot0 + ld.row[j];
        if (slot >= total) slot = 0;
        const int k = slot / p.tpb;
        const uint8_t* row = p.base + s_off[k] + (int64_t)(slot - k * p.tpb) * p.ts;
        ka[j] = row + ld.koff[j];
        va[j] = row + ld.voff[j];
      }
      dma_chunk_vaddr<kFp8>(st, ka, va);
    }
  };

  if (wave < nchunks) {
    issue(wave, my_stage_lds);
    for (int i = 0;; ++i) {
      const int c = wave + kWaves * i;
      if (c >= nchunks) break;
      const int cn = c + kWaves;
      const int s = i & 1;
      if (cn < nchunks) {
        issue(cn, my_stage_lds + (s ^ 1) * kChunkBytes);
        wait_vmcnt<kOpsPerChunk>();
      } else {
        wait_vmcnt<0>();
      }
      // the chunk has landed: read one word of it back
      seen += *(const SDA_LDS uint32_t*)((const SDA_LDS uint8_t*)(my_stage + s * kChunkBytes) +
                                         4 * lane);
      // keep the next iteration's DMA behind this read of its stage
      __asm__ __volatile__("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  }
  if (lane == 0) p.sink[blockIdx.x * 4 + wave] = (int32_t)seen;
}

template <bool kFp8, int kAddr>
void launch_gather(const ProbeParams& p, unsigned groups, int cus, hipStream_t stream) {
  // the split kernel's shapes: one 4-wave workgroup per CU for grids of at
  // most one per CU, else 2-wave workgroups, two per CU
  if ((int64_t)groups >= 2 * (int64_t)cus)
    hipLaunchKernelGGL((gather_kernel<kFp8, kAddr, 2>), dim3(groups), dim3(128), 0, stream, p);
  else
    hipLaunchKernelGGL((gather_kernel<kFp8, kAddr, 4>), dim3(groups), dim3(256), 0, stream, p);
}

template <bool kFp8>
void launch_dtype(const ProbeParams& p, unsigned groups, int cus, hipStream_t stream) {
  if (p.tpb % Cfg<kFp8>::kTok == 0)
    launch_gather<kFp8, kProbeUniform>(p, groups, cus, stream);
  else if (2 * p.tpb == Cfg<kFp8>::kTok)
    launch_gather<kFp8, kProbePair>(p, groups, cus, stream);
  else if (kFp8 && p.tpb == 8)
    launch_gather<kFp8, kFp8 ? kProbeQuad : kProbeGeneral>(p, groups, cus, stream);
  else
    launch_gather<kFp8, kProbeGeneral>(p, groups, cus, stream);
}

// VALU issue-rate probe: each wave runs `iters` rounds of 64 independent
// chains' worth of one instruction kind (8 register chains, 8 steps each), so
// issue, not latency, bounds it once a few waves share a SIMD.
template <int kKind>
__global__ __launch_bounds__(kValuThreads) void valu_kernel(int32_t* sink, int iters, float a) {
  float v[8];
  uint32_t u[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    v[q] = a + (float)threadIdx.x * 0.001f + (float)q;
    u[q] = threadIdx.x * 7u + (uint32_t)q;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (kKind == SDA_PROBE_VALU_FMA) v[q] = __builtin_fmaf(v[q], a, 0.5f);
        if (kKind == SDA_PROBE_VALU_XOR_ADD) u[q] = (u[q] ^ (uint32_t)it) + 0x9E3779B9u;
        if (kKind == SDA_PROBE_VALU_SHIFTS) u[q] = (u[q] >> 3) | (u[q] << 5);
      }
  }
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < 8; ++q) s += v[q] + (float)u[q];
  sink[(int64_t)blockIdx.x * kValuThreads + threadIdx.x] = __float_as_int(s);
}

}  // namespace
}  // namespace sda

extern "C" int sda_probe_valu(int32_t kind, int32_t workgroups, int32_t iters, int32_t* sink,
                              hipStream_t stream) {
  if (workgroups < 0 || iters < 0 || (workgroups > 0 && !sink)) return SDA_ERR_INVALID;
  if (workgroups == 0) return SDA_OK;
  const dim3 grid((unsigned)workgroups), block(sda::kValuThreads);
  switch (kind) {
    case SDA_PROBE_VALU_FMA:
      hipLaunchKernelGGL(sda::valu_kernel<SDA_PROBE_VALU_FMA>, grid, block, 0, stream, sink, iters,
                         0.999f);
      break;
    case SDA_PROBE_VALU_XOR_ADD:
      hipLaunchKernelGGL(sda::valu_kernel<SDA_PROBE_VALU_XOR_ADD>, grid, block, 0, stream, sink,
                         iters, 0.999f);
      break;
    case SDA_PROBE_VALU_SHIFTS:
      hipLaunchKernelGGL(sda::valu_kernel<SDA_PROBE_VALU_SHIFTS>, grid, block, 0, stream, sink,
                         iters, 0.999f);
      break;
    default:
      return SDA_ERR_INVALID;
  }
  return hipGetLastError() == hipSuccess ? SDA_OK : SDA_ERR_LAUNCH;
}

extern "C" size_t sda_probe_args_size(void) { return sizeof(sda_probe_args); }

extern "C" int sda_probe_gather(const sda_probe_args* a, hipStream_t stream) {
  if (!a || a->groups < 0 || a->block_tokens < 1) return SDA_ERR_INVALID;
  if (a->kv_dtype != SDA_KV_BF16 && a->kv_dtype != SDA_KV_FP8_E4M3) return SDA_ERR_INVALID;
  const bool fp8 = a->kv_dtype == SDA_KV_FP8_E4M3;
  const int64_t row_bytes = fp8 ? SDA_KV_ROW : 2 * SDA_KV_ROW;
  if (a->token_stride < row_bytes || a->token_stride % 16 ||
      (int64_t)a->block_tokens * a->token_stride > 0xFFFFFFFFll ||
      (int64_t)a->block_tokens * SDA_PROBE_MAX_BLOCKS > 0x7FFFFFFFll)
    return SDA_ERR_INVALID;
  if (a->groups == 0) return SDA_OK;
  if (!a->base || !a->block_offsets || !a->group_start || !a->sink) return SDA_ERR_INVALID;
  int device = -1, cus = 0;
  if ((stream ? hipStreamGetDevice(stream, &device) : hipGetDevice(&device)) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      cus <= 0)
    return SDA_ERR_LAUNCH;
  sda::ProbeParams p{};
  p.base = static_cast<const uint8_t*>(a->base);
  p.ts = a->token_stride;
  p.offsets = a->block_offsets;
  p.start = a->group_start;
  p.sink = a->sink;
  p.tpb = a->block_tokens;
  if (fp8)
    sda::launch_dtype<true>(p, (unsigned)a->groups, cus, stream);
  else
    sda::launch_dtype<false>(p, (unsigned)a->groups, cus, stream);
  return hipGetLastError() == hipSuccess ? SDA_OK : SDA_ERR_LAUNCH;
}
