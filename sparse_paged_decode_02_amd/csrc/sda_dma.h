// The split kernel's chunk loads, shared with the gather-ceiling probe
// (sda_probe.hip): one chunk of token slots (16 bf16 or 32 FP8 token rows of
// the [.., 384] cache: 6 KiB of K and 6 KiB of V) moves from HBM to a
// wave-private LDS stage with 12 global_load_lds_dwordx4 instructions issued
// from inline assembly, marked non-temporal, and awaited with an explicit
// vmcnt.  This header holds the lane geometry (which 16-byte piece of which
// token row each lane moves, and where it lands under the LDS swizzles), the
// DMA sequences for the addressing modes, and the waits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define SDA_LDS __attribute__((address_space(3)))

namespace sda {
namespace {

constexpr int kDim = 192;
constexpr int kOpsPerChunk = 12;    // vector-memory instructions per chunk issue
constexpr int kStageBytes = 6144;   // K (or V) bytes of one chunk (16 bf16 / 32 FP8 tokens)
constexpr int kChunkBytes = 2 * kStageBytes;  // one stage: K then V

// Per cache dtype: tokens per chunk, V bytes per token, 16-byte V pieces per token.
template <bool kFp8>
struct Cfg {
  static constexpr int kTok = kFp8 ? 32 : 16;
  static constexpr int kEsz = kFp8 ? 1 : 2;
  static constexpr int kVBytes = kDim * kEsz;
  static constexpr int kPieces = kVBytes / 16;
  static_assert(kTok * kVBytes == kStageBytes, "one chunk of V fills one stage");
};

// LDS swizzles.  A stage holds one chunk's V rows, one per token, as 16-byte
// pieces.  Piece p of token row r is stored at piece position p ^ swz(r).
// The XOR keeps a piece inside its aligned 8-piece (bf16) or 4-piece (FP8)
// block.  The swizzle makes the transposing reads of one 16-lane group hit 32
// distinct banks:
//  bf16: lanes 4y+q of group g read row 4g+y, pieces 2nt+(q>>1);
//  FP8:  lanes 2y+h of group g read row 16(y>>2)+4g+(y&3), piece nt.
template <bool kFp8>
__device__ __forceinline__ int swz(int row) {
  return kFp8 ? 2 * ((row >> 4) & 1) + ((row >> 1) & 1) : 2 * (row & 3) + ((row >> 2) & 1);
}
// K pieces: the A-operand reads of 8 consecutive lanes (rows i..i+7 of one
// tile, one piece) hit 32 distinct banks.
template <bool kFp8>
__device__ __forceinline__ int swz_k(int row) {
  return kFp8 ? (row >> 1) & 3 : row & 7;
}

// One chunk's 12 LDS-DMAs (global_load_lds_dwordx4: each lane moves 16 bytes
// to LDS address M0 + 16 * lane).  K pieces land at stage + 1024*j, V pieces
// at stage + 6144 + 1024*j, j = 0..5.  Issued from inline assembly so that
// the compiler does not tie later LDS reads to them; completion is awaited
// with wait_vmcnt.  M0 is saved and restored around the block.
//
// Cache policy: K|V bytes are read exactly once, so every DMA is
// non-temporal (`nt`); bf16 gated measured 72.4 -> 64.3 us with nt on
// MI355X.  A 384-byte FP8 token row puts K[128:192] and V[0:64] in one
// 128-byte line.  FP8 chunks therefore issue K DMA j and V DMA j, which cover
// the same token rows, back to back (SDA_CHUNK_ASM_KV), so the second request
// for the shared line meets the first in flight: all-nt FP8 then fetches
// 1.000x the K|V bytes, where K-then-V order with nt fetched 1.024x.  (K had
// kept the default policy to avoid that re-fetch, but its cacheable loads
// evict dirty lines of earlier kernels, and the write-backs land inside the
// call: 81 us on the FP8 cache workload after a 1 GiB write.)
#define SDA_LDDMA(op, addr, suf) "global_load_lds_dwordx4 %[" op "], " addr suf "\n\t"
#define SDA_NEXT "s_add_u32 m0, m0, 0x400\n\t"
#define SDA_CHUNK_ASM(addr, ksuf, vsuf)                                                      \
  "s_mov_b32 %[sv], m0\n\t"                                                                  \
  "s_mov_b32 m0, %[st]\n\t" SDA_LDDMA("k0", addr, ksuf) SDA_NEXT SDA_LDDMA("k1", addr, ksuf) \
      SDA_NEXT SDA_LDDMA("k2", addr, ksuf) SDA_NEXT SDA_LDDMA("k3", addr, ksuf) SDA_NEXT     \
      SDA_LDDMA("k4", addr, ksuf) SDA_NEXT SDA_LDDMA("k5", addr, ksuf) SDA_NEXT              \
      SDA_LDDMA("v0", addr, vsuf) SDA_NEXT SDA_LDDMA("v1", addr, vsuf) SDA_NEXT              \
      SDA_LDDMA("v2", addr, vsuf) SDA_NEXT SDA_LDDMA("v3", addr, vsuf) SDA_NEXT              \
      SDA_LDDMA("v4", addr, vsuf) SDA_NEXT SDA_LDDMA("v5", addr, vsuf)                       \
  "s_mov_b32 m0, %[sv]"

// FP8 chunk: K DMA j then V DMA j for j = 0..5 (the same token rows), with
// M0 set from the stage base for each: K slice j at stage + 1 KiB j, V slice
// j at stage + 6 KiB + 1 KiB j, the layout SDA_CHUNK_ASM writes in order.
#define SDA_M0(off) "s_add_u32 m0, %[st], " off "\n\t"
#define SDA_CHUNK_ASM_KV(addr, suf)                                                          \
  "s_mov_b32 %[sv], m0\n\t"                                                                  \
  "s_mov_b32 m0, %[st]\n\t" SDA_LDDMA("k0", addr, suf) SDA_M0("0x1800")                      \
      SDA_LDDMA("v0", addr, suf) SDA_M0("0x400") SDA_LDDMA("k1", addr, suf) SDA_M0("0x1c00")    \
      SDA_LDDMA("v1", addr, suf) SDA_M0("0x800") SDA_LDDMA("k2", addr, suf) SDA_M0("0x2000")    \
      SDA_LDDMA("v2", addr, suf) SDA_M0("0xc00") SDA_LDDMA("k3", addr, suf) SDA_M0("0x2400")    \
      SDA_LDDMA("v3", addr, suf) SDA_M0("0x1000") SDA_LDDMA("k4", addr, suf) SDA_M0("0x2800")   \
      SDA_LDDMA("v4", addr, suf) SDA_M0("0x1400") SDA_LDDMA("k5", addr, suf) SDA_M0("0x2c00")   \
      SDA_LDDMA("v5", addr, suf) "s_mov_b32 m0, %[sv]"
static_assert(kStageBytes == 0x1800, "SDA_CHUNK_ASM_KV: V slices start 6 KiB into the stage");

// Two-region chunk (bf16, 8-token regions): the first three K and V DMAs
// cover token rows 0..7 (pieces 0..191 of a 384-piece half) and the last
// three rows 8..15, so each half takes its own uniform base.
#define SDA_CHUNK_ASM2(addra, addrb, suf)                                                      \
  "s_mov_b32 %[sv], m0\n\t"                                                                    \
  "s_mov_b32 m0, %[st]\n\t" SDA_LDDMA("k0", addra, suf) SDA_NEXT SDA_LDDMA("k1", addra, suf)   \
      SDA_NEXT SDA_LDDMA("k2", addra, suf) SDA_NEXT SDA_LDDMA("k3", addrb, suf) SDA_NEXT       \
      SDA_LDDMA("k4", addrb, suf) SDA_NEXT SDA_LDDMA("k5", addrb, suf) SDA_NEXT                \
      SDA_LDDMA("v0", addra, suf) SDA_NEXT SDA_LDDMA("v1", addra, suf) SDA_NEXT                \
      SDA_LDDMA("v2", addra, suf) SDA_NEXT SDA_LDDMA("v3", addrb, suf) SDA_NEXT                \
      SDA_LDDMA("v4", addrb, suf) SDA_NEXT SDA_LDDMA("v5", addrb, suf)                         \
  "s_mov_b32 m0, %[sv]"

// Two-region FP8 chunk (16-token regions): K and V DMAs 0..2 cover token
// rows 0..15 and DMAs 3..5 rows 16..31, each half from its own uniform base,
// in SDA_CHUNK_ASM_KV's K/V order and LDS placement.
#define SDA_CHUNK_ASM_KV2(addra, addrb, suf)                                                   \
  "s_mov_b32 %[sv], m0\n\t"                                                                   \
  "s_mov_b32 m0, %[st]\n\t" SDA_LDDMA("k0", addra, suf) SDA_M0("0x1800")                      \
      SDA_LDDMA("v0", addra, suf) SDA_M0("0x400") SDA_LDDMA("k1", addra, suf) SDA_M0("0x1c00")  \
      SDA_LDDMA("v1", addra, suf) SDA_M0("0x800") SDA_LDDMA("k2", addra, suf) SDA_M0("0x2000")  \
      SDA_LDDMA("v2", addra, suf) SDA_M0("0xc00") SDA_LDDMA("k3", addrb, suf) SDA_M0("0x2400")  \
      SDA_LDDMA("v3", addrb, suf) SDA_M0("0x1000") SDA_LDDMA("k4", addrb, suf) SDA_M0("0x2800") \
      SDA_LDDMA("v4", addrb, suf) SDA_M0("0x1400") SDA_LDDMA("k5", addrb, suf) SDA_M0("0x2c00") \
      SDA_LDDMA("v5", addrb, suf) "s_mov_b32 m0, %[sv]"

// Two uniform bases: DMAs 0..2 from base_a, 3..5 from base_b (K and V).
template <bool kFp8>
__device__ __forceinline__ void dma_chunk_sbase2(const uint8_t* base_a, const uint8_t* base_b,
                                                 uint32_t stage, const uint32_t (&ko)[6],
                                                 const uint32_t (&vo)[6]) {
  uint32_t saved;
#define SDA_SBASE2_OPERANDS                                                                     \
  : [sv] "=&s"(saved)                                                                           \
  : [st] "s"(stage), [b] "s"(base_a), [b2] "s"(base_b), [k0] "v"(ko[0]), [k1] "v"(ko[1]),      \
    [k2] "v"(ko[2]), [k3] "v"(ko[3]), [k4] "v"(ko[4]), [k5] "v"(ko[5]), [v0] "v"(vo[0]),        \
    [v1] "v"(vo[1]), [v2] "v"(vo[2]), [v3] "v"(vo[3]), [v4] "v"(vo[4]), [v5] "v"(vo[5])         \
  : "memory"
  if constexpr (kFp8)
    __asm__ __volatile__(SDA_CHUNK_ASM_KV2("%[b]", "%[b2]", " nt") SDA_SBASE2_OPERANDS);
  else
    __asm__ __volatile__(SDA_CHUNK_ASM2("%[b]", "%[b2]", " nt") SDA_SBASE2_OPERANDS);
#undef SDA_SBASE2_OPERANDS
}

// Four-region chunk (FP8, 8-token regions).  K DMA j covers token rows
// (64j + lane) / 12: DMAs 0, 2, 3 and 5 lie inside regions 0, 1, 2 and 3 and
// take that region's uniform base; DMAs 1 and 4 cover rows 5..10 and 21..26,
// whose lanes 0..31 read region 0 / 2 and lanes 32..63 region 1 / 3, so they
// take per-lane 64-bit addresses.  V DMA j covers the same rows.  The K/V
// order and LDS placement are SDA_CHUNK_ASM_KV's.
#define SDA_CHUNK_ASM_QUAD(suf)                                                               \
  "s_mov_b32 %[sv], m0\n\t"                                                                   \
  "s_mov_b32 m0, %[st]\n\t" SDA_LDDMA("k0", "%[b0]", suf) SDA_M0("0x1800")                    \
      SDA_LDDMA("v0", "%[b0]", suf) SDA_M0("0x400") SDA_LDDMA("k1", "off", suf)                \
          SDA_M0("0x1c00") SDA_LDDMA("v1", "off", suf) SDA_M0("0x800")                         \
              SDA_LDDMA("k2", "%[b1]", suf) SDA_M0("0x2000") SDA_LDDMA("v2", "%[b1]", suf)     \
                  SDA_M0("0xc00") SDA_LDDMA("k3", "%[b2]", suf) SDA_M0("0x2400")               \
                      SDA_LDDMA("v3", "%[b2]", suf) SDA_M0("0x1000")                           \
                          SDA_LDDMA("k4", "off", suf) SDA_M0("0x2800")                         \
                              SDA_LDDMA("v4", "off", suf) SDA_M0("0x1400")                     \
                                  SDA_LDDMA("k5", "%[b3]", suf) SDA_M0("0x2c00")               \
                                      SDA_LDDMA("v5", "%[b3]", suf) "s_mov_b32 m0, %[sv]"

// Token row of K DMA j, lane l, in an FP8 chunk (12 pieces per row).
constexpr int fp8_dma_row(int j, int l) { return (64 * j + l) / Cfg<true>::kPieces; }
// The region (of four 8-row regions) that every lane of DMA j reads, or -1
// when the DMA's lanes span two regions.
constexpr int quad_region(int j) {
  int q = fp8_dma_row(j, 0) / 8;
  for (int l = 1; l < 64; ++l)
    if (fp8_dma_row(j, l) / 8 != q) return -1;
  return q;
}
// DMA j spans regions q and q + 1, split exactly at lane 32.
constexpr bool quad_split_at_32(int j) {
  for (int l = 0; l < 64; ++l)
    if (fp8_dma_row(j, l) / 8 != fp8_dma_row(j, 0) / 8 + (l >= 32 ? 1 : 0)) return false;
  return true;
}
static_assert(quad_region(0) == (0 + 1) / 2 && quad_region(2) == (2 + 1) / 2 &&
                  quad_region(3) == (3 + 1) / 2 && quad_region(5) == (5 + 1) / 2,
              "SDA_CHUNK_ASM_QUAD: DMAs 0, 2, 3, 5 each inside one region");
static_assert(quad_split_at_32(1) && fp8_dma_row(1, 0) / 8 == 0 && quad_split_at_32(4) &&
                  fp8_dma_row(4, 0) / 8 == 2,
              "SDA_CHUNK_ASM_QUAD: DMAs 1 and 4 split at lane 32");

// SDA_CHUNK_ASM_KV2: DMAs 0..2 inside rows 0..15, DMAs 3..5 inside rows 16..31.
static_assert(fp8_dma_row(0, 0) == 0 && fp8_dma_row(2, 63) == 15 && fp8_dma_row(3, 0) == 16 &&
                  fp8_dma_row(5, 63) == 31,
              "SDA_CHUNK_ASM_KV2: DMAs 0..2 and 3..5 each inside one 16-row half");

// ko/vo: 32-bit lane offsets of DMAs 0, 2, 3, 5 from their region's base;
// k1/v1, k4/v4: the lane's 64-bit addresses for DMAs 1 and 4.
__device__ __forceinline__ void dma_chunk_quad(const uint8_t* b0, const uint8_t* b1,
                                               const uint8_t* b2, const uint8_t* b3,
                                               uint32_t stage, const uint32_t (&ko)[6],
                                               const uint32_t (&vo)[6], const uint8_t* k1,
                                               const uint8_t* v1, const uint8_t* k4,
                                               const uint8_t* v4) {
  uint32_t saved;
  __asm__ __volatile__(SDA_CHUNK_ASM_QUAD(" nt")
                       : [sv] "=&s"(saved)
                       : [st] "s"(stage), [b0] "s"(b0), [b1] "s"(b1), [b2] "s"(b2),
                         [b3] "s"(b3), [k0] "v"(ko[0]), [k1] "v"(k1), [k2] "v"(ko[2]),
                         [k3] "v"(ko[3]), [k4] "v"(k4), [k5] "v"(ko[5]), [v0] "v"(vo[0]),
                         [v1] "v"(v1), [v2] "v"(vo[2]), [v3] "v"(vo[3]), [v4] "v"(v4),
                         [v5] "v"(vo[5])
                       : "memory");
}

// dma_chunk_sbase: one uniform 64-bit base (SGPRs) plus 32-bit per-lane
// byte offsets (chunks inside one region or one page).
template <bool kFp8>
__device__ __forceinline__ void dma_chunk_sbase(const uint8_t* base, uint32_t stage,
                                                const uint32_t (&ko)[6],
                                                const uint32_t (&vo)[6]) {
  uint32_t saved;
#define SDA_SBASE_OPERANDS                                                                      \
  : [sv] "=&s"(saved)                                                                           \
  : [st] "s"(stage), [b] "s"(base), [k0] "v"(ko[0]), [k1] "v"(ko[1]), [k2] "v"(ko[2]),          \
    [k3] "v"(ko[3]), [k4] "v"(ko[4]), [k5] "v"(ko[5]), [v0] "v"(vo[0]), [v1] "v"(vo[1]),        \
    [v2] "v"(vo[2]), [v3] "v"(vo[3]), [v4] "v"(vo[4]), [v5] "v"(vo[5])                          \
  : "memory"
  if constexpr (kFp8)
    __asm__ __volatile__(SDA_CHUNK_ASM_KV("%[b]", " nt") SDA_SBASE_OPERANDS);
  else
    __asm__ __volatile__(SDA_CHUNK_ASM("%[b]", " nt", " nt") SDA_SBASE_OPERANDS);
#undef SDA_SBASE_OPERANDS
}

// dma_chunk_vaddr: per-lane 64-bit addresses (chunks spanning regions).
template <bool kFp8>
__device__ __forceinline__ void dma_chunk_vaddr(uint32_t stage, const uint8_t* const (&ka)[6],
                                                const uint8_t* const (&va)[6]) {
  uint32_t saved;
#define SDA_VADDR_OPERANDS                                                                     \
  : [sv] "=&s"(saved)                                                                          \
  : [st] "s"(stage), [k0] "v"(ka[0]), [k1] "v"(ka[1]), [k2] "v"(ka[2]), [k3] "v"(ka[3]),       \
    [k4] "v"(ka[4]), [k5] "v"(ka[5]), [v0] "v"(va[0]), [v1] "v"(va[1]), [v2] "v"(va[2]),       \
    [v3] "v"(va[3]), [v4] "v"(va[4]), [v5] "v"(va[5])                                          \
  : "memory"
  if constexpr (kFp8)
    __asm__ __volatile__(SDA_CHUNK_ASM_KV("off", " nt") SDA_VADDR_OPERANDS);
  else
    __asm__ __volatile__(SDA_CHUNK_ASM("off", " nt", " nt") SDA_VADDR_OPERANDS);
#undef SDA_VADDR_OPERANDS
}

// One global_load_lds_dword: each lane moves the 4 bytes at its address to
// LDS address lds + 4 * lane.  No register receives the data, so nothing
// depends on the load until an explicit wait.  M0 is saved and restored.
__device__ __forceinline__ void dma_dword(uint32_t lds, const int32_t* addr) {
  uint32_t saved;
  __asm__ __volatile__(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[st]\n\t"
      "global_load_lds_dword %[a], off\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [st] "s"(lds), [a] "v"(addr)
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __asm__ __volatile__("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const SDA_LDS void*)p;
}

// Loop-invariant DMA geometry of one lane.  Stage slot 64j + lane (j = 0..5)
// is token row r = slot / kPieces, piece position slot % kPieces, which holds
// global piece (position ^ swizzle(r)).  koff/voff are that piece's byte
// offsets within the token's cache row (V after the 192 K elements).
struct LaneDma {
  int row[6];
  uint32_t koff[6], voff[6];
};

template <bool kFp8>
__device__ __forceinline__ LaneDma lane_dma(int lane) {
  using C = Cfg<kFp8>;
  LaneDma d;
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    const int slot = 64 * j + lane;
    const int r = slot / C::kPieces;
    const int pos = slot - r * C::kPieces;
    d.row[j] = r;
    d.koff[j] = 16u * (uint32_t)(pos ^ swz_k<kFp8>(r));
    d.voff[j] = (uint32_t)C::kVBytes + 16u * (uint32_t)(pos ^ swz<kFp8>(r));
  }
  return d;
}

// Wave-uniform 64-bit address from a per-lane value that is uniform in fact.
// readfirstlane returns int: go through uint32_t so the low half is
// zero-extended, never sign-extended into the high half.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* ptr) {
  const uint64_t b64 = (uint64_t)(uintptr_t)ptr;
  const uint32_t b_lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b64);
  const uint32_t b_hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32));
  return (const uint8_t*)(uintptr_t)(((uint64_t)b_hi << 32) | (uint64_t)b_lo);
}

}  // namespace
}  // namespace sda
