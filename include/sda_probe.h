/*
 * sda_probe.h - gather-ceiling and VALU issue-rate probes for MI355X
 * (gfx950).  C ABI of libsda_probe.so, a measurement library beside libsda.so
 * (bench.py --gather-ceiling and --valu-rate use it; the decode path never
 * does).
 *
 * The probe moves a list of token blocks from HBM into LDS through the split
 * kernel's own chunk loop (the same 12 LDS-DMAs per chunk of 16 bf16 or 32
 * FP8 token rows, the same lane geometry, non-temporal policy, two-stage
 * per-wave pipeline and launch shape) and does nothing with the data beyond
 * one LDS read per chunk.  Its time for a decode call's blocks is the memory
 * system's rate for that access pattern: the ceiling against which the split
 * kernel's streaming is judged.
 *
 * All pointers are device pointers.  The call allocates nothing.
 *
 *  base          buffer holding the blocks (e.g. the KV cache).
 *  kv_dtype      SDA_KV_BF16 (768-byte token rows) or SDA_KV_FP8_E4M3
 *                (384-byte rows), as in sda.h.
 *  token_stride  bytes between consecutive token rows of a block; a
 *                multiple of 16, at least the row size; block_tokens rows
 *                at this stride must span less than 4 GiB.
 *  groups        workgroups, one per decode row (>= 0; 0 returns OK).
 *  block_tokens  token rows per block (the region size), >= 1.
 *  block_offsets int64 [total blocks]: byte offset in `base` of each block's
 *                first token row, 16-byte aligned.
 *  group_start   int32 [groups + 1], non-decreasing: workgroup g streams
 *                blocks group_start[g] .. group_start[g + 1] - 1, at most
 *                SDA_PROBE_MAX_BLOCKS of them, in that order.
 *  sink          int32 [groups * 4]: each wave writes one word (what it read
 *                back from LDS), so the transfers have an observable use.
 *
 * Returns an sda_status (sda.h): SDA_ERR_INVALID for a bad argument,
 * SDA_ERR_LAUNCH if the launch or the device query fails.  Group sizes and
 * offsets are device data and are trusted.
 */
#ifndef SDA_PROBE_H_
#define SDA_PROBE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDA_PROBE_MAX_BLOCKS 2048

typedef struct sda_probe_args {
  const void *base;
  int32_t kv_dtype;
  int64_t token_stride;
  int32_t groups, block_tokens;
  const int64_t *block_offsets;
  const int32_t *group_start;
  int32_t *sink;
} sda_probe_args;

int sda_probe_gather(const sda_probe_args *args, hipStream_t stream);

/*
 * VALU issue-rate probe: `workgroups` workgroups of 256 threads, each wave
 * running `iters` rounds of 8 steps over 8 independent register chains of
 * one instruction kind.  Per wave that is 64 * iters instructions
 * (SDA_PROBE_VALU_FMA: v_fma_f32) or 128 * iters (the two-instruction kinds:
 * v_xor_b32 + v_add_u32 with scalar and literal operands, v_lshrrev_b32 +
 * v_lshl_or_b32).  Timed over a full chip of resident waves, it gives the
 * SIMD cycles one wave64 instruction of that kind holds, which counter-based
 * VALU estimates need.  sink: int32 [workgroups * 256], one word per thread.
 * Returns SDA_ERR_INVALID for a bad argument or kind, SDA_ERR_LAUNCH if the
 * launch fails.
 */
#define SDA_PROBE_VALU_FMA 0
#define SDA_PROBE_VALU_XOR_ADD 1
#define SDA_PROBE_VALU_SHIFTS 2

int sda_probe_valu(int32_t kind, int32_t workgroups, int32_t iters, int32_t *sink,
                   hipStream_t stream);

/* sizeof(sda_probe_args), for bindings that mirror the struct. */
size_t sda_probe_args_size(void);

#ifdef __cplusplus
}
#endif

#endif /* SDA_PROBE_H_ */
