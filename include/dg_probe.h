/*
 * dg_probe.h - C ABI of libdg_probe: measurement kernels that give the achievable
 * ceilings of an MI355X (gfx950), against which the step's kernels are judged. They
 * are not part of the denoising step: they stream bytes or issue matrix instructions
 * and nothing else.
 *
 *   dg_probe_read   a read-only stream over `bytes` of device memory (16-byte loads,
 *                   several in flight per thread), the HBM read ceiling of a pass like
 *                   the sampler's logits read or the self-conditioning embedding read;
 *   dg_probe_copy   a copy of `bytes` (read once, written once);
 *   dg_probe_mfma_bf16  back-to-back v_mfma_f32_32x32x16_bf16 on register operands,
 *                   8 independent accumulators per wave, the dense bf16 matrix ceiling;
 *                   with operands that change from instruction to instruction (as in a
 *                   GEMM) or one fixed pair.
 *
 * Conventions: device pointers, 16-byte aligned; `bytes` a multiple of 16; every call
 * is asynchronous on `stream` (a hipStream_t, NULL for the default stream). Each returns
 * 0, or -1 for an invalid argument (nothing launched), or the hipError_t of a refused
 * launch. The callers time them with events on the same stream.
 */
#ifndef DG_PROBE_H
#define DG_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads src[0, bytes); each of the `blocks` work groups (256 threads) writes one word of
 * the XOR of what it read to sink[block] (device [blocks] uint32), so no load is dead.
 * blocks in [1, 65536]. */
int dg_probe_read(const void* src, size_t bytes, uint32_t* sink, int blocks, void* stream);

/* dst[0, bytes) = src[0, bytes); the ranges must not overlap. blocks in [1, 65536]. */
int dg_probe_copy(void* dst, const void* src, size_t bytes, int blocks, void* stream);

/* `blocks` work groups of 4 waves (one per SIMD of a compute unit when blocks is a
 * multiple of the CU count); each wave issues iters x 8 MFMAs of 32x32x16 (bf16 inputs,
 * fp32 accumulation): 2 * 32 * 32 * 16 * 8 * iters flops per wave. ops: device
 * [blocks * 256][8] 16-byte vectors (per lane 4 A and 4 B operands, bf16; each MFMA of a
 * group of 4 iterations takes another pair), or NULL for one fixed pair. Lane sums of
 * the accumulators go to sink (device [blocks * 256] float). blocks in [1, 65536],
 * iters a multiple of 4 in [4, 2^24]. */
int dg_probe_mfma_bf16(const void* ops, float* sink, int blocks, int iters, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DG_PROBE_H */
