/*
 * strata_probe.h -- measurement probes that set the achievable peaks the
 * MoE layer's kernels are compared against on this GPU.
 *
 * The layer's decode kernels stream packed expert weights from HBM and its
 * larger-batch kernels are bf16 matrix-core GEMMs.  Vendor peaks (8 TB/s of
 * HBM3E, 2.5 PFLOP/s dense bf16) are not what a kernel can reach, so two
 * probes measure what plain kernels do reach:
 *   - a stream read: every byte of a buffer loaded once with 16-byte loads
 *     (the buffer should be far larger than the 256 MB Infinity Cache);
 *   - bf16 matrix-core rate: independent v_mfma_f32_32x32x16_bf16 chains
 *     on register operands, no memory traffic.
 * Both enqueue on `stream` (hipStream_t as void*) and return at once; the
 * caller times them with events.  Pointers are device pointers.
 */
#ifndef STRATA_PROBE_H
#define STRATA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "strata_moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes of `buf` (16-byte aligned, bytes % 16 == 0) with
 * `blocks` blocks of 256 threads; each block writes one word of the loaded
 * data's XOR to sink[block] so the loads cannot be dropped.  EINVAL: a null
 * or misaligned pointer, bytes not a positive multiple of 16, or blocks
 * outside 1..65536; EHIP: the launch failed. */
strata_status strata_probe_hbm_read(const void *buf, size_t bytes, uint32_t *sink, int32_t blocks, void *stream);

/* `blocks` blocks of 256 threads, each wave running 4 independent chains of
 * `iters` bf16 32x32x16 matrix-core products; each block writes one float to
 * sink[block].  *flops (host) receives the floating-point operations of the
 * launch (2 * 32 * 32 * 16 per product).  EINVAL: a null pointer, iters
 * outside 1..2^20 or blocks outside 1..65536; EHIP: the launch failed. */
strata_status strata_probe_mfma_bf16(int32_t iters, float *sink, int32_t blocks, double *flops, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* STRATA_PROBE_H */
