/*
 * ttt_probe.h - peak probes of the TTT attention library (MI355X / gfx950), for measurement.
 *
 * The roofline fractions of the attention kernels are quoted against MI355X's published
 * peaks (bf16 dense matrix cores 2.5 PFLOP/s, HBM3E 8 TB/s); these two kernels measure what
 * the same chip reaches on the plainest possible workload, so that a fraction can also be read
 * against an attainable peak.  Both enqueue on `stream` (a hipStream_t; NULL = default) and
 * return 0 on success or a negative TTT_E_* code (ttt_attn.h); the caller times them (e.g.
 * with hipEvents on the same stream).
 */
#ifndef TTT_PROBE_H
#define TTT_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * bf16 matrix-core probe: `workgroups` workgroups of 4 waves (two per CU resident); each wave
 * issues `iters` rounds of 8 v_mfma_f32_32x32x16_bf16 on 4 independent fp32 accumulators
 * (operands in registers, no memory traffic in the loop), then writes one float per lane to
 * sink[workgroups * 256] so the work is kept.  Flops = workgroups * 4 * iters * 8 * 32768.
 * Errors: TTT_E_NULL (sink), TTT_E_SHAPE (workgroups or iters < 1), TTT_E_ALIGN, TTT_E_HIP.
 */
int ttt_probe_mfma_bf16(float* sink, int32_t workgroups, int32_t iters, void* stream);

/*
 * HBM stream-copy probe: dst[0, bytes) = src[0, bytes) with 16-byte loads and stores, one
 * workgroup of 256 lanes per 16 KB chunk, four loads in flight per lane before its stores.
 * Bytes moved = 2 * bytes.
 * src and dst are device memory, 16-byte aligned, not overlapping; bytes a multiple of 16.
 * Errors: TTT_E_NULL, TTT_E_SHAPE (bytes 0, not a multiple of 16, or 2^31 chunks or more),
 * TTT_E_ALIGN, TTT_E_HIP.
 */
int ttt_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TTT_PROBE_H */
