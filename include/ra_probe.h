/*
 * ra_probe.h -- calibration kernel of the ring-attention library (gfx950).
 *
 * Not part of the attention path. The attention kernels are measured against
 * the MI355X's published dense bf16 MFMA peak and, beside it, against the rate
 * that the bf16 matrix instruction they use (v_mfma_f32_32x32x16_bf16, 32x32
 * output, 16-deep reduction) actually sustains on the chip when it does
 * nothing else. This entry point measures that second figure.
 */
#ifndef RA_PROBE_H
#define RA_PROBE_H

#include <stdint.h>

#include "ra.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Launches `workgroups` workgroups of `waves` waves (4: one wave per SIMD; 8: two)
 * that each run `iters` iterations of 4 independent v_mfma_f32_32x32x16_bf16 on
 * register operands (no memory traffic in the loop), then write one float per
 * lane to `sink` (device, fp32 [workgroups * waves * 64]) so the work is kept.
 * Executed FLOPs = workgroups * waves * iters * 4 * 32768. Time it with events on
 * `stream`. iters in [1, 2^24], workgroups in [1, 2^20]; waves 4 or 8, else
 * RA_ERR_SHAPE; sink NULL gives RA_ERR_NULL. */
ra_status ra_probe_mfma(int32_t iters, int32_t workgroups, int32_t waves, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RA_PROBE_H */
