/*
 * mla_peaks.h -- measured peaks of the MI355X pipes the MLA kernels are
 * priced against (HBM read bandwidth, dense MFMA rate).
 *
 * The pages quote the part's datasheet HBM bandwidth, 8 TB/s ("Inside Kimi K3
 * optimization", table of published per-GPU specifications in the benchmark
 * notes); a roofline fraction is reported against it and against what a
 * plain streaming read reaches on the same GPU.  These
 * entry points launch one such kernel each on `stream` (asynchronous; the
 * caller times them, e.g. with HIP events on that stream).  Status codes are
 * the mla_status values of mla.h; a failed launch returns MLA_ERR_HIP.
 */
#ifndef MLA_PEAKS_H
#define MLA_PEAKS_H

#include <stdint.h>

#include "mla.h"

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_PEAK_READ_VGPR 0   /* 16-byte vector loads into registers */
#define MLA_PEAK_READ_LDS 1    /* 16-byte buffer loads straight into LDS (the split kernels' copy path) */
#define MLA_PEAK_MFMA_FP8 0    /* v_mfma_scale_f32_32x32x64_f8f6f4, FP8 E4M3 operands */
#define MLA_PEAK_MFMA_BF16 1   /* v_mfma_f32_32x32x16_bf16 */

/* Reads `bytes` bytes at device address `buf` (16-byte aligned, a multiple
 * of 1 KiB, larger than the last-level cache to measure HBM) once, with
 * `workgroups` workgroups of 256 threads (1..1024) in grid-stride order, in
 * the given mode; writes a fold of the data to sink[0 .. workgroups - 1]
 * (device, uint32) so the loads are kept.
 * Errors: NULL_ARG, BAD_SHAPE (size, alignment, mode, workgroups), HIP. */
mla_status mla_peak_hbm_read(const void* buf, int64_t bytes, int32_t mode, uint32_t* sink,
                             int32_t workgroups, void* stream);

/* `workgroups` workgroups of four waves (one per SIMD when one workgroup runs
 * per CU), each wave issuing `iters` x 4 MFMAs of the given kind on four
 * independent accumulators (no dependency stalls): 32x32x64 FP8 MFMAs carry
 * 131,072 flops each, 32x32x16 bf16 MFMAs 32,768.  sink (device, float,
 * `workgroups` entries) is written only in a case that does not occur; it
 * keeps the work from being removed.
 * Errors: NULL_ARG, BAD_SHAPE (kind, iters outside 1..2^24, workgroups), HIP. */
mla_status mla_peak_mfma(int32_t kind, int32_t iters, float* sink, int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PEAKS_H */
