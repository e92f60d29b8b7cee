/*
 * moe_peaks.h -- measurement helpers of libmoe.so: the two machine peaks the layer's kernels
 * are judged against, measured on the running GPU instead of taken from a data sheet.
 *
 * The roofline of a kernel is set by HBM bandwidth (weight streaming: "S23-J10" §3, read volume
 * R = b_W * N_e * U) or by the matrix cores (expert groups of hundreds of rows: intensity about
 * t_e FLOP per weight byte, same section).  A data-sheet peak assumes the top clock; under a
 * sustained load the chip holds a lower one, so both peaks are also measured here with a
 * plain streaming read and a register-only MFMA loop of the same instruction the layer's GEMMs
 * use.  Neither call computes anything of the layer.
 *
 * Conventions as in moe.h: device pointers, caller-owned, asynchronous on `stream`, no
 * allocation, errors returned as moe_status codes (MOE_ERR_INVALID_ARG for NULL or misaligned
 * pointers or sizes, MOE_ERR_HIP for a failed launch).
 */
#ifndef MOE_PEAKS_H_
#define MOE_PEAKS_H_

#include <stddef.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes of `buf` once with 16-byte vector loads: up to 8192 work-groups of 8
 * waves, each sweeping one contiguous chunk with four loads in flight per lane.  sink (2048
 * floats) is written only if a work-group's loaded words XOR to a fixed value; it keeps the
 * loads from being removed.  bytes must be a positive multiple of 64 KiB; buf and sink 16-byte
 * aligned.  Time it with events: bytes / duration is the achieved read rate.  A read of 1 GiB
 * also evicts the L2s and the 256 MiB MALL without leaving dirty lines behind. */
int moe_peak_hbm_read(const void *buf, size_t bytes, float *sink, moe_stream_t stream);

/* Runs `iters` rounds of 4 independent v_mfma_f32_32x32x16_bf16 per wave on register
 * operands, on `waves` waves (64 lanes each; a multiple of 4, at most 65536), and writes one
 * float per wave to sink[0..waves-1].  FLOPs executed: waves * iters * 4 * 32768. */
int moe_peak_mfma_bf16(int waves, int iters, float *sink, moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PEAKS_H_ */
