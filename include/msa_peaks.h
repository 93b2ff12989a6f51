/*
 * msa_peaks.h -- measured machine peaks for libmsa's roofline reports.
 *
 * The MSA kernels are read against the published MI355X peaks (8 TB/s HBM,
 * 2.5 PFLOP/s dense bf16) and against what this device actually sustains with
 * nothing else in the way.  These probes measure the latter; they are
 * measurement aids, not steps of the MSA path, and follow the conventions of
 * msa.h (status codes, msa_last_error(), asynchronous on the caller's stream,
 * no allocation, device pointers unless stated).
 */
#ifndef MSA_PEAKS_H_
#define MSA_PEAKS_H_

#include "msa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` bytes at `buf` (device, 16-byte aligned, bytes a
 * multiple of 16), every byte once: one 256-thread workgroup per 64 KB chunk,
 * each thread keeping eight non-temporal 16-byte loads in flight.  `sink` (device, one float) is written only in a case no
 * real data reaches; it keeps the loads from being optimised away.  Time the
 * launch with events around it: bytes / time is the sustained HBM read rate
 * (use a buffer much larger than the 256 MB last-level cache).
 * Errors: MSA_ERR_INVALID (alignment, size), MSA_ERR_NULL, MSA_ERR_HIP. */
msa_status_t msa_peak_stream_read(const void *buf, size_t bytes, float *sink,
                                  msa_stream_t stream);

/* Streaming write of `bytes` bytes at `buf` (device, 16-byte aligned, bytes a
 * multiple of 16), every 16-byte unit i set to a value made of tag ^ i, one
 * 256-thread workgroup per 64 KB chunk, cached stores.  Time it with events for
 * the write rate; time msa_peak_stream_read of the same bytes right after it
 * (caches otherwise cold) for the rate at which freshly written data reads
 * back from the last-level cache (sizes below its 256 MB) or from HBM.
 * Errors: MSA_ERR_INVALID (alignment, size), MSA_ERR_NULL, MSA_ERR_HIP. */
msa_status_t msa_peak_stream_write(void *buf, size_t bytes, uint32_t tag, msa_stream_t stream);

/* Row gather-scatter: for i < n, destination row store_idx[i] receives source
 * row load_idx[i], rows of 256 bytes (device pointers; src and dst 16-byte
 * aligned).  This is the memory pattern of the KV-block-major prefill kernel
 * (msa_sparse_attn_prefill) without its arithmetic: with load_idx the query
 * rows of the (row, head) pairs in the order the kernel's units take them and
 * store_idx their partial rows, its time is what the kernel's query loads and
 * partial stores cost by themselves.  The rows go in tiles of 32; each
 * 256-thread workgroup takes tiles_per_wg (1..64) consecutive tiles, its four
 * waves one tile each in turn.  load_layout 0 loads four whole rows per
 * instruction (16 bytes per lane), 1 loads 32 rows x 32 bytes per instruction
 * (the layout of 32 matrix-core operand rows, as the kernel loads queries);
 * either way a wave passes its 32 rows through LDS and stores four whole rows
 * per instruction, non-temporally, and issues the next tile's loads before the
 * current tile's stores.  n is a multiple of 32.  Preconditions (device data,
 * not checked): every load_idx names a source row, every store_idx a
 * destination row; with distinct store_idx the destination rows are an exact
 * copy.  Errors: MSA_ERR_INVALID (n, tiles_per_wg, load_layout, alignment),
 * MSA_ERR_NULL, MSA_ERR_HIP. */
msa_status_t msa_peak_row_copy(const void *src, void *dst, const int32_t *load_idx,
                               const int32_t *store_idx, int64_t n, int32_t tiles_per_wg,
                               int32_t load_layout, msa_stream_t stream);

/* Register-resident bf16 matrix-core loop: two 256-thread workgroups per CU,
 * each wave runs `iters` iterations of four independent 32x32x16 bf16 MFMA
 * accumulation chains.  *flops (host) receives the floating-point operations the
 * launch performs (2 * 32 * 32 * 16 per MFMA); flops / time is the sustained
 * dense bf16 rate.  `sink` as above.
 * Errors: MSA_ERR_INVALID (iters < 1), MSA_ERR_NULL, MSA_ERR_HIP. */
msa_status_t msa_peak_mfma_bf16(int32_t iters, float *sink, double *flops, msa_stream_t stream);

/* The same loop on pseudo-random operands: each lane holds 8 A and 8 B
 * fragments of roughly normal bf16 values (unit variance, from an integer hash
 * of the lane and element), and each wave runs `iters` iterations of two
 * accumulation chains of 8 MFMAs cycling through them.  The matrix cores'
 * sustained rate depends on the operand data (the chip lowers its rate under
 * the power draw of random bits), so this is the rate a contraction of
 * N(0,1)-like values can reach, below the fixed-operand loop above.  *flops
 * and `sink` as above.
 * Errors: MSA_ERR_INVALID (iters < 1), MSA_ERR_NULL, MSA_ERR_HIP. */
msa_status_t msa_peak_mfma_bf16_random(int32_t iters, float *sink, double *flops,
                                       msa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_PEAKS_H_ */
