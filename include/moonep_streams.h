/*
 * moonep_streams.h -- plain 16-byte memory streams that measure, on the same GPU, the
 * ceilings the hot path's kernels are measured against.  Not part of the hot path: the
 * benchmark times them beside the path (libmoonep_streams.so).
 *
 * The pages quote no bandwidth or ceiling ("Moonshot AI Open-Sources MoonEP"
 * (tldrocket.com), paragraph 4 and "MoonshotAI/MoonEP 딥다이브" (fiv.co.kr), section 2
 * give only curves against DeepEP); these streams supply the GPU's own reference points:
 * a linear read, write and copy, and the row mixes of dispatch (one row read, K rows
 * written), combine (K rows read, one row written) and the combine backward (one row and
 * K rows read, the K rows written elsewhere) over contiguous or scattered rows.
 *
 * Conventions: device pointers 16-byte aligned, sizes multiples of 16 bytes, everything
 * enqueued on `stream` and asynchronous.  Return 0, -1 for an invalid argument (nothing
 * enqueued) or -4 when a launch failed.  Row indices outside [0, rows of the buffer) are
 * skipped, never dereferenced.  Streams write constant or copied bytes and keep no state.
 */
#ifndef MOONEP_STREAMS_H_
#define MOONEP_STREAMS_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Launch shapes: MOONEP_SHAPE_WAVE_2K = one 64-lane workgroup per 2 KB (the dispatch
 * kernel's chunk); MOONEP_SHAPE_BLOCK_4K = one 256-lane workgroup per 4 KB block.
 * Cache policy: 0 = plain loads/stores, 1 = non-temporal. */
#define MOONEP_SHAPE_WAVE_2K 0
#define MOONEP_SHAPE_BLOCK_4K 1

/* Reads nbytes from src; writes 16 bytes to sink only for a data pattern that never occurs
 * in practice (so the loads are not optimised away). */
int moonep_stream_read(const void* src, int64_t nbytes, int shape, int policy, void* sink,
                       hipStream_t stream);
/* Writes nbytes of a fixed pattern to dst. */
int moonep_stream_write(void* dst, int64_t nbytes, int shape, int policy, hipStream_t stream);
/* dst[0, nbytes) = src[0, nbytes). */
int moonep_stream_copy(const void* src, void* dst, int64_t nbytes, int shape, int policy,
                       hipStream_t stream);

/* Dispatch's mix: for i < n, k < K:  dst row rows[i*K + k] = src row i (read_src != 0), or a
 * fixed pattern (read_src == 0: writes only).  Rows of row_bytes; dst has dst_rows rows.
 * One 64-lane workgroup per (i, 2 KB chunk), non-temporal stores, at most 5 workgroups per
 * CU: the dispatch kernel's shape and residency. */
int moonep_rows_fanout(const int32_t* rows, int64_t n, int K, const void* src, void* dst,
                       int64_t dst_rows, int row_bytes, int read_src, hipStream_t stream);

/* Combine's mix: for i < n:  dst row i = XOR over k < K of src row rows[i*K + k]
 * (write_dst != 0), or nothing written (write_dst == 0: reads only).  src has src_rows
 * rows.  One 64-lane workgroup per (i, 1 KB chunk), non-temporal loads and stores, at most
 * 9 workgroups per CU when src exceeds 256 MB: the combine kernel's shape and residency. */
int moonep_rows_gather(const int32_t* rows, int64_t n, int K, const void* src, int64_t src_rows,
                       void* dst, int row_bytes, int write_dst, hipStream_t stream);

/* The combine backward's mix: for i < n, k < K:  b row r = a row r XOR src row i, where
 * r = rows[i*K + k] (rows outside [0, rows_ab) skipped); a and b have rows_ab rows.  One
 * workgroup per source row, its K rows taken in groups of up to 8 (every load of the
 * group, one wait, the non-temporal stores): the combine backward kernel's shape. */
int moonep_rows_update(const int32_t* rows, int64_t n, int K, const void* src, const void* a,
                       void* b, int64_t rows_ab, int row_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOONEP_STREAMS_H_ */
