/* idxcache_calib.h -- measurement support for the benchmark (not an operation
 * of the indexer or of sparse attention).
 *
 * Two calls, each timed by the caller (HIP events on `stream`):
 *  - idxc_calib_mfma_rate: the MFMA rate that given operand bytes allow;
 *  - idxc_calib_gather_rate: the HBM rate of reading exactly the rows that an
 *    index set names, with nothing else to do.
 *
 * On MI355X the engine clock, and with it the MFMA rate, depends on how much
 * the MFMA operands toggle: chains of dense MFMAs on zero operands run near
 * the published peak, on random operands well below it.  This call runs such
 * a chain on operand bytes taken from the caller's buffers (for example the
 * benchmark's own query and key tensors), so that a kernel's MFMA rate can be
 * set against the rate its operands allow.  The caller times the launch (HIP
 * events on `stream`).
 */
#ifndef IDXCACHE_CALIB_H
#define IDXCACHE_CALIB_H

#include <stddef.h>
#include <stdint.h>

#include "idxcache.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    IDXC_CALIB_FP8_32X32X64 = 0,  /* v_mfma_f32_32x32x64_f8f6f4, e4m3 operands: 131072 flop each */
    IDXC_CALIB_BF16_32X32X16 = 1  /* v_mfma_f32_32x32x16_bf16: 32768 flop each */
} idxc_calib_kind;

/* Enqueues one launch of `blocks` workgroups of 256 threads (four wavefronts);
 * each wavefront loads four A and four B operand registers from `a` and `b`
 * (thread t, register r: consecutive 16-byte chunks from chunk 8t + 2r for
 * fp8, 4t + r for bf16, wrapping around the buffer) and then issues
 * 16 * iters MFMAs of `kind` into four independent accumulators, rotating
 * over its operand registers.  Total work: blocks * 4 * 16 * iters MFMAs.
 *   a, b         device buffers of a_bytes, b_bytes bytes, 16-byte aligned,
 *                at least 16 bytes each; read only (borrowed).
 *   out          device buffer of blocks * 256 floats (one sum per thread,
 *                written so that the work is not removed); borrowed.
 *   stream       hipStream_t, or NULL for the null stream.
 * Returns IDXC_ERR_NULL, IDXC_ERR_SHAPE (bytes < 16, iters or blocks < 1),
 * IDXC_ERR_ALIGN, IDXC_ERR_DTYPE (unknown kind) before any HIP call, or
 * IDXC_ERR_HIP when the launch fails. */
int idxc_calib_mfma_rate(int kind, const void *a, size_t a_bytes, const void *b, size_t b_bytes, int iters, int blocks,
                         float *out, void *stream);

/* Enqueues one launch of `blocks` workgroups of 256 threads that read the
 * rows an index set names, the access pattern of the sparse attention gather
 * (itoverdose.com, "IndexCache: Wie DeepSeek O(NL²)-Kosten in Sparse Attention
 * um 75% reduziert", section "Wie der Indexer funktioniert und warum MLA
 * entscheidend ist": each selected token contributes one latent row), and
 * nothing else.  Entry j of query b names row b * rows_per_seq + t[b * k + j]
 * of `rows`; entries outside [0, rows_per_seq) are skipped.  A wavefront
 * reads 8 consecutive entries at a time, each lane one 16-byte piece of every
 * 128-byte line of its entry's row (row_bytes / 128 loads in flight per lane).
 *   rows         device buffer of nq * rows_per_seq rows of row_bytes bytes,
 *                16-byte aligned; read only (borrowed).
 *   row_bytes    a multiple of 128, at most 2048 (1152 for the latent rows).
 *   t            device int32 [nq, k], 4-byte aligned; read only (borrowed).
 *   out          device buffer of blocks * 256 uint32: each thread's XOR of
 *                the 32-bit words it read from rows it did not skip (written
 *                so that the loads are not removed); borrowed.
 *   stream       hipStream_t, or NULL for the null stream.
 * Returns IDXC_ERR_NULL, IDXC_ERR_SHAPE (row_bytes not a multiple of 128 in
 * [128, 2048], rows_per_seq, nq, k or blocks below 1, blocks above 2^20,
 * nq * k above 2^30),
 * IDXC_ERR_ALIGN before any HIP call, or IDXC_ERR_HIP when the launch
 * fails. */
int idxc_calib_gather_rate(const void *rows, size_t row_bytes, long long rows_per_seq, const int32_t *t, int nq, int k,
                           int blocks, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* IDXCACHE_CALIB_H */
