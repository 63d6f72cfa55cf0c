/* idxcache_calib.h -- measurement support for the benchmark (not an operation
 * of the indexer or of sparse attention).
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

#ifdef __cplusplus
}
#endif

#endif /* IDXCACHE_CALIB_H */
