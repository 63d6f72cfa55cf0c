// paged.hip -- serving metadata for varlen batches over paged caches.
//
// The method ships as patches for serving engines that batch many requests
// (parapluman.nl, sections "Real-world versnellingen op productiemodellen":
// decode throughput of a saturated server, and "IndexCache in productie
// brengen": vLLM and SGLang), engines whose caches are pools of fixed-size
// pages (setupai.cc, "IndexCache 加速長上下文推理 1.82 倍", comparison table:
// paged memory allocation).  A serving batch packs the query rows of several
// sequences (decode tokens, or the last chunk of a prefill) one after
// another, and each sequence's cache rows are found through its block table.
// The scoring, top-k and attention kernels are the ones of the contiguous
// path; these two kernels supply the one extra level of indirection: each
// row's (sequence, position), and pool row numbers for the index sets that
// the attention gathers.
#include "device_common.h"
#include "kernels.h"

namespace idxc {
namespace {

// Row r belongs to the sequence b with query_start[b] <= r < query_start[b+1]
// (binary search); its position is seq_len - q_len + (r - query_start[b]),
// i.e. the rows of a sequence are its last q_len positions.  Out-of-contract
// metadata is clamped so that every row maps to some sequence and to a
// position inside that sequence's pages.
__global__ void row_info_kernel(const int32_t *qs, const int32_t *seq_lens, int B, int rows, int max_pos,
                                int32_t *row_info, int32_t *row_pos) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    int lo = 0, hi = B - 1;   // last b with qs[b] <= r
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (qs[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    const int b = lo;
    const int qlen = qs[b + 1] - qs[b];
    int pos = seq_lens[b] - qlen + (r - qs[b]);
    pos = min(max(pos, 0), max_pos);
    row_info[2 * r] = b;
    row_info[2 * r + 1] = pos;
    if (row_pos) row_pos[r] = pos;
}

__global__ void translate_kernel(const int32_t *t, const int32_t *row_info, const int32_t *seq_lens,
                                 const int32_t *block_table, int rows, int topk, int bs_log2, int max_blocks,
                                 int num_blocks, int32_t *out) {
    const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (size_t)rows * topk) return;
    const int r = (int)(e / topk);
    const int b = row_info[2 * r];
    const int len = (int)min((long long)seq_lens[b], (long long)max_blocks << bs_log2);
    const int ix = t[e];
    int v = -1;
    if (ix >= 0 && ix < len) {
        const int pg = min(max(block_table[(size_t)b * max_blocks + (ix >> bs_log2)], 0), num_blocks - 1);
        v = (pg << bs_log2) | (ix & ((1 << bs_log2) - 1));
    }
    out[e] = v;
}

// Prefix of row blocks over sequences (one workgroup of 1024 threads, the
// sequences in chunks of 1024: a wavefront scan, then the wavefront totals).
__global__ __launch_bounds__(1024) void row_blocks_kernel(const int32_t *qs, int B, int total_q, int rows,
                                                          int lk_cap, int32_t *rb_start) {
    __shared__ int wsum[16];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    int carry = 0;
    for (int c0 = 0; c0 < B; c0 += 1024) {
        const int b = c0 + tid;
        int n = 0;
        if (b < B) {
            // the clamps of the paged prefill kernel
            const int q0 = min(max(qs[b], 0), total_q);
            const int q1 = min(max(qs[b + 1], q0), total_q);
            n = (min(q1 - q0, lk_cap) + rows - 1) / rows;
        }
        int incl = n;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int t = __shfl_up(incl, d, kWave);
            if (lane >= d) incl += t;
        }
        if (lane == kWave - 1) wsum[wave] = incl;
        __syncthreads();
        int before = 0, total = 0;
        for (int w = 0; w < 16; ++w) {
            if (w < wave) before += wsum[w];
            total += wsum[w];
        }
        if (b < B) rb_start[b] = carry + before + incl - n;
        carry += total;
        __syncthreads();   // wsum is rewritten by the next chunk
    }
    if (tid == 0) rb_start[B] = carry;
}

}  // namespace

hipError_t launch_row_blocks(const int32_t *query_start, int B, int total_q, int rows, int lk_cap,
                             int32_t *rb_start, hipStream_t s) {
    hipLaunchKernelGGL(row_blocks_kernel, dim3(1), dim3(1024), 0, s, query_start, B, total_q, rows, lk_cap,
                       rb_start);
    return hipGetLastError();
}

hipError_t launch_row_info(const int32_t *query_start, const int32_t *seq_lens, int B, int rows, int max_pos,
                           int32_t *row_info, int32_t *row_pos, hipStream_t s) {
    hipLaunchKernelGGL(row_info_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, query_start, seq_lens, B,
                       rows, max_pos, row_info, row_pos);
    return hipGetLastError();
}

hipError_t launch_translate_index(const int32_t *t, const int32_t *row_info, const int32_t *seq_lens,
                                  const int32_t *block_table, int rows, int topk, int bs_log2, int max_blocks,
                                  int num_blocks, int32_t *out, hipStream_t s) {
    const size_t n = (size_t)rows * topk;
    hipLaunchKernelGGL(translate_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, t, row_info, seq_lens,
                       block_table, rows, topk, bs_log2, max_blocks, num_blocks, out);
    return hipGetLastError();
}

}  // namespace idxc
