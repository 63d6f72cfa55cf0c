// calib.hip -- measurement support: dense MFMA chains on caller-given operand
// bytes (the MFMA rate the benchmark's own operands allow on this part), and
// a plain gather of the rows an index set names (the HBM rate that pattern of
// rows allows, with no computation behind the loads).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "idxcache_calib.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;

template <int KIND>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 2))) void mfma_rate_kernel(
    const v4i *a, size_t na, const v4i *b, size_t nb, int iters, float *out) {
    const size_t t = (size_t)blockIdx.x * kThreads + threadIdx.x;
    v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
    if constexpr (KIND == IDXC_CALIB_FP8_32X32X64) {
        v8i A[4], B[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const v4i a0 = a[(8 * t + 2 * r) % na], a1 = a[(8 * t + 2 * r + 1) % na];
            const v4i b0 = b[(8 * t + 2 * r) % nb], b1 = b[(8 * t + 2 * r + 1) % nb];
            A[r] = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
            B[r] = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[r], B[r], c0, 0, 0, 0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[(r + 1) & 3], B[r], c1, 0, 0, 0, 0, 0, 0);
                c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[r], B[(r + 2) & 3], c2, 0, 0, 0, 0, 0, 0);
                c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[(r + 3) & 3], B[(r + 1) & 3], c3, 0, 0, 0, 0,
                                                                     0, 0);
            }
        }
    } else {
        v8bf A[4], B[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            A[r] = __builtin_bit_cast(v8bf, a[(4 * t + r) % na]);
            B[r] = __builtin_bit_cast(v8bf, b[(4 * t + r) % nb]);
        }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[r], B[r], c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[(r + 1) & 3], B[r], c1, 0, 0, 0);
                c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[r], B[(r + 2) & 3], c2, 0, 0, 0);
                c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[(r + 3) & 3], B[(r + 1) & 3], c3, 0, 0, 0);
            }
        }
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += (c0[i] + c1[i]) + (c2[i] + c3[i]);
    out[t] = s;
}

// Gather of the rows named by t (query b, entry j: row b * rows_per_seq +
// t[b * k + j]), in the layout the sparse attention copies use: a wavefront
// takes 8 consecutive entries, lane l reads 16-byte piece l % 8 of every
// 128-byte line of entry l / 8's row, all LINES loads of a row group in
// flight together; the next group's index is loaded before this group's
// rows.  Entries outside [0, rows_per_seq) are skipped (their loads read row
// 0 and are discarded, so every group issues the same loads).  Each thread
// writes the XOR of the 32-bit words it used.
template <int LINES>
__global__ __launch_bounds__(kThreads) void gather_rate_kernel(const unsigned char *rows, long long rows_per_seq,
                                                               const int32_t *t, int k, int n_entries, uint32_t *out) {
    constexpr int kWaves = kThreads / 64;
    constexpr size_t kRowBytes = 128 * LINES;
    const int lane = threadIdx.x % 64;
    const int wave = (int)blockIdx.x * kWaves + (int)threadIdx.x / 64;
    const int nwaves = (int)gridDim.x * kWaves;
    const int ngroups = (n_entries + 7) / 8;
    const int sub = lane / 8, piece = 16 * (lane % 8);
    auto index_of = [&](int g) { return t[min(8 * g + sub, n_entries - 1)]; };
    uint32_t acc = 0;
    int ix = index_of(min(wave, ngroups - 1));
    for (int g = wave; g < ngroups; g += nwaves) {
        const int ix_next = index_of(min(g + nwaves, ngroups - 1));
        const int e = 8 * g + sub;
        const bool ok = e < n_entries && ix >= 0 && (long long)ix < rows_per_seq;
        const long long r = ok ? (long long)(e / k) * rows_per_seq + ix : 0;
        const unsigned char *src = rows + (size_t)r * kRowBytes + piece;
        v4i v[LINES];
#pragma unroll
        for (int q = 0; q < LINES; ++q) v[q] = *reinterpret_cast<const v4i *>(src + 128 * q);
        uint32_t x = 0;
#pragma unroll
        for (int q = 0; q < LINES; ++q) x ^= (uint32_t)(v[q][0] ^ v[q][1] ^ v[q][2] ^ v[q][3]);
        acc ^= ok ? x : 0u;
        ix = ix_next;
    }
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

template <int LINES>
void launch_gather(int lines, dim3 grid, hipStream_t st, const unsigned char *rows, long long rows_per_seq,
                   const int32_t *t, int k, int n_entries, uint32_t *out) {
    if constexpr (LINES <= 16) {
        if (lines == LINES)
            hipLaunchKernelGGL(gather_rate_kernel<LINES>, grid, dim3(kThreads), 0, st, rows, rows_per_seq, t, k,
                               n_entries, out);
        else
            launch_gather<LINES + 1>(lines, grid, st, rows, rows_per_seq, t, k, n_entries, out);
    }
}

}  // namespace

extern "C" int idxc_calib_gather_rate(const void *rows, size_t row_bytes, long long rows_per_seq, const int32_t *t,
                                      int nq, int k, int blocks, uint32_t *out, void *stream) {
    if (!rows || !t || !out) return IDXC_ERR_NULL;
    if (row_bytes % 128 != 0 || row_bytes < 128 || row_bytes > 16 * 128 || rows_per_seq < 1 || nq < 1 || k < 1 ||
        blocks < 1 || blocks > (1 << 20) || (long long)nq * k > (1ll << 30))
        return IDXC_ERR_SHAPE;
    if (((uintptr_t)rows | (uintptr_t)out) & 15u || (uintptr_t)t & 3u) return IDXC_ERR_ALIGN;
    launch_gather<1>((int)(row_bytes / 128), dim3(blocks), static_cast<hipStream_t>(stream),
                     static_cast<const unsigned char *>(rows), rows_per_seq, t, k, nq * k, out);
    return hipGetLastError() == hipSuccess ? IDXC_OK : IDXC_ERR_HIP;
}

extern "C" int idxc_calib_mfma_rate(int kind, const void *a, size_t a_bytes, const void *b, size_t b_bytes, int iters,
                                    int blocks, float *out, void *stream) {
    if (!a || !b || !out) return IDXC_ERR_NULL;
    if (a_bytes < 16 || b_bytes < 16 || iters < 1 || blocks < 1) return IDXC_ERR_SHAPE;
    if (((uintptr_t)a | (uintptr_t)b | (uintptr_t)out) & 15u) return IDXC_ERR_ALIGN;
    if (kind != IDXC_CALIB_FP8_32X32X64 && kind != IDXC_CALIB_BF16_32X32X16) return IDXC_ERR_DTYPE;
    const v4i *pa = static_cast<const v4i *>(a), *pb = static_cast<const v4i *>(b);
    const size_t na = a_bytes / 16, nb = b_bytes / 16;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (kind == IDXC_CALIB_FP8_32X32X64)
        hipLaunchKernelGGL(mfma_rate_kernel<IDXC_CALIB_FP8_32X32X64>, dim3(blocks), dim3(kThreads), 0, st, pa, na, pb,
                           nb, iters, out);
    else
        hipLaunchKernelGGL(mfma_rate_kernel<IDXC_CALIB_BF16_32X32X16>, dim3(blocks), dim3(kThreads), 0, st, pa, na,
                           pb, nb, iters, out);
    return hipGetLastError() == hipSuccess ? IDXC_OK : IDXC_ERR_HIP;
}
