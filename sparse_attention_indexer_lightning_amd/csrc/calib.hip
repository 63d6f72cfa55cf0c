// calib.hip -- dense MFMA chains on caller-given operand bytes (measurement
// support: the MFMA rate the benchmark's own operands allow on this part).
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

}  // namespace

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
