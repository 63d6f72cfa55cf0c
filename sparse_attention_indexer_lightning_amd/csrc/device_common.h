// device_common.h -- wavefront helpers and MFMA wrappers for gfx950 (CDNA4).
// Internal to libidxcache; every kernel here runs 64-lane wavefronts.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idxc {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0)); }

// number of set bits of `m` in lanes below the calling lane
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// the builtin takes the predicate as a lane mask (the HIP wrapper takes an
// int, which makes the compiler materialise a comparison result first)
__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// LDS instructions of one wavefront execute in issue order, so a later LDS
// read sees an earlier LDS write by any lane of the same wavefront as long
// as the compiler keeps program order; this is that compiler barrier.
__device__ __forceinline__ void wave_lds_order() { __asm__ volatile("" ::: "memory"); }

// Full wavefront-scope fence (waits for outstanding LDS operations).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Order-preserving 32-bit key of a score: larger key <=> larger float,
// with -0 and +0 mapped to the same key.  NaN is outside the contract.
__device__ __forceinline__ uint32_t score_key(float f) {
    const uint32_t u = __float_as_uint(f + 0.0f);   // -0 + 0 = +0; exact otherwise (denormals kept)
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// max(x, 0) for fp32 as one integer max: every negative float (-0 included)
// is a negative int32, every positive float a positive one.  Unlike fmaxf it
// needs no NaN canonicalisation of MFMA results.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// D(16x16, fp32) = A(16x128, fp8 e4m3) * B(128x16, fp8 e4m3) + C.
// Lane l supplies row/column l%16 and the 32 k-values 32*(l/16)..+31 of A/B;
// it receives D[4*(l/16)+i][l%16], i = 0..3.
__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i &a, const v8i &b, const v4f &c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

typedef float v16f __attribute__((ext_vector_type(16)));

// D(32x32, fp32) = A(32x64, fp8 e4m3) * B(64x32, fp8 e4m3) + C.
// Lane l supplies row/column l%32 and the 32 k-values 32*(l/32)..+31 of A/B;
// it receives D[8*(r/4) + 4*(l/32) + r%4][l%32] in register r = 0..15.
__device__ __forceinline__ v16f mfma_fp8_32x32x64(const v8i &a, const v8i &b, const v16f &c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// D(16x16, fp32) = A(16x32, bf16) * B(32x16, bf16) + C.
// Lane l supplies row/column l%16 and k-values 8*(l/16)..+7; output as above.
__device__ __forceinline__ v4f mfma_bf16_16x16x32(const v8bf &a, const v8bf &b, const v4f &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// s_waitcnt immediate for vmcnt(n) with the other counters unconstrained
// (vmcnt is split over bits 3:0 and 15:14).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Workgroup barrier ordering LDS accesses only.  __syncthreads also waits for
// every global load in flight (vmcnt(0)); kernels that keep loads in flight
// across the barrier wait for them with explicit vmcnt bounds instead.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m) { return __shfl_xor(v, m, kWave); }

}  // namespace idxc
