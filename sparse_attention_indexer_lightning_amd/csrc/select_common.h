// select_common.h -- block-wide radix selection shared by the top-k kernels
// and the decode score kernel (which derives its key range's top-k bound while
// the scores are in registers).  Internal to libidxcache.
#pragma once
#include "device_common.h"

namespace idxc {

constexpr int kLocal = 4;                  // keys kept per thread for a bound
constexpr int kDigit = 11;                 // radix digit width
constexpr int kBins = 1 << kDigit;

__device__ __forceinline__ uint32_t wave_max32(uint32_t v) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, kWave));
    return v;
}

// Insert u into a descending list of the 4 largest keys seen.
__device__ __forceinline__ void keep_top4(uint32_t (&top)[kLocal], uint32_t u) {
    if (u > top[3]) {
        top[3] = u;
        if (top[3] > top[2]) { const uint32_t x = top[2]; top[2] = top[3]; top[3] = x; }
        if (top[2] > top[1]) { const uint32_t x = top[1]; top[1] = top[2]; top[2] = x; }
        if (top[1] > top[0]) { const uint32_t x = top[0]; top[0] = top[1]; top[1] = x; }
    }
}

// The need-th largest key among `n` keys produced by get(i) (block-wide),
// returning the key and, through *above, how many keys are strictly larger.
// MSB-first radix select with 11-bit digits, starting below the bits that the
// smallest and largest key share (so the first digit already spreads keys).
template <int NT, typename Sh, typename Get>
__device__ uint32_t block_select(Sh &sh, int n, int need, Get get, uint32_t *above_out) {
    constexpr int NW = NT / kWave;
    constexpr int BPT = kBins / NT;            // histogram bins per thread
    static_assert(BPT == 2 || (BPT % 4 == 0 && BPT > 0), "bins per thread: 2 or a multiple of 4");
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    for (int i = tid; i < n; i += NT) {
        const uint32_t u = get(i);
        mn = min(mn, u);
        mx = max(mx, u);
    }
    mn = ~wave_max32(~mn);
    mx = wave_max32(mx);
    if (lane == 0) { sh.wtot[0][wave] = mn; sh.wtot[1][wave] = mx; }
    __syncthreads();
    mn = 0xFFFFFFFFu; mx = 0u;
    for (int w = 0; w < NW; ++w) { mn = min(mn, sh.wtot[0][w]); mx = max(mx, sh.wtot[1][w]); }
    int top = (mn == mx) ? 0 : 32 - __builtin_clz(mn ^ mx);
    const bool top_was_zero = top == 0;   // block-uniform: mn, mx come from the same LDS words
    uint32_t pmask = top == 32 ? 0u : ~((1u << top) - 1u);
    uint32_t prefix = mn & pmask;
    uint32_t above_total = 0;
    while (top > 0) {
        const int width = top < kDigit ? top : kDigit;
        const int shift = top - width;
        const uint32_t dmask = (1u << width) - 1u;
        for (int j = tid; j < kBins; j += NT) sh.hist[j] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += NT) {
            const uint32_t u = get(i);
            if ((u & pmask) == prefix) atomicAdd(&sh.hist[(u >> shift) & dmask], 1u);
        }
        __syncthreads();
        // Suffix sums over the bins, highest first.  Thread t owns the BPT
        // consecutive bins [BPT t, BPT t + BPT) (one 8- or 16-byte LDS read
        // each); a wavefront scan and the wavefront totals give every thread
        // S = the keys in its bins and above, and the one thread whose bins
        // hold the need-th largest key picks the bin.
        uint32_t h[BPT];
        if constexpr (BPT == 2) {
            const uint2 v = *reinterpret_cast<const uint2 *>(&sh.hist[2 * tid]);
            h[0] = v.x;
            h[1] = v.y;
        } else {
#pragma unroll
            for (int j = 0; j < BPT; j += 4) {
                const uint4 v = *reinterpret_cast<const uint4 *>(&sh.hist[BPT * tid + j]);
                h[j] = v.x;
                h[j + 1] = v.y;
                h[j + 2] = v.z;
                h[j + 3] = v.w;
            }
        }
        uint32_t sum = 0;
#pragma unroll
        for (int j = 0; j < BPT; ++j) sum += h[j];
        uint32_t S = sum;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const uint32_t v = __shfl_down(S, o, kWave);
            if (lane + o < kWave) S += v;
        }
        if (lane == 0) sh.wtot[0][wave] = S;
        __syncthreads();
        for (int w = wave + 1; w < NW; ++w) S += sh.wtot[0][w];
        const uint32_t E = S - sum;
        if (E < (uint32_t)need && S >= (uint32_t)need) {
            uint32_t c = E;
            int bsel = 0;
#pragma unroll
            for (int j = BPT - 1; j >= 0; --j) {
                if (c + h[j] >= (uint32_t)need) {
                    bsel = j;
                    break;
                }
                c += h[j];
            }
            sh.sh_bin = BPT * tid + bsel;
            sh.sh_above = c;
        }
        __syncthreads();
        prefix |= (uint32_t)sh.sh_bin << shift;
        pmask |= dmask << shift;
        need -= (int)sh.sh_above;
        above_total += sh.sh_above;
        top = shift;
        __syncthreads();
    }
    // Every caller writes sh.wtot next.  When all keys are equal the loop above
    // never runs, so without this barrier a wavefront could overwrite a slot
    // that a slower one is still reading in the min/max reduction.
    if (top_was_zero) __syncthreads();
    *above_out = above_total;
    return prefix;
}

// Shared memory of split_bound for a 256-thread block.
struct BoundShared {
    uint32_t ukey[256 * kLocal];
    alignas(16) uint32_t hist[kBins];   // read as 16-byte vectors
    uint32_t wtot[2][256 / kWave];
    int sh_bin;
    uint32_t sh_above;
};

// Lower bound on the m-th largest key of split s of a row whose first n keys
// are valid, split into ranges of N keys, from every thread's 4 largest keys
// of its share (top, descending) -- their m-th largest is <= the split's.
// Only the F = n / N completely filled splits vouch for keys, m = ceil(k / F)
// each, so that at least F * m >= k keys of the row are >= the minimum over
// the splits; the others report the neutral maximum.  With F = 0, or m beyond
// the per-thread lists, the bound is 0 (no pruning for the row).  Block-wide
// (NT threads); the result is valid in every thread.
template <int NT, typename Sh>
__device__ uint32_t split_bound(Sh &sh, const uint32_t (&top)[kLocal], int n, int N, int s, int k) {
    const int full = n / N;
    if (full == 0 || s >= full) return (full == 0 && s == 0) ? 0u : 0xFFFFFFFFu;
    const int m = (k + full - 1) / full;
    if (m > NT * kLocal) return 0u;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kLocal; ++i) sh.ukey[tid * kLocal + i] = top[i];
    __syncthreads();
    uint32_t dummy;
    return block_select<NT>(sh, NT * kLocal, m, [&](int i) { return sh.ukey[i]; }, &dummy);
}

}  // namespace idxc
