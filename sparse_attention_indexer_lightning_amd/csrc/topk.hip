// topk.hip -- exact per-row top-k over fp32 scores held in HBM.
//
// The top-k step of the inference loop in itoverdose.com, "IndexCache: Wie
// DeepSeek O(NL²)-Kosten in Sparse Attention um 75% reduziert", section
// "Einfache Implementierung, enorme Effizienzgewinne": T = top-k(I), with ties
// going to the lower key index and T written in ascending index order.
//
// One workgroup (16 wavefronts) per row.  The k-th largest order-preserving key
// is found by MSB-first radix select, four 8-bit digits, each digit one
// coalesced pass over the row with a shared LDS histogram.  The output pass
// walks the row in 1024-key chunks; one workgroup scan per chunk of the packed
// pair (count above the threshold, count equal to it) gives every kept key its
// output slot: slot = above_before + min(equal_before, equal_needed).  Keys
// are therefore written in ascending order with no sort.
#include "device_common.h"
#include "kernels.h"

namespace idxc {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;

__global__ __launch_bounds__(kThreads) void row_topk_kernel(TopkArgs a) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t wtot[kWaves];
    __shared__ int sh_bin;
    __shared__ uint32_t sh_above;

    const int r = blockIdx.x;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    int pos;
    if (a.pos_Lq > 0) pos = a.Lk - a.pos_Lq + r % a.pos_Lq;
    else pos = a.row_pos ? a.row_pos[r] : a.Lk - 1;
    pos = min(pos, a.Lk - 1);
    const int n = pos + 1 > 0 ? pos + 1 : 0;
    const int k = a.topk;
    int32_t *out = a.t_out + (size_t)r * k;
    if (n <= k) {
        for (int j = tid; j < k; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }
    const float *s = a.scores + (size_t)r * a.Lk;

    uint32_t prefix = 0, pmask = 0;
    int need = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int j = tid; j < 256; j += kThreads) hist[j] = 0;
        __syncthreads();
        for (int j = tid; j < n; j += kThreads) {
            const uint32_t u = score_key(s[j]);
            if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2],
                           h3 = hist[4 * lane + 3];
            const uint32_t sum = h0 + h1 + h2 + h3;
            uint32_t S = sum;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const uint32_t v = __shfl_down(S, o, kWave);
                if (lane + o < kWave) S += v;
            }
            const uint32_t E = S - sum;
            if (E < (uint32_t)need && S >= (uint32_t)need) {
                uint32_t c = E;
                int bsel;
                if (c + h3 >= (uint32_t)need) bsel = 3;
                else {
                    c += h3;
                    if (c + h2 >= (uint32_t)need) bsel = 2;
                    else {
                        c += h2;
                        if (c + h1 >= (uint32_t)need) bsel = 1;
                        else { c += h1; bsel = 0; }
                    }
                }
                sh_bin = 4 * lane + bsel;
                sh_above = c;
            }
        }
        __syncthreads();
        prefix |= (uint32_t)sh_bin << shift;
        pmask |= 0xFFu << shift;
        need -= (int)sh_above;
        __syncthreads();
    }

    // ordered output: slot = above_before + min(equal_before, need)
    uint32_t gt_base = 0, eq_base = 0;
    for (int c0 = 0; c0 < n; c0 += kThreads) {
        const int j = c0 + tid;
        uint32_t u = 0;
        if (j < n) u = score_key(s[j]);
        const bool gt = j < n && u > prefix;
        const bool eq = j < n && u == prefix;
        const uint64_t gm = ballot(gt), em = ballot(eq);
        if (lane == 0) wtot[wave] = (uint32_t)__popcll(gm) | ((uint32_t)__popcll(em) << 16);
        __syncthreads();
        uint32_t before = 0, total = 0;
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t v = wtot[w];
            if (w < wave) before += v;
            total += v;
        }
        const uint32_t gt_before = gt_base + (before & 0xFFFFu) + lanes_below(gm);
        const uint32_t eq_before = eq_base + (before >> 16) + lanes_below(em);
        if (gt || (eq && eq_before < (uint32_t)need)) {
            const uint32_t slot = gt_before + (eq_before < (uint32_t)need ? eq_before : (uint32_t)need);
            out[slot] = j;
        }
        gt_base += total & 0xFFFFu;
        eq_base += total >> 16;
        __syncthreads();
        if (gt_base + (eq_base < (uint32_t)need ? eq_base : (uint32_t)need) >= (uint32_t)k) break;
    }
}

}  // namespace

hipError_t launch_row_topk(const TopkArgs &a, hipStream_t st) {
    if (a.R <= 0) return hipSuccess;
    hipLaunchKernelGGL(row_topk_kernel, dim3((unsigned)a.R), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace idxc
