// overlap.hip -- adjacent-layer index-set overlap.
//
// The measurement behind the cross-layer redundancy that IndexCache exploits
// (itoverdose.com, "IndexCache: Wie DeepSeek O(NL²)-Kosten in Sparse Attention
// um 75% reduziert", the introduction and section "Der unsichtbare
// Datenstrom": neighbouring layers pick largely the same top-k tokens;
// parapluman.nl, section "Aandacht cachen met IndexCache"): for every query
// row, how many of the indices one layer selected another layer selected too.
//
// Rows hold ascending indices followed by -1 padding, as the top-k writes
// them.  One wavefront per row: each valid entry of row a is looked up in row
// b by binary search (padding compares as +infinity), and the hits are
// counted with ballots.
#include "device_common.h"
#include "kernels.h"

namespace idxc {
namespace {

constexpr int kOverlapWaves = 4;

__device__ __forceinline__ int key_of(int v) { return v < 0 ? 0x7FFFFFFF : v; }

__global__ __launch_bounds__(kOverlapWaves * kWave) void overlap_kernel(OverlapArgs a) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int r = blockIdx.x * kOverlapWaves + wave;
    if (r >= a.R) return;
    const int32_t *ta = a.t_a + (size_t)r * a.topk;
    const int32_t *tb = a.t_b + (size_t)r * a.topk;
    int hits = 0;
    for (int j0 = 0; j0 < a.topk; j0 += kWave) {
        const int j = j0 + lane;
        const int x = j < a.topk ? ta[j] : -1;
        bool hit = false;
        if (x >= 0) {
            int lo = 0, hi = a.topk;   // first position with key >= x
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (key_of(tb[mid]) < x) lo = mid + 1;
                else hi = mid;
            }
            hit = lo < a.topk && tb[lo] == x;
        }
        hits += __popcll(ballot(hit));
    }
    if (lane == 0) a.counts[r] = hits;
}

}  // namespace

hipError_t launch_overlap(const OverlapArgs &a, hipStream_t st) {
    if (a.R <= 0) return hipSuccess;
    const unsigned nwg = (unsigned)((a.R + kOverlapWaves - 1) / kOverlapWaves);
    hipLaunchKernelGGL(overlap_kernel, dim3(nwg), dim3(kOverlapWaves * kWave), 0, st, a);
    return hipGetLastError();
}

}  // namespace idxc
