// topk.hip -- exact per-row top-k over fp32 scores held in HBM.
//
// The top-k step of the inference loop in itoverdose.com, "IndexCache: Wie
// DeepSeek O(NL²)-Kosten in Sparse Attention um 75% reduziert", section
// "Einfache Implementierung, enorme Effizienzgewinne": T = top-k(I), with ties
// going to the lower key index and T written in ascending index order.
//
// Everything runs on order-preserving 32-bit keys of the scores.
//
// Few long rows (decode: 32 rows of 200K scores) are split over S workgroups
// each, in three launches:
//  1. bound: split s of a row computes a lower bound b_s on its own m-th
//     largest key, m = ceil(k / S) (the m-th largest of the union of
//     per-thread top-4 lists, a subset of the split).  At least m keys of the
//     split are >= b_s, so at least S*m >= k keys of the row are >= min_s b_s:
//     theta = min_s b_s never exceeds the row's k-th largest key;
//  2. collect: each quarter of a split (one wavefront) writes its keys >=
//     theta, in index order, to its own region of the workspace;
//  3. select: one workgroup per row loads the candidates of all regions (in
//     split and quarter order, so in index order) into LDS and runs the
//     exact selection.
// Otherwise one workgroup (16 wavefronts) handles a whole row:
//  1. bound: every thread keeps the 4 largest keys of its strided share of
//     the row; the k-th largest of these 4096 keys is <= the row's k-th
//     largest key (they are a subset of the row), so every member of the
//     top-k is >= it;
//  2. collect: one coalesced pass appends every key >= the bound to an LDS
//     candidate list in ascending index order (block prefix sums);
//  3. select: exact MSB-first radix select on the candidates, then one
//     ordered pass writes the indices above the k-th key plus the lowest-index
//     ties.
// For i.i.d. scores the candidate list is a little over k long.  If it would
// not fit in LDS, the row falls back to radix selection over the row in HBM.
#include "device_common.h"
#include "kernels.h"
#include "select_common.h"

namespace idxc {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnion = kThreads * kLocal;  // 4096
constexpr int kCandCap = 8192;             // LDS candidate capacity

struct TopkShared {
    uint32_t ukey[kUnion];          // step 1 union, then reused
    uint32_t ckey[kCandCap];        // candidates: key
    int32_t cidx[kCandCap];         //             index
    alignas(16) uint32_t hist[kBins];   // read as 8-byte vectors
    uint32_t wtot[2][kWaves];
    int sh_bin;
    uint32_t sh_above;
};

// Ordered output of the top-k from keys get(i), i < n, in index order:
// slot = above_before + min(equal_before, need_eq), index = idx(i).
template <typename Get, typename Idx>
__device__ void ordered_output(TopkShared &sh, int n, uint32_t theta, int need_eq, int k, Get get, Idx idx,
                               int32_t *out) {
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    uint32_t gt_base = 0, eq_base = 0;
    int par = 0;
    for (int c0 = 0; c0 < n; c0 += kThreads, par ^= 1) {
        const int j = c0 + tid;
        const uint32_t u = j < n ? get(j) : 0u;
        const bool gt = j < n && u > theta;
        const bool eq = j < n && u == theta;
        const uint64_t gm = ballot(gt), em = ballot(eq);
        if (lane == 0) sh.wtot[par][wave] = (uint32_t)__popcll(gm) | ((uint32_t)__popcll(em) << 16);
        __syncthreads();
        uint32_t before = 0, total = 0;
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t v = sh.wtot[par][w];
            if (w < wave) before += v;
            total += v;
        }
        const uint32_t gt_before = gt_base + (before & 0xFFFFu) + lanes_below(gm);
        const uint32_t eq_before = eq_base + (before >> 16) + lanes_below(em);
        const uint32_t ne = (uint32_t)need_eq;
        if (gt || (eq && eq_before < ne)) out[gt_before + (eq_before < ne ? eq_before : ne)] = idx(j);
        gt_base += total & 0xFFFFu;
        eq_base += total >> 16;
        if (gt_base + (eq_base < ne ? eq_base : ne) >= (uint32_t)k) break;
    }
}

__global__ __launch_bounds__(kThreads) void row_topk_kernel(TopkArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    TopkShared &sh = *reinterpret_cast<TopkShared *>(smem_raw);
    const int r = blockIdx.x;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
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

    // 1. lower bound from the union of per-thread top-4 lists
    uint32_t top[kLocal] = {0u, 0u, 0u, 0u};
    for (int c0 = 0; c0 < n; c0 += 4 * kThreads) {
        const int j0 = c0 + 4 * tid;
        uint32_t u[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = j0 + e < n ? score_key(s[j0 + e]) : 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) keep_top4(top, u[e]);
    }
#pragma unroll
    for (int i = 0; i < kLocal; ++i) sh.ukey[tid * kLocal + i] = top[i];
    __syncthreads();
    uint32_t dummy;
    const uint32_t bound = block_select<kThreads>(sh, kUnion, k, [&](int i) { return sh.ukey[i]; }, &dummy);

    // 2. collect keys >= bound in index order (4 per thread per step)
    uint32_t base = 0;
    bool overflow = false;
    int par = 0;
    const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    for (int c0 = 0; c0 < n; c0 += 4 * kThreads, par ^= 1) {
        const int j0 = c0 + 4 * tid;
        uint32_t u[4];
        bool f[4];
        uint64_t B[4];
        int below = 0, mine = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            u[e] = j0 + e < n ? score_key(s[j0 + e]) : 0u;
            f[e] = j0 + e < n && u[e] >= bound;
            B[e] = ballot(f[e]);
            below += __popcll(B[e] & lt);
            mine += __popcll(B[e]);
        }
        if (lane == 0) sh.wtot[par][wave] = (uint32_t)mine;
        __syncthreads();
        uint32_t wbefore = 0, total = 0;
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t v = sh.wtot[par][w];
            if (w < wave) wbefore += v;
            total += v;
        }
        uint32_t p = base + wbefore + (uint32_t)below;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (f[e]) {
                if (p < (uint32_t)kCandCap) { sh.ckey[p] = u[e]; sh.cidx[p] = j0 + e; }
                ++p;
            }
        }
        base += total;
        if (base > (uint32_t)kCandCap) { overflow = true; break; }
    }
    __syncthreads();

    if (!overflow) {
        // 3. exact selection among the candidates
        const int nc = (int)base;
        uint32_t above;
        const uint32_t theta = block_select<kThreads>(sh, nc, k, [&](int i) { return sh.ckey[i]; }, &above);
        const int need_eq = k - (int)above;
        ordered_output(sh, nc, theta, need_eq, k, [&](int i) { return sh.ckey[i]; },
                       [&](int i) { return sh.cidx[i]; }, out);
        return;
    }
    // fallback: radix selection over the row in HBM
    uint32_t above;
    const uint32_t theta = block_select<kThreads>(sh, n, k, [&](int i) { return score_key(s[i]); }, &above);
    ordered_output(sh, n, theta, k - (int)above, k, [&](int i) { return score_key(s[i]); },
                   [&](int i) { return i; }, out);
}

// ------------------------------------------------------------ split rows

constexpr int kSplitThreads = 256;
constexpr int kSplitWaves = kSplitThreads / kWave;
constexpr int kMinSplit = 4096;        // keys per split at least
constexpr int kSplitTarget = 512;      // aim for about this many workgroups in total
constexpr int kSplitVec = 16;          // keys per thread per step (bound pass)
constexpr int kCollectVec = 32;        // collect: keys per lane whose loads are issued together
constexpr int kRegions = kSplitWaves;  // candidate regions per split: one per collect wavefront
static_assert(kSplitTarget * kRegions <= 2 * kThreads, "region offsets: two per select thread");


struct SplitPlan {
    int S;          // splits per row (1: whole-row kernel)
    int N;          // keys per split
};

__host__ inline SplitPlan split_plan(int R, int Lk) {
    SplitPlan pl{1, Lk};
    if (R <= 0 || R >= kSplitTarget / 2 || Lk < 4 * kMinSplit) return pl;
    int S = (kSplitTarget + R - 1) / R;
    if (S > Lk / kMinSplit) S = Lk / kMinSplit;
    if (S < 2) return pl;
    pl.S = S;
    pl.N = ((Lk + S - 1) / S + 255) / 256 * 256;   // whole 256-key steps, as the decode score kernel's ranges
    return pl;
}

struct SplitWs {
    uint32_t *bound;     // [R][S]
    int *count;          // [R][S][kRegions]
    uint2 *cand;         // [R][S][kRegions][N / kRegions]: (key, index)
    size_t bytes;
};

__host__ __device__ inline SplitWs split_ws(void *base, int R, const SplitPlan &pl) {
    SplitWs w;
    unsigned char *p = static_cast<unsigned char *>(base);
    const size_t rs = (size_t)R * pl.S;
    size_t off = 0;
    w.bound = reinterpret_cast<uint32_t *>(p + off);
    off += (rs * 4 + 255) & ~(size_t)255;
    w.count = reinterpret_cast<int *>(p + off);
    off += (rs * kRegions * 4 + 255) & ~(size_t)255;
    w.cand = reinterpret_cast<uint2 *>(p + off);
    off += rs * pl.N * 8;
    w.bytes = off;
    return w;
}

__device__ __forceinline__ int row_valid(const TopkArgs &a, int r) {
    int pos;
    if (a.pos_Lq > 0) pos = a.Lk - a.pos_Lq + r % a.pos_Lq;
    else pos = a.row_pos ? a.row_pos[r] : a.Lk - 1;
    pos = min(pos, a.Lk - 1);
    return pos + 1 > 0 ? pos + 1 : 0;
}

// 1. per split: a lower bound on its m-th largest key (split_bound).  The
// decode score kernel computes the same bounds while scoring when its key
// ranges are these splits; the launch then skips this kernel.
__global__ __launch_bounds__(kSplitThreads) void topk_split_bound(TopkArgs a, SplitPlan pl, SplitWs ws) {
    __shared__ BoundShared sh;
    const int s = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
    const int n = row_valid(a, r);
    const int j0 = s * pl.N, j1 = min(j0 + pl.N, n);
    const float *row = a.scores + (size_t)r * a.Lk;
    uint32_t top[kLocal] = {0u, 0u, 0u, 0u};
    if (n / pl.N > s) {   // filled splits only (split_bound ignores the others)
        for (int c0 = j0; c0 < j1; c0 += kSplitVec * kSplitThreads) {
            float v[kSplitVec];
#pragma unroll
            for (int e = 0; e < kSplitVec; ++e) {
                const int j = c0 + e * kSplitThreads + tid;
                v[e] = j < j1 ? row[j] : -INFINITY;
            }
#pragma unroll
            for (int e = 0; e < kSplitVec; ++e) keep_top4(top, score_key(v[e]));
        }
    }
    const uint32_t b = split_bound<kSplitThreads>(sh, top, n, pl.N, s, a.topk);
    if (tid == 0) ws.bound[(size_t)r * pl.S + s] = b;
}

// 2. per split: keys >= theta = min over the row's bounds, in index order.
// Wavefront w of a split takes the w-th quarter of its keys (N is a multiple
// of 256) and appends its candidates, in index order, to a region of its own
// (ballot + lane prefix per 64 keys): no block-wide ordering, so no barriers.
// The regions of a row, in (split, wavefront) order, are in index order.
__global__ __launch_bounds__(kSplitThreads) void topk_split_collect(TopkArgs a, SplitPlan pl, SplitWs ws) {
    const int s = blockIdx.x, r = blockIdx.y, tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / kWave),
              lane = tid % kWave;
    const int n = row_valid(a, r);
    const int q = pl.N / kRegions;
    const int j0 = s * pl.N + wave * q, j1 = min(j0 + q, n);
    const float *row = a.scores + (size_t)r * a.Lk;
    float v[kCollectVec];
    auto load_chunk = [&](int c0) {
#pragma unroll
        for (int e = 0; e < kCollectVec; ++e) {
            const int j = c0 + e * kWave + lane;
            v[e] = j < j1 ? row[j] : -INFINITY;
        }
    };
    // the first chunk's loads go out before theta's (bounds, then a wave minimum)
    load_chunk(j0);
    uint32_t tmin = 0xFFFFFFFFu;
    for (int i = lane; i < pl.S; i += kWave) tmin = min(tmin, ws.bound[(size_t)r * pl.S + i]);
    const uint32_t theta = ~wave_max32(~tmin);
    uint2 *out = ws.cand + ((size_t)r * pl.S + s) * pl.N + (size_t)wave * q;
    uint32_t cnt = 0;
    for (int c0 = j0; c0 < j1; c0 += kCollectVec * kWave) {
        if (c0 != j0) load_chunk(c0);
#pragma unroll
        for (int e = 0; e < kCollectVec; ++e) {
            const int j = c0 + e * kWave + lane;
            const uint32_t u = score_key(v[e]);
            const bool keep = j < j1 && u >= theta;
            const uint64_t B = ballot(keep);
            if (keep) out[cnt + (uint32_t)lanes_below(B)] = make_uint2(u, (uint32_t)j);
            cnt += (uint32_t)__popcll(B);
        }
    }
    if (lane == 0) ws.count[((size_t)r * pl.S + s) * kRegions + wave] = (int)cnt;
}

// 3. per row: exact selection over all splits' candidates.
__global__ __launch_bounds__(kThreads) void topk_split_select(TopkArgs a, SplitPlan pl, SplitWs ws) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    TopkShared &sh = *reinterpret_cast<TopkShared *>(smem_raw);
    const int r = blockIdx.x, tid = threadIdx.x;
    const int n = row_valid(a, r);
    const int k = a.topk;
    int32_t *out = a.t_out + (size_t)r * k;
    if (n <= k) {
        for (int j = tid; j < k; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }
    // offsets of the candidate regions, (split, wavefront) order being index
    // order: two counts per thread, a wavefront scan, then the wavefront totals
    int *soff = reinterpret_cast<int *>(sh.ukey);   // [nreg + 1]; ukey is unused here
    const int nreg = pl.S * kRegions;
    const int q = pl.N / kRegions;
    {
        const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
        const int i0 = 2 * tid;
        const int c0 = i0 < nreg ? ws.count[(size_t)r * nreg + i0] : 0;
        const int c1 = i0 + 1 < nreg ? ws.count[(size_t)r * nreg + i0 + 1] : 0;
        const int sum = c0 + c1;
        int incl = sum;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int t = __shfl_up(incl, d, kWave);
            if (lane >= d) incl += t;
        }
        if (lane == kWave - 1) sh.wtot[0][wave] = (uint32_t)incl;
        __syncthreads();
        int woff = 0;
        for (int w = 0; w < wave; ++w) woff += (int)sh.wtot[0][w];
        const int ex = woff + incl - sum;
        if (i0 < nreg) soff[i0] = ex;
        if (i0 + 1 < nreg) soff[i0 + 1] = ex + c0;
        if (tid == kThreads - 1) soff[nreg] = ex + sum;
    }
    __syncthreads();
    const int total = soff[nreg];
    if (total <= kCandCap) {
        // gather the candidates of every region: candidate g of the row is
        // entry g - soff[i] of the last region i with soff[i] <= g; each
        // thread issues all its loads before storing any
        constexpr int kPer = kCandCap / kThreads;
        uint2 v[kPer];
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int gi = tid + e * kThreads;
            if (gi < total) {
                int lo = 0, hi = nreg - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (soff[mid] <= gi) lo = mid;
                    else hi = mid - 1;
                }
                v[e] = ws.cand[(size_t)r * pl.S * pl.N + (size_t)lo * q + (gi - soff[lo])];
            }
        }
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int gi = tid + e * kThreads;
            if (gi < total) {
                sh.ckey[gi] = v[e].x;
                sh.cidx[gi] = (int32_t)v[e].y;
            }
        }
        __syncthreads();
        uint32_t above;
        const uint32_t theta = block_select<kThreads>(sh, total, k, [&](int i) { return sh.ckey[i]; }, &above);
        ordered_output(sh, total, theta, k - (int)above, k, [&](int i) { return sh.ckey[i]; },
                       [&](int i) { return sh.cidx[i]; }, out);
        return;
    }
    // too many candidates for LDS: radix selection over the row in HBM
    const float *srow = a.scores + (size_t)r * a.Lk;
    uint32_t above;
    const uint32_t theta = block_select<kThreads>(sh, n, k, [&](int i) { return score_key(srow[i]); }, &above);
    ordered_output(sh, n, theta, k - (int)above, k, [&](int i) { return score_key(srow[i]); },
                   [&](int i) { return i; }, out);
}

}  // namespace

bool row_topk_split_geometry(int R, int Lk, int *S, int *N) {
    const SplitPlan pl = split_plan(R, Lk);
    *S = pl.S;
    *N = pl.N;
    return pl.S > 1;
}

uint32_t *row_topk_split_bounds(void *ws, int R, int Lk) {
    const SplitPlan pl = split_plan(R, Lk);
    return pl.S > 1 ? split_ws(ws, R, pl).bound : nullptr;
}

size_t row_topk_ws_bytes(int R, int Lk) {
    const SplitPlan pl = split_plan(R, Lk);
    if (pl.S == 1) return 0;
    return split_ws(nullptr, R, pl).bytes;
}

hipError_t launch_row_topk(const TopkArgs &a, hipStream_t st) {
    if (a.R <= 0) return hipSuccess;
    const size_t lds = sizeof(TopkShared);
    const SplitPlan pl = split_plan(a.R, a.Lk);
    if (pl.S > 1) {
        const SplitWs ws = split_ws(a.ws, a.R, pl);
        if (!a.ws || a.ws_bytes < ws.bytes) return hipErrorInvalidValue;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(topk_split_select),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        const dim3 g((unsigned)pl.S, (unsigned)a.R);
        if (!a.bounds_given) hipLaunchKernelGGL(topk_split_bound, g, dim3(kSplitThreads), 0, st, a, pl, ws);
        hipLaunchKernelGGL(topk_split_collect, g, dim3(kSplitThreads), 0, st, a, pl, ws);
        hipLaunchKernelGGL(topk_split_select, dim3((unsigned)a.R), dim3(kThreads), lds, st, a, pl, ws);
        return hipGetLastError();
    }
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(row_topk_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(row_topk_kernel, dim3((unsigned)a.R), dim3(kThreads), lds, st, a);
    return hipGetLastError();
}

}  // namespace idxc
