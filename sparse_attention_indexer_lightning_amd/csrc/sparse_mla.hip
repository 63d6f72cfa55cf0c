// sparse_mla.hip -- sparse MLA attention over the selected latent rows.
//
// itoverdose.com, "IndexCache: Wie DeepSeek O(NL²)-Kosten in Sparse Attention
// um 75% reduziert": the introduction (attention runs only over the k selected
// tokens) and section "Wie der Indexer funktioniert und warum MLA entscheidend
// ist" (every head reads one compressed latent row per token).  In the absorbed
// form all heads share the row: keys are the whole row (Dqk columns), values its
// first Dv columns.
//
// One workgroup (4 wavefronts) per (query, group of 16 heads).  The index set
// is consumed in blocks of 64 rows: the rows are gathered from HBM into LDS
// with 16-byte loads (coalesced within each row), wavefront w computes the
// 16 x 16 logit tile of rows 16w..16w+15 on bf16 MFMA (query fragment held in
// registers for the whole sweep), the online-softmax statistics are combined
// across the four wavefronts through LDS, the probabilities go to LDS as bf16,
// and each wavefront accumulates its share of the Dv output columns with a
// second MFMA (P x V).  Out-of-range and negative indices contribute nothing.
#include "device_common.h"
#include "kernels.h"

namespace idxc {
namespace {

constexpr int HG = 16;      // heads per workgroup
constexpr int BR = 64;      // selected rows per block
constexpr int kWavesMla = 4;

template <int DQK, int DV>
struct MlaLds {
    static constexpr int PITCH = DQK * 2 + 16;                 // bytes per gathered row
    static constexpr int KV = 0;
    static constexpr int P = KV + BR * PITCH;                  // bf16 [HG][BR]
    static constexpr int IDX = P + HG * BR * 2;                // int [BR]
    static constexpr int WMAX = IDX + BR * 4;                  // float [4][HG]
    static constexpr int WSUM = WMAX + kWavesMla * HG * 4;     // float [4][HG]
    static constexpr int TOTAL = WSUM + kWavesMla * HG * 4;
};

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <int DQK, int DV>
__global__ __launch_bounds__(kWavesMla * kWave) void sparse_mla_kernel(MlaArgs a) {
    using L = MlaLds<DQK, DV>;
    constexpr int KS = DQK / 32;              // k-steps of the logit MFMA
    constexpr int NT = DV / 16;               // 16-column output tiles
    constexpr int NTW = (NT + kWavesMla - 1) / kWavesMla;  // tiles per wavefront
    __shared__ __align__(16) unsigned char smem[L::TOTAL];
    unsigned char *kvs = smem + L::KV;
    uint16_t *P = reinterpret_cast<uint16_t *>(smem + L::P);
    int *idx = reinterpret_cast<int *>(smem + L::IDX);
    float *wmax = reinterpret_cast<float *>(smem + L::WMAX);
    float *wsum = reinterpret_cast<float *>(smem + L::WSUM);

    const int row = blockIdx.x;              // flat query b*Lq + i
    const int h0 = blockIdx.y * HG;
    const int b = row / a.Lq;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave, g = lane >> 4, n = lane & 15;
    const uint16_t *kvb = reinterpret_cast<const uint16_t *>(a.kv) + (size_t)b * a.Lk * DQK;
    const int32_t *trow = a.t + (size_t)row * a.topk;
    const float sl2 = a.sm_scale * 1.4426950408889634f;   // logits in log2 units

    // query fragment: A rows = heads h0 + n, k-values 32c + 8g .. +7
    v4i qa[KS];
    {
        const int h = h0 + n;
        const uint16_t *qh = reinterpret_cast<const uint16_t *>(a.q) + ((size_t)row * a.Hq + h) * DQK;
#pragma unroll
        for (int c = 0; c < KS; ++c)
            qa[c] = h < a.Hq ? *reinterpret_cast<const v4i *>(qh + 32 * c + 8 * g) : v4i{0, 0, 0, 0};
    }
    v4f o[NTW];
#pragma unroll
    for (int u = 0; u < NTW; ++u) o[u] = v4f{0.f, 0.f, 0.f, 0.f};
    float m_run[4], l_run[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { m_run[i] = -INFINITY; l_run[i] = 0.f; }

    for (int j0 = 0; j0 < a.topk; j0 += BR) {
        if (tid < BR) {
            int v = j0 + tid < a.topk ? trow[j0 + tid] : -1;
            idx[tid] = (v >= 0 && v < a.Lk) ? v : -1;
        }
        __syncthreads();
        // gather: BR rows x DQK bf16, 16-byte chunks
        constexpr int CPR = DQK / 8;        // chunks per row
        for (int c = tid; c < BR * CPR; c += kWavesMla * kWave) {
            const int rr = c / CPR, cc = c % CPR;
            const int sidx = idx[rr];
            v4i v = {0, 0, 0, 0};
            if (sidx >= 0) v = *reinterpret_cast<const v4i *>(kvb + (size_t)sidx * DQK + 8 * cc);
            *reinterpret_cast<v4i *>(kvs + rr * L::PITCH + 16 * cc) = v;
        }
        __syncthreads();

        // logits for rows 16*wave + n; lane holds heads 4g + i
        v4f s = {0.f, 0.f, 0.f, 0.f};
        {
            const unsigned char *kr = kvs + (16 * wave + n) * L::PITCH;
#pragma unroll
            for (int c = 0; c < KS; ++c) {
                const v4i kb = *reinterpret_cast<const v4i *>(kr + 64 * c + 16 * g);
                s = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, qa[c]), __builtin_bit_cast(v8bf, kb), s);
            }
        }
        const bool valid = idx[16 * wave + n] >= 0;
        float z[4], mx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            z[i] = valid ? s[i] * sl2 : -INFINITY;
            float v = z[i];
#pragma unroll
            for (int o2 = 1; o2 < 16; o2 <<= 1) v = fmaxf(v, shfl_xor(v, o2));
            mx[i] = v;
        }
        if (n == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) wmax[wave * HG + 4 * g + i] = mx[i];
        }
        __syncthreads();
        float m_new[4], alpha[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float m = m_run[i];
#pragma unroll
            for (int w = 0; w < kWavesMla; ++w) m = fmaxf(m, wmax[w * HG + 4 * g + i]);
            m_new[i] = m;
            alpha[i] = (m == -INFINITY) ? 1.f : exp2f(m_run[i] - m);
        }
        float ps[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float pv = (z[i] == -INFINITY) ? 0.f : exp2f(z[i] - m_new[i]);
            P[(4 * g + i) * BR + 16 * wave + n] = f32_to_bf16_rne(pv);
            float v = pv;
#pragma unroll
            for (int o2 = 1; o2 < 16; o2 <<= 1) v += shfl_xor(v, o2);
            ps[i] = v;
        }
        if (n == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) wsum[wave * HG + 4 * g + i] = ps[i];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float add = 0.f;
#pragma unroll
            for (int w = 0; w < kWavesMla; ++w) add += wsum[w * HG + 4 * g + i];
            l_run[i] = alpha[i] * l_run[i] + add;
            m_run[i] = m_new[i];
        }
        // O = alpha * O + P V for this wave's output tiles
#pragma unroll
        for (int u = 0; u < NTW; ++u) {
            const int nt = wave + kWavesMla * u;
            if (nt >= NT) break;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[u][i] *= alpha[i];
#pragma unroll
            for (int c = 0; c < BR / 32; ++c) {
                const v4i pa = *reinterpret_cast<const v4i *>(P + n * BR + 32 * c + 8 * g);
                uint16_t vb[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    vb[e] = *reinterpret_cast<const uint16_t *>(kvs + (32 * c + 8 * g + e) * L::PITCH +
                                                                2 * (16 * nt + n));
                v4i vv;
                vv[0] = (int)vb[0] | ((int)vb[1] << 16);
                vv[1] = (int)vb[2] | ((int)vb[3] << 16);
                vv[2] = (int)vb[4] | ((int)vb[5] << 16);
                vv[3] = (int)vb[6] | ((int)vb[7] << 16);
                o[u] = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, pa), __builtin_bit_cast(v8bf, vv), o[u]);
            }
        }
        __syncthreads();
    }

    // out[h][col]: lane holds heads 4g + i, column 16*nt + n
    uint16_t *ob = reinterpret_cast<uint16_t *>(a.out) + (size_t)row * a.Hq * DV;
#pragma unroll
    for (int u = 0; u < NTW; ++u) {
        const int nt = wave + kWavesMla * u;
        if (nt >= NT) break;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = h0 + 4 * g + i;
            if (h < a.Hq) {
                const float v = l_run[i] > 0.f ? o[u][i] / l_run[i] : 0.f;
                ob[(size_t)h * DV + 16 * nt + n] = f32_to_bf16_rne(v);
            }
        }
    }
    if (a.lse && wave == 0 && n == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = h0 + 4 * g + i;
            if (h < a.Hq)
                a.lse[(size_t)row * a.Hq + h] =
                    l_run[i] > 0.f ? (m_run[i] + log2f(l_run[i])) * 0.6931471805599453f : -INFINITY;
        }
    }
}

}  // namespace

hipError_t launch_sparse_mla(const MlaArgs &a, hipStream_t st) {
    const dim3 grid((unsigned)(a.B * a.Lq), (unsigned)((a.Hq + HG - 1) / HG));
    if (a.Dqk == 576 && a.Dv == 512) {
        hipLaunchKernelGGL((sparse_mla_kernel<576, 512>), grid, dim3(kWavesMla * kWave), 0, st, a);
    } else if (a.Dqk == 32 && a.Dv == 32) {
        hipLaunchKernelGGL((sparse_mla_kernel<32, 32>), grid, dim3(kWavesMla * kWave), 0, st, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace idxc
