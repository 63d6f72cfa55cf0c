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
#include <type_traits>

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

// ---------------------------------------------------------------------------
// Latent-row kernel for the MLA shape (Dqk = 576 latent + rope columns,
// Dv = 512).  One workgroup per (query, group of 16 heads), four wavefronts
// in two pairs.  Pair p consumes tiles p, p+2, p+4, ... of 32 selected rows:
//  * the rows of a tile are copied straight from HBM into an LDS slot with
//    LDS-direct 16-byte loads (each load moves one 128-byte line, an "octet"
//    of eight 16-byte pieces, of 8 rows; slots are octet-major
//    [octet][row][piece] with the pieces rotated per row).  Each pair
//    owns two slots, so the copy of its next tile overlaps the current one;
//  * wavefront (p, h) computes the logits of rows 16h .. 16h+15 of the tile,
//    transposed: S^T = K Q^T (rows x heads), from the slot and the query
//    fragments held in registers;
//  * the softmax reference is shared by the pair and raised lazily (only when
//    a logit exceeds it by more than kSlack, which is rare), so the common
//    path needs no cross-wave exchange before the probabilities are formed;
//    the bf16 probabilities of both halves meet in a small LDS tile;
//  * wavefront (p, h) accumulates output columns 256h .. 256h+255 over all 32
//    rows: O^T += V^T P^T, V^T read from the slot with transposing LDS loads;
//  * at the end the two pairs' (reference, sum, O) states are merged in LDS.
// Workgroup ids are remapped so that the head groups of one query are
// dispatched to the same XCD and share its L2 copy of the gathered rows.
namespace latent {
constexpr int DQK = 576, DV = 512;
constexpr int RT = 32;                        // rows per tile
constexpr int ROWB = DQK * 2;                 // bytes per latent row
constexpr int PIECES = ROWB / 16;             // 16-byte pieces per row
constexpr int OCTETS = PIECES / 8;            // 128-byte lines per row
constexpr int OCT_BYTES = RT * 128;           // one octet of every row of a tile
constexpr int SLOT = OCTETS * OCT_BYTES;      // bytes per tile
constexpr int WAVES = 4;
constexpr int KC = DQK / 32;                  // logit k-steps
constexpr int MTW = DV / 2 / 16;              // output tiles per wavefront
constexpr int OPITCH = DV + 4;                // floats per head in the merge buffer
constexpr float kSlack = 8.f;                 // lazy-raise margin of the softmax reference (log2 units)
constexpr int kMaxTopk = 2048;                // index sets up to this size
static_assert(PIECES % 8 == 0, "rows are whole octets");
static_assert(2 * OCTETS == KC, "one copy load per logit k-step");
static_assert(2 * 16 * OPITCH * 4 <= 2 * SLOT, "merge buffer must fit in one buffer set");

// Piece rotation of row r: piece 8q + s of the row is stored at position
// (s + r) mod 8 of octet q.  Rows of an octet are 128 bytes apart; the
// rotation spreads the 16-row x one-piece logit reads over all banks (the
// transposing reads cost the same for any placement).
__device__ __forceinline__ int pos_of(int s, int r) { return (s + r) & 7; }
__device__ __forceinline__ int piece_at(int p, int r) { return (p - r) & 7; }

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

__device__ __forceinline__ v4s lds_read_tr16(const lds_u8 *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)p);
}
__device__ __forceinline__ v4i lds_read_b128(const lds_u8 *p) { return *(const __attribute__((address_space(3))) v4i *)p; }

// Copy of 16 rows (two groups of 8) of a tile: load (Q, hl) moves octet Q of
// rows 8*hl0 + 8*hl .. +7 (lane l: row + l/8, position l%8).  The immediate
// offset 128Q applies to the global and to the LDS address, so the LDS base
// is lowered by the same amount.
template <int Q>
__device__ __forceinline__ void fill_octets(const unsigned char *s0, const unsigned char *s1, lds_u8 *slot, int hl0) {
    if constexpr (Q < OCTETS) {
        __builtin_amdgcn_global_load_lds(s0, (__attribute__((address_space(3))) void *)(slot + (OCT_BYTES - 128) * Q + 1024 * hl0),
                                         16, 128 * Q, 0);
        __builtin_amdgcn_global_load_lds(s1, (__attribute__((address_space(3))) void *)(slot + (OCT_BYTES - 128) * Q + 1024 * (hl0 + 1)),
                                         16, 128 * Q, 0);
        fill_octets<Q + 1>(s0, s1, slot, hl0);
    }
}

// max / sum over the four 16-lane groups, result in every lane
__device__ __forceinline__ float group_max4(float v) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum4(float v) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__global__ __launch_bounds__(WAVES * kWave) void sparse_mla_latent_kernel(MlaArgs a) {
    // Separate LDS objects per buffer parity: the LDS-direct copies into one
    // set are then not waited for by reads of the other.
    __shared__ __align__(16) unsigned char bufE[2 * SLOT];     // [pair] tiles of even steps
    __shared__ __align__(16) unsigned char bufO[2 * SLOT];     // [pair] tiles of odd steps
    __shared__ __align__(16) unsigned char ptile[2][16 * 4 * 2 * 4 * 2];   // [pair][head][g][half][4] bf16
    __shared__ float xmax[2][2][16];                           // [pair][half][head]
    __shared__ int raise_flag[WAVES];
    __shared__ float mstat[WAVES][16], lstat[WAVES][16];
    __shared__ __align__(16) int tidx[kMaxTopk + 2 * RT];      // index row, -1 padded

    const int ng = a.Hq / 16;
    const int total = a.B * a.Lq * ng;
    int id = (int)blockIdx.x;
    if (total % 8 == 0) id = (id % 8) * (total / 8) + id / 8;   // one query's groups on one XCD
    const int qrow = id / ng, h0 = (id % ng) * 16;
    const int b = qrow / a.Lq;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int pair = wave >> 1, half = wave & 1;
    const int n = lane & 15, g = lane >> 4;
    const unsigned char *kvb = static_cast<const unsigned char *>(a.kv) + (size_t)b * a.Lk * ROWB;
    const int32_t *trow = a.t + (size_t)qrow * a.topk;
    const float sl2 = a.sm_scale * 1.4426950408889634f;

    // query fragments (B operand of S^T): head h0 + n, piece 4c + g of the row
    v4i qf[KC];
    {
        const v4i *qh = reinterpret_cast<const v4i *>(static_cast<const unsigned char *>(a.q) +
                                                      ((size_t)qrow * a.Hq + h0 + n) * ROWB);
#pragma unroll
        for (int c = 0; c < KC; ++c) qf[c] = qh[4 * c + g];
    }
    // logit A operand: own row r = 16*half + n, piece 4c + g = octet c/2, position 4(c&1) + g
    const int kr = 16 * half + n;
    const int kb_even = pair * SLOT + 128 * kr + 16 * pos_of(g, kr);
    const int kb_odd = pair * SLOT + 128 * kr + 16 * pos_of(4 + g, kr);
    // transposing reads of V: lane (g, j, cc) -> row 16*hh + 4g + j, columns 256*half + 16*mt + 4cc .. +3
    // (piece 32*half + 2mt + cc/2 = octet 4*half + mt/4, position 2(mt&3) + cc/2)
    int vbase[2][4];
    {
        const int j = (lane & 15) >> 2, cc = lane & 3;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int r = 16 * hh + 4 * g + j;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                vbase[hh][k] = pair * SLOT + 4 * half * OCT_BYTES + 128 * r + 16 * pos_of(2 * k + (cc >> 1), r) + 8 * (cc & 1);
        }
    }
    // copy: lane l fills position l%8 of rows 16*half + 8*hl + l/8
    const int lrow = lane >> 3;
    const int pofs0 = 16 * piece_at(lane & 7, 16 * half + lrow);
    const int pofs1 = 16 * piece_at(lane & 7, 16 * half + 8 + lrow);

    const int ntiles = (a.topk + RT - 1) / RT;
    const int steps = (ntiles + 1) / 2;           // every wavefront runs the same number of steps
    // the index row, -1 padded to whole steps, lives in LDS for the whole sweep
    for (int j = tid; j < 2 * RT * steps; j += WAVES * kWave) tidx[j] = j < a.topk ? trow[j] : -1;
    __syncthreads();
    // copy sources of step s: rows 16*half + lrow and 16*half + 8 + lrow of tile 2s + pair
    auto copy_src = [&](int s, const unsigned char *&s0, const unsigned char *&s1) {
        const int base = RT * (2 * s + pair) + 16 * half + lrow;
        const int i0 = tidx[base], i1 = tidx[base + 8];
        const int r0 = (i0 >= 0 && i0 < a.Lk) ? i0 : 0;
        const int r1 = (i1 >= 0 && i1 < a.Lk) ? i1 : 0;
        s0 = kvb + (size_t)(uint32_t)r0 * ROWB + pofs0;
        s1 = kvb + (size_t)(uint32_t)r1 * ROWB + pofs1;
    };
    v4f o[MTW];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) o[mt] = v4f{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY, l_lane = 0.f;

    {
        const unsigned char *s0, *s1;
        copy_src(0, s0, s1);
        fill_octets<0>(s0, s1, (lds_u8 *)bufE + pair * SLOT, 2 * half);
    }

    auto step = [&](auto even, int s) {
        constexpr bool E = decltype(even)::value;
        lds_u8 *cur = (lds_u8 *)(E ? bufE : bufO);
        lds_u8 *nxt = (lds_u8 *)(E ? bufO : bufE);
        __builtin_amdgcn_s_waitcnt(0);   // own copy of this tile
        __syncthreads();                 // all copies of this tile landed; the other slot is free
        // the copy of the next tile is issued one load per logit k-step, so the
        // wavefront never stalls on a full memory queue for long
        const bool has_next = s + 1 < steps;
        const unsigned char *cs0 = nullptr, *cs1 = nullptr;
        if (has_next) copy_src(s + 1, cs0, cs1);
        lds_u8 *cslot = nxt + pair * SLOT;
        const v4i mr = *reinterpret_cast<const v4i *>(tidx + RT * (2 * s + pair) + 16 * half + 4 * g);

        // S^T for own rows: lane holds rows 16*half + 4g + j of head n
        v4f sacc;
        {
            // two accumulation chains (even / odd k-steps); reads run PF steps ahead
            constexpr int PF = 4;
            v4f sa[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            v4i kf[PF];
#pragma unroll
            for (int c = 0; c < PF; ++c) kf[c] = lds_read_b128(cur + ((c & 1) ? kb_odd : kb_even) + OCT_BYTES * (c >> 1));
#pragma unroll
            for (int c = 0; c < KC; ++c) {
                const v4i cf = kf[c % PF];
                if (c + PF < KC)
                    kf[c % PF] = lds_read_b128(cur + (((c + PF) & 1) ? kb_odd : kb_even) + OCT_BYTES * ((c + PF) >> 1));
                if (has_next) {   // load (octet c/2, row group c&1) of the next tile
                    const int q = c >> 1, hl = c & 1;
                    __builtin_amdgcn_global_load_lds((hl ? cs1 : cs0) + 128 * q,
                                                     (__attribute__((address_space(3))) void *)(cslot + OCT_BYTES * q + 1024 * (2 * half + hl)),
                                                     16, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                sa[c & 1] = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, cf), __builtin_bit_cast(v8bf, qf[c]), sa[c & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
            sacc = sa[0] + sa[1];
        }
        // first V reads overlap the softmax
        constexpr int PG = 4;
        v4s vlo[2][PG], vhi[2][PG];
#pragma unroll
        for (int u = 0; u < PG; ++u) {
            vlo[0][u] = lds_read_tr16(cur + vbase[0][u]);
            vhi[0][u] = lds_read_tr16(cur + vbase[1][u]);
        }
        float z[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) z[j] = (mr[j] >= 0 && mr[j] < a.Lk) ? sacc[j] * sl2 : -INFINITY;
        const float lm = group_max4(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) p[j] = z[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[j] - m_ref);
        uint16_t *pt = reinterpret_cast<uint16_t *>(ptile[pair]) + ((n * 4 + g) * 2 + half) * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) pt[j] = __builtin_bit_cast(uint16_t, (__bf16)p[j]);
        if (g == 0) xmax[pair][half][n] = lm;
        const bool need = ballot(lm > m_ref + kSlack) != 0;
        if (lane == 0) raise_flag[wave] = need ? 1 : 0;
        __syncthreads();
        if (raise_flag[0] | raise_flag[1] | raise_flag[2] | raise_flag[3]) {
            // rare: some head's logits exceed its reference by more than kSlack
            const float tmax = fmaxf(xmax[pair][0][n], xmax[pair][1][n]);
            if (tmax > m_ref + kSlack) {
                const float alpha = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - tmax);
                m_ref = tmax;
                l_lane *= alpha;
#pragma unroll
                for (int mt = 0; mt < MTW; ++mt) o[mt] *= alpha;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                p[j] = z[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[j] - m_ref);
                pt[j] = __builtin_bit_cast(uint16_t, (__bf16)p[j]);
            }
            __syncthreads();   // the probability tile is read only after this point
        }
        l_lane += (p[0] + p[1]) + (p[2] + p[3]);

        // O^T (dv x heads) += V^T P^T over the 32 rows of the tile
        const v8bf pb = __builtin_bit_cast(v8bf, lds_read_b128((lds_u8 *)ptile[pair] + (n * 4 + g) * 16));
#pragma unroll
        for (int grp = 0; grp < MTW / PG; ++grp) {
            const int cb = grp & 1;
            if (grp + 1 < MTW / PG) {
#pragma unroll
                for (int u = 0; u < PG; ++u) {
                    const int mt = PG * (grp + 1) + u;
                    vlo[cb ^ 1][u] = lds_read_tr16(cur + vbase[0][mt & 3] + OCT_BYTES * (mt >> 2));
                    vhi[cb ^ 1][u] = lds_read_tr16(cur + vbase[1][mt & 3] + OCT_BYTES * (mt >> 2));
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < PG; ++u) {
                const int mt = PG * grp + u;
                const v8bf va = __builtin_bit_cast(v8bf, __builtin_shufflevector(vlo[cb][u], vhi[cb][u], 0, 1, 2, 3, 4, 5, 6, 7));
                o[mt] = mfma_bf16_16x16x32(va, pb, o[mt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    for (int s = 0; s < steps; s += 2) {
        step(std::integral_constant<bool, true>{}, s);
        if (s + 1 < steps) step(std::integral_constant<bool, false>{}, s + 1);
    }

    // merge: pair sums, then the two pairs' references
    __syncthreads();
    const float l_own = group_sum4(l_lane);
    if (g == 0) { mstat[wave][n] = m_ref; lstat[wave][n] = l_own; }
    __syncthreads();
    const float M = fmaxf(mstat[0][n], mstat[2][n]);
    const float scale = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - M);
    float *mb = reinterpret_cast<float *>(bufE) + pair * 16 * OPITCH;
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
        *reinterpret_cast<v4f *>(mb + n * OPITCH + 256 * half + 16 * mt + 4 * g) = o[mt] * scale;
    __syncthreads();
    {
        const int hh = tid >> 4, d0 = (tid & 15) * 32;
        const float m0 = mstat[0][hh], m1 = mstat[2][hh];
        const float Mh = fmaxf(m0, m1);
        float L = 0.f;
        if (m0 != -INFINITY) L += (lstat[0][hh] + lstat[1][hh]) * __builtin_amdgcn_exp2f(m0 - Mh);
        if (m1 != -INFINITY) L += (lstat[2][hh] + lstat[3][hh]) * __builtin_amdgcn_exp2f(m1 - Mh);
        const float inv = L > 0.f ? 1.f / L : 0.f;
        const float *s0 = reinterpret_cast<const float *>(bufE) + hh * OPITCH + d0;
        const float *s1 = s0 + 16 * OPITCH;
        uint16_t *dst = reinterpret_cast<uint16_t *>(a.out) + ((size_t)qrow * a.Hq + h0 + hh) * DV + d0;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            v4i packed;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const int c0 = 8 * v + 2 * e2;
                const float x0 = (s0[c0] + s1[c0]) * inv, x1 = (s0[c0 + 1] + s1[c0 + 1]) * inv;
                packed[e2] = (int)f32_to_bf16_rne(x0) | ((int)f32_to_bf16_rne(x1) << 16);
            }
            *reinterpret_cast<v4i *>(dst + 8 * v) = packed;
        }
        if (a.lse && (tid & 15) == 0)
            a.lse[(size_t)qrow * a.Hq + h0 + hh] = L > 0.f ? (Mh + log2f(L)) * 0.6931471805599453f : -INFINITY;
    }
}
}  // namespace latent

}  // namespace

hipError_t launch_sparse_mla(const MlaArgs &a, hipStream_t st) {
    const dim3 grid((unsigned)(a.B * a.Lq), (unsigned)((a.Hq + HG - 1) / HG));
    if (a.Dqk == latent::DQK && a.Dv == latent::DV && a.Hq % 16 == 0) {
        const void *fn = reinterpret_cast<const void *>(latent::sparse_mla_latent_kernel);
        (void)fn;
        const unsigned nwg = (unsigned)(a.B * a.Lq * (a.Hq / 16));
        hipLaunchKernelGGL(latent::sparse_mla_latent_kernel, dim3(nwg), dim3(latent::WAVES * kWave), 0, st, a);
    } else if (a.Dqk == 32 && a.Dv == 32) {
        hipLaunchKernelGGL((sparse_mla_kernel<32, 32>), grid, dim3(kWavesMla * kWave), 0, st, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace idxc
