// sparse_mla_wide.hip -- sparse MLA attention with 64 heads of a query per
// workgroup.
//
// itoverdose.com, "IndexCache: Wie DeepSeek O(NL²)-Kosten in Sparse Attention
// um 75% reduziert": the introduction (attention runs only over the k selected
// tokens) and section "Wie der Indexer funktioniert und warum MLA entscheidend
// ist" (every head reads one compressed latent row per token).  In the absorbed
// form all heads share the row: keys are the whole row (576 columns), values
// its first 512 columns.
//
// Each gathered row is used by 64 heads at once, so the rows of a query move
// from L2 into compute units Hq/64 times instead of once per 16-head group.
// When there are too few queries to fill the chip (decode), each query's
// index set is split into chunks that run as separate workgroups, and a second
// kernel merges their normalised partial outputs by log-sum-exp weights.
//
// Workgroup: one query, 64 heads, one chunk of the index set; 8 wavefronts
// in two roles that run one tile apart, one of each role per SIMD:
//  * Rows are consumed in tiles of 32.  Tiles are copied straight from HBM
//    into a ring of four LDS slots with LDS-direct 16-byte loads, two tiles
//    ahead; the index values that drive the copies are themselves copied
//    into a small LDS ring four tiles ahead.  The consumers copy.
//  * Producers (wavefronts 0-3; heads 16p..16p+15): S = K Q^T for the 32 rows
//    of tile s on 16x16x32 bf16 MFMA, query fragments held in AGPRs for the
//    whole sweep; the softmax probabilities go to LDS in bf16.  Each head's
//    reference is raised lazily, only when a tile's maximum exceeds it by more
//    than kSlack (log2 units), and the producer publishes the rescale factor
//    with the probabilities.
//  * Consumers (wavefronts 4-7; output columns 128c..128c+127 of all 64
//    heads): O^T += V^T P^T for tile s-1, V^T read with transposing LDS
//    loads; a published rescale is applied before the tile it belongs to.
//  * One workgroup barrier per tile.  The two roles are separate code paths,
//    so the query fragments (producers) and the output accumulators
//    (consumers) never need registers in the same wavefront; both sit in the
//    AGPR file, which VGPRs and AGPRs being budgeted per kernel requires.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace idxc {
namespace {
namespace wide {

constexpr int DQK = 576, DV = 512;
constexpr int HW = 64;                        // heads per workgroup
constexpr int RT = 32;                        // rows per tile
constexpr int ROWB = DQK * 2;                 // bytes per latent row
constexpr int OCTETS = ROWB / 128;            // 128-byte lines per row
constexpr int OCT_BYTES = RT * 128;           // one line of every row of a tile
constexpr int SLOT = OCTETS * OCT_BYTES;      // bytes per tile
constexpr int WAVES = 8;                      // 4 producers, 4 consumers
constexpr int KS = DQK / 32;                  // logit k-steps (16x16x32 MFMA)
constexpr int RING = 8;                       // index ring, in tiles
constexpr int PB = HW * RT * 2;               // probability tile, bf16 [head][row]
constexpr float kSlack = 8.f;
static_assert(ROWB % 128 == 0, "rows are whole 128-byte lines");
static_assert(RT == 8 * 4, "each consumer copies one 8-row group");
static_assert(HW == 64 && DV == 512 && RT == 32, "four producers of 16 heads, four consumers of 128 columns");

// Slot layout: line-major [line q][row r][position], where 16-byte piece
// 8q + p of row r sits at position (p + f(r)) mod 8, f(r) = 4 r1 + 2 r2
// (r_i: bit i of r).  LDS has 64 four-byte banks; a 16-byte read serves 16
// lanes per cycle, the lanes l with one value of (l5, l2 ^ l3 ^ l4), and an
// 8-byte read serves 32 consecutive lanes.  For the logit operand (lane
// (n, g) reads row n of a 16-row block, piece g + const) each such lane set
// takes rows n and pieces g whose (n0, position) pairs are all distinct, and
// so do the transposed V reads (4 consecutive rows x 4 aligned pieces per
// 16 lanes): no read waits on a bank conflict.
__device__ __forceinline__ int rot(int r) { return 4 * ((r >> 1) & 1) + 2 * ((r >> 2) & 1); }
__device__ __forceinline__ int pos_of(int p, int r) { return (p + rot(r)) & 7; }
__device__ __forceinline__ int piece_at(int pos, int r) { return (pos - rot(r)) & 7; }

typedef short v4s __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

__device__ __forceinline__ v4s lds_read_tr16(const lds_u8 *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)p);
}
__device__ __forceinline__ v4i lds_read_b128(const lds_u8 *p) { return *(const __attribute__((address_space(3))) v4i *)p; }
__device__ __forceinline__ void lds_write_b64(lds_u8 *p, v2i v) { *(__attribute__((address_space(3))) v2i *)p = v; }

// D(32x32, fp32) = A(32x16, bf16) * B(16x32, bf16) + C.  Lane l supplies
// row/column l%32 and k-values 8*(l/32)..+7; register r of the result holds
// D[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ v16f mfma_bf16_32x32x16(const v8bf &a, const v8bf &b, const v16f &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// One 8-row group rg of a tile: load Q moves line Q of the group's rows
// (lane l: row 8rg + l/8, position l%8).  The immediate offset 128Q applies
// to the global and to the LDS address, so the LDS base is lowered by it.
template <int Q>
__device__ __forceinline__ void fill_group(const unsigned char *src, lds_u8 *slot, int rg) {
    if constexpr (Q < OCTETS) {
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(slot + (OCT_BYTES - 128) * Q + 1024 * rg),
                                         16, 128 * Q, 0);
        fill_group<Q + 1>(src, slot, rg);
    }
}

// v_max_f32 as is: fmaxf would first quieten both operands (two more
// instructions per use), and no NaN reaches these maxima
__device__ __forceinline__ float max_f32(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float swap32_max(float v) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return max_f32(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
// maxima and sums over lanes l and l^16 (the 16-lane rows swapped pairwise)
__device__ __forceinline__ float swap16_max(float v) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return max_f32(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float swap16_sum(float v) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}
__device__ __forceinline__ float swap32_sum(float v) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
// two floats rounded to bf16 (nearest even) in one packed conversion, lo in bits 0-15
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){lo, hi}, v2bf));
}

// Keeps a per-step copy of an LDS offset opaque, so that the compiler adds
// the slot base inside the step instead of holding base + offset for every
// slot in registers across the loop.
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

// Keeps an accumulator block in accumulation registers at this point (an
// empty asm with an AGPR operand): the output accumulators fill the AGPR
// file, and this stops the compiler from holding whole sets of them in
// VGPRs around the rare rescale and the final read-out.
__device__ __forceinline__ void pin_acc(v16f &x) { asm volatile("" : "+a"(x)); }

struct Smem {
    unsigned char ptile[2][PB];               // [tile parity] bf16 [head][4 chunks of 8 rows]
    int ring[RING][RT];                       // index values of tiles t % RING
    float alpha[2][HW];                       // [tile parity] rescale factor per head
    int flag[2][4];                           // [tile parity][producer] some head was rescaled
    float lsum[HW], mref[HW];
};

__global__ __launch_bounds__(WAVES * kWave) void sparse_mla_wide_kernel(MlaWideArgs a) {
    __shared__ __align__(16) unsigned char slot0[SLOT];
    __shared__ __align__(16) unsigned char slot1[SLOT];
    __shared__ __align__(16) unsigned char slot2[SLOT];
    __shared__ __align__(16) unsigned char slot3[SLOT];
    __shared__ __align__(16) Smem sm;

    // workgroup -> (query, head block, chunk); the chunks and head blocks of
    // one query, and runs of neighbouring queries, share an XCD and its L2
    const int total = (int)gridDim.x;
    int id = (int)blockIdx.x;
    if (total % 8 == 0) id = (id % 8) * (total / 8) + id / 8;
    const int chunk = id % a.nchunk;
    const int qb = id / a.nchunk;                 // query * head blocks + head block
    const int nhb = a.Hq / HW;
    const int qrow = qb / nhb, h0 = (qb % nhb) * HW;
    const int b = qrow / a.Lq;
    const int cs = chunk * a.chunk_rows;          // first position of the chunk
    const int clen = min(a.chunk_rows, a.topk - cs);
    const int ntiles = (clen + RT - 1) / RT;

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int n = lane & 31, hh = lane >> 5;
    const unsigned char *kvb = static_cast<const unsigned char *>(a.kv) + (size_t)b * a.Lk * ROWB;
    const int32_t *trow = a.t + (size_t)qrow * a.topk;
    auto SL = [&](auto I) -> lds_u8 * {
        constexpr int i = decltype(I)::value & 3;
        if constexpr (i == 0) return (lds_u8 *)slot0;
        else if constexpr (i == 1) return (lds_u8 *)slot1;
        else if constexpr (i == 2) return (lds_u8 *)slot2;
        else return (lds_u8 *)slot3;
    };

    // index ring: tiles 0..3 now, tile s+4 at the end of step s
    if (tid < 4 * RT) sm.ring[tid / RT][tid % RT] = trow[min(cs + tid, a.topk - 1)];
    lds_barrier();

    // Copies are issued by the consumer wavefronts only (consumer c copies
    // row group c of every tile), so that the producers, which set the pace,
    // spend no issue slots on them.  Lane l of a group copy moves position
    // l%8 of row 8rg + l/8.
    auto copy_group = [&](lds_u8 *slot, int t, int ix, int rg) {
        const int row = 8 * rg + (lane >> 3);
        const bool ok = RT * t + row < clen && ix >= 0 && ix < a.Lk;
        fill_group<0>(kvb + (size_t)(uint32_t)(ok ? ix : 0) * ROWB + 16 * piece_at(lane & 7, row), slot, rg);
    };
    // steps 0..ntiles in groups of four (slot parity is a template argument;
    // no conditional step inside the loop keeps the compiler's tracking of
    // the copies exact), the remainder after the loop
    auto run = [&](auto &&step) {
        int s = 0;
        for (; s + 3 <= ntiles; s += 4) {
            step(std::integral_constant<int, 0>{}, s);
            step(std::integral_constant<int, 1>{}, s + 1);
            step(std::integral_constant<int, 2>{}, s + 2);
            step(std::integral_constant<int, 3>{}, s + 3);
        }
        if (s <= ntiles) step(std::integral_constant<int, 0>{}, s);
        if (s + 1 <= ntiles) step(std::integral_constant<int, 1>{}, s + 1);
        if (s + 2 <= ntiles) step(std::integral_constant<int, 2>{}, s + 2);
    };

    if (wave < 4) {
        // ---------------- producer: heads 16p..16p+15, all rows of each tile
        const int p = wave;
        const int n16 = lane & 15, g = lane >> 4;
        const int H = 16 * p + n16;               // head (within the block) of this lane
        const float sl2 = a.sm_scale * 1.4426950408889634f;
        v4i qf[KS];                               // B operand: head H, d = 32ks + 8g..+7
        {
            const unsigned char *qh = static_cast<const unsigned char *>(a.q) + ((size_t)qrow * a.Hq + h0 + H) * ROWB;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const v4i *>(qh + 64 * ks + 16 * g);
            // the query fragments live in AGPRs (MFMA operands may come from
            // either file): VGPRs and AGPRs are allocated per kernel, and the
            // consumers' output accumulators fill the AGPR budget anyway
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+a"(qf[ks]));
        }
        // A operand of k-step ks, row block rb: row 16rb + n16 of the tile,
        // 16-byte piece 4ks + g = line ks/2, piece 4(ks%2) + g
        int kb[2][2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int k = 0; k < 2; ++k) kb[rb][k] = 128 * (16 * rb + n16) + 16 * pos_of(4 * k + g, 16 * rb + n16);
        float m_ref = -INFINITY, l_lane = 0.f;
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // query fragments
        lds_barrier();   // tile 0 landed (consumers' copies)
        int ix_mask = sm.ring[0][n];
        auto step = [&](auto PI_, int s) {
            constexpr int PI = decltype(PI_)::value;
            lds_u8 *cur = SL(std::integral_constant<int, PI>{});
            const int par = s & 1;
            const int ix_mask_next = sm.ring[(s + 1) & (RING - 1)][n];
            if (s < ntiles) {
                int kbs[2][2];
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int k = 0; k < 2; ++k) kbs[rb][k] = opaque(kb[rb][k]);
                // software pipeline over pairs of k-steps: the reads of pairs
                // q+1 and q+2 are in flight while pair q runs on the MFMA unit
                // (one pair of MFMAs does not cover the LDS latency when the
                // four producers read at once)
                v4f acc[2];
                acc[0] = v4f{0.f, 0.f, 0.f, 0.f};
                acc[1] = acc[0];
                v4i kf[3][2][2];   // [buffer][k-step of the pair][row block]
                auto read_pair = [&](int q, v4i (&dst)[2][2]) {
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const int ks = 2 * q + i;
#pragma unroll
                        for (int rb = 0; rb < 2; ++rb) dst[i][rb] = lds_read_b128(cur + kbs[rb][ks & 1] + OCT_BYTES * (ks >> 1));
                    }
                };
                read_pair(0, kf[0]);
                read_pair(1, kf[1]);
#pragma unroll
                for (int q = 0; q < KS / 2; ++q) {
                    if (q + 2 < KS / 2) read_pair(q + 2, kf[(q + 2) % 3]);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int rb = 0; rb < 2; ++rb)
                            acc[rb] = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, kf[q % 3][i][rb]),
                                                         __builtin_bit_cast(v8bf, qf[2 * q + i]), acc[rb]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                // rows of this lane: 16rb + 4g + i for register i of block rb;
                // logits stay unscaled (z * sl2 is formed inside the exponent)
                const bool vrow = (RT * s + n < clen) & (ix_mask >= 0) & (ix_mask < a.Lk);
                const uint32_t vball = (uint32_t)ballot(vrow && hh == 0);   // bit r: row r
                const bool all_valid = vball == 0xFFFFFFFFu;
                if (!all_valid) {
                    // a partial tile (the set's tail, or entries outside the
                    // cache); the empty asm keeps this a branch, so full tiles
                    // run no per-element selects
                    asm volatile("" ::: "memory");
                    const uint32_t bits = vball >> (4 * g);   // bit 16rb + i: row 16rb + 4g + i
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (!((bits >> (16 * rb + i)) & 1u)) acc[rb][i] = -INFINITY;
                }
                float lm = -INFINITY;
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) lm = fmaxf(lm, acc[rb][i]);
                lm = swap32_max(swap16_max(lm)) * sl2;   // sl2 > 0: the maximum of the scaled logits
                const float m_new = lm > m_ref + kSlack ? lm : m_ref;
                const float alpha = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
                // every lane stores: the four lanes of a head hold the same
                // alpha, and the flag is uniform (no exec-mask changes)
                sm.alpha[par][H] = alpha;
                const bool raised = ballot(m_new != m_ref) != 0;
                sm.flag[par][p] = raised ? 1 : 0;
                // exp2(-inf) = 0 takes care of masked rows whenever m_new is
                // finite; m_new = -inf means no valid row so far (all zero)
                const float mneg = m_new == -INFINITY ? 0.f : -m_new;
                lds_u8 *ptp = (lds_u8 *)sm.ptile[par];
                float ps = 0.f;
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    float pv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[rb][i], sl2, mneg));
                        ps = rb == 0 && i == 0 ? pv[i] : ps + pv[i];   // (0 + p = p: p >= 0)
                    }
                    // rows 16rb + 4g..+3: half g%2 of chunk q = 2rb + g/2, chunk q
                    // of head H stored at 16((q + H/4) mod 4)
                    v2i w2;
                    w2[0] = (int)pack_bf16(pv[0], pv[1]);
                    w2[1] = (int)pack_bf16(pv[2], pv[3]);
                    const int q = 2 * rb + (g >> 1);
                    lds_write_b64(ptp + 64 * H + 16 * ((q + (H >> 2)) & 3) + 8 * (g & 1), w2);
                }
                l_lane = l_lane * alpha + ps;
                m_ref = m_new;
            }
            lds_barrier();   // P of tile s visible; tile s+1 landed (consumers' copies)
            ix_mask = ix_mask_next;
        };
        run(step);
        const float l_head = swap32_sum(swap16_sum(l_lane));
        if (g == 0) {
            sm.lsum[H] = l_head;
            sm.mref[H] = m_ref;
        }
        lds_barrier();   // statistics visible
        lds_barrier();   // consumers staged the output
    } else {
        // ---------------- consumer: output columns 128c..128c+127 of all 64 heads
        const int c = wave - 4;
        // transposed V reads: lane (G = lane/16, j = (lane/4)%4, cc = lane%4) ->
        // row 8(G/2) + 4t + j, columns 128c + 32mb + 16(G%2) + 4cc..+3 = line
        // 2c + mb/2, piece 4(mb%2) + 2(G%2) + cc/2, byte 8(cc%2)
        int vb[2][2];
        {
            const int G = lane >> 4, j = (lane >> 2) & 3, cc = lane & 3;
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int r = 8 * (G >> 1) + 4 * t + j;
                    vb[m2][t] = OCT_BYTES * 2 * c + 128 * r + 16 * pos_of(4 * m2 + 2 * (G & 1) + (cc >> 1), r) + 8 * (cc & 1);
                }
        }
        // B operand of k-step cp: head 32nb + n, rows 16cp + 8hh..+7 = chunk
        // q = 2cp + hh, stored at 16((q + H/4) mod 4)
        int pbase[2];
#pragma unroll
        for (int cp = 0; cp < 2; ++cp) pbase[cp] = 64 * n + 16 * ((2 * cp + hh + (n >> 2)) & 3);
        v16f o[4][2];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) o[mb][nb] = v16f{};
        // index values of tile t for rows 8c..8c+7 (lane l holds row 8c + l%8),
        // loaded by every lane so that each step issues the same number of
        // vector-memory operations whatever the lane mask
        auto load_index = [&](int t) -> int { return trow[min(cs + RT * t + 8 * c + (lane & 7), a.topk - 1)]; };
        const int crow = 8 * c + (lane >> 3);   // copy row of group c
        // index loads by step parity (moving a register whose load is in
        // flight would wait for it)
        int pendb[2] = {0, load_index(4)};
        copy_group(SL(std::integral_constant<int, 0>{}), 0, sm.ring[0][crow], c);
        copy_group(SL(std::integral_constant<int, 1>{}), 1, sm.ring[1][crow], c);
        int ix = sm.ring[2][crow];
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(OCTETS));   // the index load and tile 0 landed
        lds_barrier();
        // step s starts with the load of the indices of tile s+5 and the copy
        // of tile s+2 (10 vector-memory operations); it ends by waiting for
        // tile s+1 and the indices of tile s+4, which then go to the ring.  The
        // products of tile s-1 run after barrier A, while the producers work
        // on the softmax of tile s.
        auto step = [&](auto PI_, int s) {
            constexpr int PI = decltype(PI_)::value;
            lds_u8 *prv = SL(std::integral_constant<int, PI + 3>{});
            lds_u8 *nx2 = SL(std::integral_constant<int, PI + 2>{});   // held tile s-2, consumed before the last barrier
            pendb[PI & 1] = load_index(s + 5);
            copy_group(nx2, s + 2, ix, c);
            const int ix_next = sm.ring[(s + 3) & (RING - 1)][crow];
            const int par = (s - 1) & 1;
            if (s >= 1 && (sm.flag[par][0] | sm.flag[par][1] | sm.flag[par][2] | sm.flag[par][3])) {
                // a reference of tile s-1 was raised: rescale tiles 0..s-2
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const float al = sm.alpha[par][32 * nb + n];
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb) {
                        pin_acc(o[mb][nb]);
                        o[mb][nb] *= al;
                        pin_acc(o[mb][nb]);
                    }
                }
            }
            if (s >= 1) {
                int vbs[2][2], pbs[2];
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                    for (int t = 0; t < 2; ++t) vbs[m2][t] = opaque(vb[m2][t]);
#pragma unroll
                for (int cp = 0; cp < 2; ++cp) pbs[cp] = opaque(pbase[cp]);
                // two batches, one per k-step of 16 rows: all V^T and P^T
                // operands of a batch are read at once; the second batch's
                // reads complete under the first batch's MFMAs
                auto read_batch = [&](int cp, v8bf (&va)[4], v8bf (&pb)[2]) {
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb)
                        pb[nb] = __builtin_bit_cast(v8bf, lds_read_b128((lds_u8 *)sm.ptile[par] + pbs[cp] + 2048 * nb));
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb) {
                        const v4s lo = lds_read_tr16(prv + vbs[mb & 1][0] + OCT_BYTES * (mb >> 1) + 2048 * cp);
                        const v4s hi = lds_read_tr16(prv + vbs[mb & 1][1] + OCT_BYTES * (mb >> 1) + 2048 * cp);
                        va[mb] = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    }
                };
                v8bf va0[4], va1[4], pb0[2], pb1[2];
                read_batch(0, va0, pb0);
                __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): batch 0 landed
                __builtin_amdgcn_sched_barrier(0);
                read_batch(1, va1, pb1);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb) o[mb][nb] = mfma_bf16_32x32x16(va0[mb], pb0[nb], o[mb][nb]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb) o[mb][nb] = mfma_bf16_32x32x16(va1[mb], pb1[nb], o[mb][nb]);
            }
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(OCTETS + 1));
            const int pend = pendb[(PI & 1) ^ 1];   // indices of tile s+4 (landed)
            if (lane < 8) sm.ring[(s + 4) & (RING - 1)][8 * c + lane] = pend;
            lds_barrier();
            ix = ix_next;
        };
        run(step);
        // the copies past the last tile may still be in flight: let them
        // land before the slots are reused and the LDS is released
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        lds_barrier();   // producers' statistics visible
        // normalised output in bf16, staged through the free slots as
        // [head][512 columns] (head H in slot H/32, 16-byte unit u of its row
        // at u ^ (H % 32)), then written with whole-row stores
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const float L = sm.lsum[32 * nb + n];
            const float inv = L > 0.f ? 1.f / L : 0.f;
            lds_u8 *stg = nb == 0 ? (lds_u8 *)slot0 : (lds_u8 *)slot1;
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                pin_acc(o[mb][nb]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int col = 128 * c + 32 * mb + 8 * i + 4 * hh;   // 4 columns, 8 bytes
                    v2i w2;
                    w2[0] = (int)pack_bf16(o[mb][nb][4 * i] * inv, o[mb][nb][4 * i + 1] * inv);
                    w2[1] = (int)pack_bf16(o[mb][nb][4 * i + 2] * inv, o[mb][nb][4 * i + 3] * inv);
                    lds_write_b64(stg + 1024 * n + 16 * ((col >> 3) ^ n) + 8 * ((col >> 2) & 1), w2);
                }
            }
        }
        lds_barrier();   // output staged
    }

    unsigned char *dst;
    if (a.nchunk == 1)
        dst = static_cast<unsigned char *>(a.out) + ((size_t)qrow * a.Hq + h0) * DV * 2;
    else
        dst = static_cast<unsigned char *>(a.part_o) + (((size_t)qrow * a.nchunk + chunk) * a.Hq + h0) * DV * 2;
    {
        const int u = tid & 63;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            lds_u8 *stg = nb == 0 ? (lds_u8 *)slot0 : (lds_u8 *)slot1;
#pragma unroll
            for (int k = 0; k < 32 / WAVES; ++k) {
                const int hl = (tid >> 6) + WAVES * k;   // head 32nb + hl
                const v4i v = lds_read_b128(stg + 1024 * hl + 16 * (u ^ hl));
                *reinterpret_cast<v4i *>(dst + (size_t)(32 * nb + hl) * DV * 2 + 16 * u) = v;
            }
        }
    }
    if (tid < HW) {
        const float L = sm.lsum[tid];
        const float lse2 = L > 0.f ? sm.mref[tid] + __log2f(L) : -INFINITY;
        if (a.nchunk == 1) {
            if (a.lse) a.lse[(size_t)qrow * a.Hq + h0 + tid] = lse2 * 0.6931471805599453f;
        } else {
            a.part_lse[((size_t)qrow * a.nchunk + chunk) * a.Hq + h0 + tid] = lse2;
        }
    }
}

// Merge of the chunk partials of one (query, head) per wavefront: weights
// 2^(lse_c - max), output = weighted mean of the normalised partials.
__global__ __launch_bounds__(256) void sparse_mla_merge_kernel(MlaWideArgs a) {
    const int w = (int)(blockIdx.x * 4 + threadIdx.x / kWave), lane = threadIdx.x % kWave;
    if (w >= a.B * a.Lq * a.Hq) return;
    const int qrow = w / a.Hq, h = w % a.Hq;
    const float *pl = a.part_lse + (size_t)qrow * a.nchunk * a.Hq + h;
    const unsigned char *po = static_cast<const unsigned char *>(a.part_o) + ((size_t)qrow * a.nchunk * a.Hq + h) * DV * 2 +
                              16 * lane;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    auto add = [&](float wc, const v4i &v) {
        wsum += wc;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            acc[2 * k] += wc * __uint_as_float((uint32_t)v[k] << 16);
            acc[2 * k + 1] += wc * __uint_as_float((uint32_t)v[k] & 0xFFFF0000u);
        }
    };
    float mx = -INFINITY;
    constexpr int kMaxChunks = 8;
    if (a.nchunk <= kMaxChunks) {
        // every chunk's statistics and partial row are loaded before any is used
        float lc[kMaxChunks];
        v4i v[kMaxChunks];
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) {
            lc[c] = c < a.nchunk ? pl[(size_t)c * a.Hq] : -INFINITY;
            v[c] = c < a.nchunk ? *reinterpret_cast<const v4i *>(po + (size_t)c * a.Hq * DV * 2) : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) mx = fmaxf(mx, lc[c]);
        if (mx != -INFINITY) {
#pragma unroll
            for (int c = 0; c < kMaxChunks; ++c)
                if (lc[c] != -INFINITY) add(__builtin_amdgcn_exp2f(lc[c] - mx), v[c]);
        }
    } else {
        for (int c = 0; c < a.nchunk; ++c) mx = fmaxf(mx, pl[(size_t)c * a.Hq]);
        if (mx != -INFINITY) {
            for (int c = 0; c < a.nchunk; ++c) {
                const float lc = pl[(size_t)c * a.Hq];
                if (lc == -INFINITY) continue;
                add(__builtin_amdgcn_exp2f(lc - mx), *reinterpret_cast<const v4i *>(po + (size_t)c * a.Hq * DV * 2));
            }
        }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    v4i o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = (int)pack_bf16(acc[2 * k] * inv, acc[2 * k + 1] * inv);
    *reinterpret_cast<v4i *>(static_cast<unsigned char *>(a.out) + ((size_t)qrow * a.Hq + h) * DV * 2 + 16 * lane) = o;
    if (a.lse && lane == 0)
        a.lse[(size_t)qrow * a.Hq + h] = wsum > 0.f ? (mx + __log2f(wsum)) * 0.6931471805599453f : -INFINITY;
}

}  // namespace wide
}  // namespace

MlaWidePlan mla_wide_plan(int B, int Lq, int Hq, int Dqk, int Dv, int topk) {
    MlaWidePlan p{};
    if (Dqk != wide::DQK || Dv != wide::DV || Hq % wide::HW != 0 || topk < 1) return p;
    const long long nq = (long long)B * Lq * (Hq / wide::HW);
    const int ntiles = (topk + wide::RT - 1) / wide::RT;
    // enough workgroups for the 256 compute units, at least 4 tiles each
    long long want = nq >= kMlaTargetWorkgroups ? 1 : (kMlaTargetWorkgroups + nq - 1) / nq;
    want = std::min<long long>(want, std::max(1, ntiles / 4));
    const int tiles_per = (int)((ntiles + want - 1) / want);
    p.chunk_rows = tiles_per * wide::RT;
    p.nchunk = (topk + p.chunk_rows - 1) / p.chunk_rows;
    p.ws_bytes = p.nchunk > 1 ? (size_t)B * Lq * Hq * p.nchunk * (wide::DV * 2 + 4) : 0;
    p.ok = true;
    return p;
}

hipError_t launch_sparse_mla_wide(const MlaWideArgs &a, hipStream_t st) {
    const unsigned nwg = (unsigned)((size_t)a.B * a.Lq * (a.Hq / wide::HW) * a.nchunk);
    hipLaunchKernelGGL(wide::sparse_mla_wide_kernel, dim3(nwg), dim3(wide::WAVES * kWave), 0, st, a);
    if (a.nchunk > 1) {
        const unsigned nm = (unsigned)(((size_t)a.B * a.Lq * a.Hq + 3) / 4);
        hipLaunchKernelGGL(wide::sparse_mla_merge_kernel, dim3(nm), dim3(256), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace idxc
