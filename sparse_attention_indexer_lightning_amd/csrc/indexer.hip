// indexer.hip -- lightning indexer scores on MFMA with the per-row top-k fused in.
//
// Score (itoverdose.com, "IndexCache: Wie DeepSeek O(NL²)-Kosten in Sparse
// Attention um 75% reduziert", section "Wie der Indexer funktioniert und warum
// MLA entscheidend ist"; parapluman.nl, section "Het DSA-knelpunt"):
//     I[t,s] = sum_h w[t,h] * max(0, q[t,h,:] . k[s,:]),   s <= position(t)
// followed by the top-k of each row (same itoverdose.com page, section
// "Einfache Implementierung, enorme Effizienzgewinne").
//
// Prefill kernel (many queries per sequence).  One workgroup owns R
// consecutive query rows of one sequence and sweeps that sequence's keys in
// blocks of 64, staging each key block in LDS (double-buffered through
// registers).  Each wavefront holds its rows' queries as MFMA A-fragments
// (64 (row, head) pairs = four 16-row fragments) in registers for the whole
// sweep.  Per 16-key sub-block it issues four MFMAs (fp8 16x16x128, or bf16
// 16x16x32 per 32-wide slice of d); the MFMAs of sub-block j+1 are interleaved
// with the ReLU / head-weight epilogue of sub-block j.  The head sum finishes
// with a cross-lane transpose-reduce on v_permlane32_swap / v_permlane16_swap
// that leaves lane l holding the score of key (block + l).  Scores never
// reach HBM.
//
// Streaming top-k.  Each row owns an LDS candidate buffer of `cap` entries
// (order-preserving 32-bit score key + key index) and a threshold key; a key
// enters the buffer when its key is strictly above the threshold.  Appends go
// in ascending key order (ballot + prefix count), so the buffer stays sorted
// by index.  Two ways to shrink a full buffer:
//  * exact: MSB-first radix select (8-bit digits, LDS histogram) finds the
//    k-th largest key; a stable in-place filter keeps every entry above it
//    plus the lowest-index entries equal to it, and it becomes the threshold
//    (a later key equal to it has a larger index and can never win, so ">"
//    is exact);
//  * binned (one query row per wavefront): a 256-bin histogram of the
//    buffered keys, log-spaced above the buffer's smallest key (finest just
//    above it, where the cut falls when the buffer is full), gives the bin
//    holding the k-th largest key; the filter keeps every entry at or above
//    that bin's lower edge (at least k entries, all of them better than
//    anything dropped), which then bounds the threshold.  Exact selection is
//    the fallback when the cut's bin is too full.
// With one row per wavefront, compactions are batched at the block barrier:
// when any row must compact, every row past a quarter of its slack compacts
// too, so waves stall on each other's compactions far less often.  At the end the
// exact selection leaves min(k, p+1) entries, already in ascending order.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "select_common.h"

namespace idxc {
namespace {

constexpr int KB = 64;          // keys per block (one per lane after the reduce)
constexpr int kMaxThreads = 512;
// Wavefronts (query rows) of a workgroup of the pipelined 64-head fp8 sweep,
// and how many such workgroups share a compute unit (its LDS split evenly):
// 4 (two workgroups per compute unit) or 8 (one).  At L = 65536 the 4-wave
// layout takes 7 % fewer cycles on random inputs and 13 % fewer on inputs
// whose selection appends little.
#ifndef IDXC_PIPE_WAVES
#define IDXC_PIPE_WAVES 4
#endif
constexpr int kPipeWaves = IDXC_PIPE_WAVES;
constexpr int kPipeGroupsPerCU = 8 / kPipeWaves;
// Key tiles of the pipelined sweep: two (one barrier per block) with one
// workgroup per compute unit; one (two barriers per block) when two
// workgroups share the LDS, which leaves room for the candidate buffers.
constexpr int kPipeTiles = kPipeGroupsPerCU == 1 ? 2 : 1;
static_assert(kPipeWaves == 4 || kPipeWaves == 8, "the linear-term MFMA covers rows in groups of four");
constexpr int kChunkMax = 4;    // 16-byte chunks each thread stages per key block
constexpr int kPadEntries = 256; // candidate-buffer padding read by 4-per-lane passes
constexpr int kHistWords = 320;  // 256 bins + one dummy slot per lane for masked-off updates
// The pipelined sweep keeps 16-bit candidate indices also for keys beyond
// 65536: a row's candidates are in index order, so segment j of the keys
// (j * 65536 ..) starts at a buffer position recorded per row (kMaxSeg
// segments, keys up to kMaxSeg * 65536), and an index is its low 16 bits plus
// the segment of its position.
constexpr int kMaxSeg = 16;
// Fourth word of a raw buffer descriptor on gfx9-family parts (32-bit data
// format; no stride, no swizzle), as the loads of the pipelined sweep use it.
constexpr int kBufferWord3 = 0x00020000;
// Sampled starting threshold of the 64-head sweep: every kSampleStride-th key
// block is scored first; a row's threshold is then its sample's r-th largest
// key, r = ceil(7/4 * k * (sampled keys) / (keys)), unless r is below
// kSampleMinRank or above the sample.  Only workgroups with at least
// kSampleMinBlocks key blocks sample.
constexpr int kSampleStride = 32;
constexpr int kSampleMarginNum = 7, kSampleMarginDen = 4;   // 7/4
constexpr int kSampleMinRank = 32;
constexpr int kSampleMinBlocks = 64;

template <Enc E, int D>
struct Shape {
    static constexpr int EB = (E == Enc::FP8) ? 1 : 2;    // bytes per element
    static constexpr int ROWB = D * EB;                    // bytes per key row
    static constexpr int PITCH = ROWB + 16;                // LDS row pitch
    static constexpr int NV = (E == Enc::FP8) ? 2 : D / 32; // 16-byte pieces per lane
};

// One lane's share of a 16-row x D operand (A or B of the MFMA).
template <Enc E, int D>
struct Frag {
    v4i x[Shape<E, D>::NV];
};

// byte offset of piece v of lane group g inside one row
template <Enc E, int D>
__device__ __forceinline__ int piece_off(int v, int g) {
    if constexpr (E == Enc::FP8) return 32 * g + 16 * v;
    else return 64 * v + 16 * g;
}

template <Enc E, int D>
__device__ __forceinline__ void load_frag(Frag<E, D> &f, const unsigned char *row, int g) {
#pragma unroll
    for (int v = 0; v < Shape<E, D>::NV; ++v)
        f.x[v] = *reinterpret_cast<const v4i *>(row + piece_off<E, D>(v, g));
}

template <Enc E, int D>
__device__ __forceinline__ void zero_frag(Frag<E, D> &f) {
#pragma unroll
    for (int v = 0; v < Shape<E, D>::NV; ++v) f.x[v] = v4i{0, 0, 0, 0};
}

template <Enc E, int D>
__device__ __forceinline__ v4f frag_mma(const Frag<E, D> &a, const Frag<E, D> &b) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (E == Enc::FP8) {
        v8i av = __builtin_shufflevector(a.x[0], a.x[1], 0, 1, 2, 3, 4, 5, 6, 7);
        v8i bv = __builtin_shufflevector(b.x[0], b.x[1], 0, 1, 2, 3, 4, 5, 6, 7);
        acc = mfma_fp8_16x16x128(av, bv, acc);
    } else {
#pragma unroll
        for (int v = 0; v < Shape<E, D>::NV; ++v)
            acc = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, a.x[v]), __builtin_bit_cast(v8bf, b.x[v]), acc);
    }
    return acc;
}

// One 32-bit load whatever the encoding, chosen by selects rather than a
// branch, so that a run of weight loads stays in flight together (a branch
// per load ends each one with a full wait).  bf16: the word holding entry
// idx; rows hold an even number of heads, so the word lies inside the row.
__device__ __forceinline__ float load_w(const void *w, Enc enc, size_t idx) {
    const bool h16 = enc == Enc::BF16;
    const uint32_t word = reinterpret_cast<const uint32_t *>(w)[h16 ? idx >> 1 : idx];
    return __uint_as_float(!h16 ? word : (idx & 1) ? (word & 0xFFFF0000u) : (word << 16));
}

// Lane group g (lanes 16g..16g+15) holds partial sums p[j] of sub-block j for
// the same 16 keys as the other three groups; returns the full sum of
// sub-block g.  permlane32_swap(x, y) exchanges the upper half of x with the
// lower half of y, permlane16_swap(x, y) the odd 16-lane rows of x with the
// even rows of y; in both cases x' + y' is, per lane, the sum of the value it
// keeps and its partner's copy of the same sub-block.
__device__ __forceinline__ float transpose_reduce4(float p0, float p1, float p2, float p3) {
    const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p2), false, false);
    const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p1), __float_as_uint(p3), false, false);
    const float a = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);  // sub-block 0 (lanes 0-31) / 2
    const float b = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);  // sub-block 1 / 3
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// ReLU and head weights of one 16-key sub-block: the four fragments' rows are
// summed as four independent chains, then added in fragment order.  Both the
// fused and the split-key kernel use this, so they round identically.
__device__ __forceinline__ void subblock_epilogue(const v4f (&acc)[4], const float (&wv)[4][4], float (&pf)[4]) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        pf[f] = wv[f][0] * relu(acc[f][0]);
#pragma unroll
        for (int ii = 1; ii < 4; ++ii) pf[f] += wv[f][ii] * relu(acc[f][ii]);
    }
}

// ---- 64 heads x 64 keys on 32x32x64 fp8 MFMAs (one query per wavefront) ----
// A fragments: row fragment rf (heads 32rf..32rf+31) and d-step s (d 64s..64s+63);
// lane l holds head 32rf + l%32, d = 64s + 32(l/32) .. +31.
struct Q32 {
    v8i a[2][2];      // [rf][s]
    float w[2][16];   // head weight of accumulator register r of row fragment rf
};

__device__ __forceinline__ v8i load32(const unsigned char *p) {
    const v4i lo = *reinterpret_cast<const v4i *>(p);
    const v4i hi = *reinterpret_cast<const v4i *>(p + 16);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// qrow: the query's 64 x 128 fp8 block; wrow(h): weight of head h.
template <typename WF>
__device__ __forceinline__ void load_q32(Q32 &Q, const unsigned char *qrow, WF wrow, int lane) {
    const int m = lane & 31, hgrp = lane >> 5;
#pragma unroll
    for (int rf = 0; rf < 2; ++rf) {
#pragma unroll
        for (int st = 0; st < 2; ++st) Q.a[rf][st] = load32(qrow + (32 * rf + m) * 128 + 64 * st + 32 * hgrp);
#pragma unroll
        for (int r = 0; r < 16; ++r) Q.w[rf][r] = wrow(32 * rf + 8 * (r / 4) + 4 * hgrp + (r % 4));
    }
}

// Sum over the lane's 32 heads of w * relu(acc) for one 32-key column
// fragment: four independent chains of eight, added pairwise.
__device__ __forceinline__ float epi32(const v16f &a0, const v16f &a1, const Q32 &Q) {
    float c[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        c[h] = Q.w[0][8 * h] * relu(a0[8 * h]);
        c[2 + h] = Q.w[1][8 * h] * relu(a1[8 * h]);
#pragma unroll
        for (int r = 1; r < 8; ++r) {
            c[h] += Q.w[0][8 * h + r] * relu(a0[8 * h + r]);
            c[2 + h] += Q.w[1][8 * h + r] * relu(a1[8 * h + r]);
        }
    }
    return (c[0] + c[1]) + (c[2] + c[3]);
}

// The same sum with the ReLU split w*relu(x) = w*|x|/2 + w*x/2: here the
// weights are already halved and only the |x| half is formed (one FMA with an
// absolute-value operand per head); the linear half is added by the caller.
__device__ __forceinline__ float epi32_abs(const v16f &a0, const v16f &a1, const Q32 &Q) {
    float c[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        c[h] = Q.w[0][8 * h] * fabsf(a0[8 * h]);
        c[2 + h] = Q.w[1][8 * h] * fabsf(a1[8 * h]);
#pragma unroll
        for (int r = 1; r < 8; ++r) {
            c[h] = __builtin_fmaf(Q.w[0][8 * h + r], fabsf(a0[8 * h + r]), c[h]);
            c[2 + h] = __builtin_fmaf(Q.w[1][8 * h + r], fabsf(a1[8 * h + r]), c[2 + h]);
        }
    }
    return (c[0] + c[1]) + (c[2] + c[3]);
}

typedef float v2f __attribute__((ext_vector_type(2)));
typedef int v2i __attribute__((ext_vector_type(2)));

// Linear half of the score for four queries (4jq .. 4jq+3 of the workgroup's
// rows): sum_h (w_h/2) (q_h . k) = qw . k with qw = sum_h (w_h/2) q_h.  qw is
// formed in fp32, scaled by S = 2^e (max_d |qw[d]| S in [128, 256)) and split
// into four fp8 e4m3 terms: term j = rne(r_j 16^j), r_0 = qw S and r_{j+1} =
// r_j - term_j 16^-j (exact in fp32), so sum_j term_j 16^-j = qw S to about
// 2^-16 relative.  Returns the A fragment of a 16x16x128 fp8 MFMA whose row
// r = l%16 is query 4jq + r/4, term r%4 (d = 32(l/16)..+31), and sets inv_s to
// 1/S of query 4jq + l/16, the one whose row block lane l receives.
__device__ v8i linear_terms_frag(const unsigned char *q, const void *w, Enc w_enc, size_t row0, int nrows,
                                 int jq, int lane, float &inv_s) {
    constexpr int H = 64, ROWB = 128;
    const int r = lane & 15, tq = 4 * jq + (r >> 2), kq = lane & 3, dr = 32 * (lane >> 4);
    // each lane of a quad sums 8 of the quad's 32 dimensions over the heads
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (tq < nrows) {
        const size_t qi = row0 + tq;
        const unsigned char *qp = q + qi * H * ROWB + dr + 8 * kq;
        for (int h = 0; h < H; ++h) {
            const float wh = 0.5f * load_w(w, w_enc, qi * H + h);
            const v2i qb = *reinterpret_cast<const v2i *>(qp + (size_t)h * ROWB);
            const v2f f[4] = {__builtin_amdgcn_cvt_pk_f32_fp8(qb[0], false), __builtin_amdgcn_cvt_pk_f32_fp8(qb[0], true),
                              __builtin_amdgcn_cvt_pk_f32_fp8(qb[1], false), __builtin_amdgcn_cvt_pk_f32_fp8(qb[1], true)};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] = __builtin_fmaf(wh, f[e][0], acc[2 * e]);
                acc[2 * e + 1] = __builtin_fmaf(wh, f[e][1], acc[2 * e + 1]);
            }
        }
    }
    float v[32];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) v[8 * k + e] = __shfl(acc[e], (lane & ~3) | k, kWave);
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) m = fmaxf(m, fabsf(v[e]));
    m = fmaxf(m, __shfl_xor(m, 16, kWave));
    m = fmaxf(m, __shfl_xor(m, 32, kWave));
    const int ex = m > 0.f ? 8 - __builtin_amdgcn_frexp_expf(m) : 0;
    const float sc = __builtin_amdgcn_ldexpf(1.f, ex);
    v8i a;
#pragma unroll
    for (int e = 0; e < 32; e += 2) {
        float pick[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float rr = v[e + u] * sc;
            pick[u] = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float x = rr * __builtin_amdgcn_ldexpf(1.f, 4 * j);
                if (j == kq) pick[u] = x;
                const int enc = __builtin_amdgcn_cvt_pk_fp8_f32(x, 0.f, 0, false);
                rr -= __builtin_amdgcn_cvt_f32_fp8(enc, 0) * __builtin_amdgcn_ldexpf(1.f, -4 * j);
            }
        }
        if (e & 2) a[e >> 2] = __builtin_amdgcn_cvt_pk_fp8_f32(pick[0], pick[1], a[e >> 2], true);
        else a[e >> 2] = __builtin_amdgcn_cvt_pk_fp8_f32(pick[0], pick[1], 0, false);
    }
    inv_s = __shfl(__builtin_amdgcn_ldexpf(1.f, -ex), 4 * (lane >> 4), kWave);
    return a;
}

// Scores of 64 keys for one query from the lane's B pieces B[cf][st]:
// key 32cf + l%32, d = 64st + 32(l/32) .. +31.  Lane l gets key l.
__device__ __forceinline__ float score64_mfma32_b(const Q32 &Q, const v8i (&B)[2][2]) {
    const v16f z = {};
    v16f acc[2][2];   // [rf][cf]
#pragma unroll
    for (int rf = 0; rf < 2; ++rf) acc[rf][0] = mfma_fp8_32x32x64(Q.a[rf][0], B[0][0], z);
#pragma unroll
    for (int rf = 0; rf < 2; ++rf) acc[rf][0] = mfma_fp8_32x32x64(Q.a[rf][1], B[0][1], acc[rf][0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rf = 0; rf < 2; ++rf) acc[rf][1] = mfma_fp8_32x32x64(Q.a[rf][0], B[1][0], z);
#pragma unroll
    for (int rf = 0; rf < 2; ++rf) acc[rf][1] = mfma_fp8_32x32x64(Q.a[rf][1], B[1][1], acc[rf][1]);
    const float p0 = epi32(acc[0][0], acc[1][0], Q);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    const float p1 = epi32(acc[0][1], acc[1][1], Q);
    // lanes 0-31 hold column fragment 0 of their head half, lanes 32-63 the other half
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// As score64_mfma32_b, with kb(cf, st) returning the lane's 32-byte B piece.
template <typename KB32>
__device__ __forceinline__ float score64_mfma32(const Q32 &Q, KB32 kb) {
    v8i B[2][2];
#pragma unroll
    for (int cf = 0; cf < 2; ++cf)
#pragma unroll
        for (int st = 0; st < 2; ++st) B[cf][st] = kb(cf, st);
    return score64_mfma32_b(Q, B);
}

// The value is computed before this point: a scheduling anchor that keeps an
// epilogue in the phase whose MFMAs it is meant to overlap.
__device__ __forceinline__ void keep_here(float &x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, kWave));
    return v;
}

// ---------------------------------------------------------------- selection
//
// Candidate buffers are walked four consecutive entries per lane (256 per
// wavefront step: one ds_read_b128 of keys, one ds_read_b64/b128 of indices),
// so each pass over ~2.8K entries is 11 steps.  Buffers are padded by 256
// entries so the last step may read past `cnt` without leaving LDS.

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
constexpr int kStep = 4 * kWave;   // entries per wavefront step
static_assert(kStep == kPadEntries, "buffer padding must cover one wavefront step");

template <typename IdxT>
__device__ __forceinline__ void load4(const uint32_t *bk, const IdxT *bi, int e0, uint32_t (&k)[4], IdxT (&ix)[4]) {
    const v4u kk = *reinterpret_cast<const v4u *>(bk + e0);
    k[0] = kk[0]; k[1] = kk[1]; k[2] = kk[2]; k[3] = kk[3];
    if constexpr (sizeof(IdxT) == 2) {
        typedef unsigned short v4s __attribute__((ext_vector_type(4)));
        const v4s ii = *reinterpret_cast<const v4s *>(bi + e0);
        ix[0] = ii[0]; ix[1] = ii[1]; ix[2] = ii[2]; ix[3] = ii[3];
    } else {
        const v4u ii = *reinterpret_cast<const v4u *>(bi + e0);
        ix[0] = ii[0]; ix[1] = ii[1]; ix[2] = ii[2]; ix[3] = ii[3];
    }
}

// Inclusive prefix sum over the wavefront's lanes (lane l gets the sum over
// lanes 0..l): Hillis-Steele shifts inside each 16-lane row, then the row
// totals are carried across rows with the row-broadcast DPP forms.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);   // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return v;
}

// Bin b holding the need-th largest entry of a 256-bin histogram (bins in
// ascending key order); `above` = entries in bins above b.  Lane l looks at
// bins 252-4l .. 255-4l, so a prefix sum over lanes counts from the top bin
// down.  Requires total >= need >= 1.
__device__ __forceinline__ void hist_find(const uint32_t *hist, int need, int lane, int &bin, uint32_t &above) {
    const int b0 = 4 * (kWave - 1 - lane);
    const v4u hv = *reinterpret_cast<const v4u *>(hist + b0);
    const uint32_t s = hv[0] + hv[1] + hv[2] + hv[3];
    const uint32_t S = wave_incl_scan(s);   // entries in bins >= b0
    const uint32_t E = S - s;               // entries in bins > b0 + 3
    const uint32_t nd = (uint32_t)need;
    const bool here = E < nd && S >= nd;
    int bsel;
    uint32_t c = E;
    if (c + hv[3] >= nd) bsel = 3;
    else {
        c += hv[3];
        if (c + hv[2] >= nd) bsel = 2;
        else {
            c += hv[2];
            if (c + hv[1] >= nd) bsel = 1;
            else { c += hv[1]; bsel = 0; }
        }
    }
    const uint64_t m = ballot(here);
    const int src = m ? __builtin_ctzll(m) : 0;
    bin = __builtin_amdgcn_readlane(b0 + bsel, src);
    above = (uint32_t)__builtin_amdgcn_readlane((int)c, src);
}

// In-place stable filter of buf[0..cnt): keeps keys > gt_than, plus (TIES)
// the first `eq_keep` keys equal to eq_key.  Returns the new count;
// *kept_max = largest kept key.  The next step's entries are read before the
// current step's kept entries are written: writes of a step land below
// base + kStep, the next step reads from there upward, so they never overlap.
template <bool TIES, typename IdxT>
__device__ int filter4(uint32_t *bk, IdxT *bi, int cnt, uint32_t gt_than, uint32_t eq_key, int eq_keep, int lane,
                       uint32_t *kept_max) {
    int out = 0, eqseen = 0;
    uint32_t mx = 0;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint32_t k[4];
    IdxT ix[4];
    if (cnt > 0) load4(bk, bi, 4 * lane, k, ix);
    for (int base = 0; base < cnt; base += kStep) {
        const int e0 = base + 4 * lane;
        uint32_t kn[4];
        IdxT ixn[4];
        if (base + kStep < cnt) load4(bk, bi, e0 + kStep, kn, ixn);
        bool keep[4];
        uint64_t KM[4];
        int keepb = 0;
        if constexpr (TIES) {
            bool eq[4];
            uint64_t EM[4];
            int eqb = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                eq[j] = e0 + j < cnt && eq_keep > 0 && k[j] == eq_key;
                EM[j] = ballot(eq[j]);
                eqb += __popcll(EM[j] & lt);
            }
            int erank = eqseen + eqb;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                keep[j] = e0 + j < cnt && (k[j] > gt_than || (eq[j] && erank < eq_keep));
                erank += eq[j] ? 1 : 0;
                eqseen += __popcll(EM[j]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) keep[j] = e0 + j < cnt && k[j] > gt_than;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            KM[j] = ballot(keep[j]);
            keepb += __popcll(KM[j] & lt);
        }
        int pos = out + keepb;
        wave_lds_order();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (keep[j]) {
                bk[pos] = k[j];
                bi[pos] = ix[j];
                mx = max(mx, k[j]);
                ++pos;
            }
        }
        wave_lds_order();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            out += __popcll(KM[j]);
            k[j] = kn[j];
            ix[j] = ixn[j];
        }
    }
    if (kept_max) *kept_max = wave_max_u32(mx);
    return out;
}

// In-place stable filter keeping keys > gt (no ties), for the binned
// compaction.  Every lane writes all four of its entries each step: kept
// ones to their compacted slot, dropped ones to its own slot in the padding
// past the last row's buffer (pad_k / pad_i), so no write is predicated.
// The next step's entries are read before this step's writes (those land
// below base + kStep).  Returns the new count.
template <typename IdxT>
__device__ int filter_gt(uint32_t *bk, IdxT *bi, int cnt, uint32_t gt, uint32_t *pad_k, IdxT *pad_i, int lane) {
    int out = 0;
    // two register buffers by step parity, so that the next step's entries
    // are read a whole step ahead without register moves (a move of a
    // register whose load is in flight would wait for it)
    uint32_t k[2][4];
    IdxT ix[2][4];
    if (cnt > 0) load4(bk, bi, 4 * lane, k[0], ix[0]);
    auto step = [&](auto P_, int base) {
        constexpr int P = decltype(P_)::value;
        const int e0 = base + 4 * lane;
        if (base + kStep < cnt) load4(bk, bi, e0 + kStep, k[P ^ 1], ix[P ^ 1]);
        const uint64_t K0 = ballot(e0 < cnt && k[P][0] > gt);
        const uint64_t K1 = ballot(e0 + 1 < cnt && k[P][1] > gt);
        const uint64_t K2 = ballot(e0 + 2 < cnt && k[P][2] > gt);
        const uint64_t K3 = ballot(e0 + 3 < cnt && k[P][3] > gt);
        const int kp0 = (int)((K0 >> lane) & 1u), kp1 = (int)((K1 >> lane) & 1u);
        const int kp2 = (int)((K2 >> lane) & 1u), kp3 = (int)((K3 >> lane) & 1u);
        const int p0 = out + lanes_below(K0) + lanes_below(K1) + lanes_below(K2) + lanes_below(K3);
        const int p1 = p0 + kp0, p2 = p1 + kp1, p3 = p2 + kp2;
        uint32_t *a0 = kp0 ? bk + p0 : pad_k + lane;
        uint32_t *a1 = kp1 ? bk + p1 : pad_k + lane;
        uint32_t *a2 = kp2 ? bk + p2 : pad_k + lane;
        uint32_t *a3 = kp3 ? bk + p3 : pad_k + lane;
        IdxT *c0 = kp0 ? bi + p0 : pad_i + lane;
        IdxT *c1 = kp1 ? bi + p1 : pad_i + lane;
        IdxT *c2 = kp2 ? bi + p2 : pad_i + lane;
        IdxT *c3 = kp3 ? bi + p3 : pad_i + lane;
        wave_lds_order();
        *a0 = k[P][0]; *a1 = k[P][1]; *a2 = k[P][2]; *a3 = k[P][3];
        *c0 = ix[P][0]; *c1 = ix[P][1]; *c2 = ix[P][2]; *c3 = ix[P][3];
        wave_lds_order();
        out += __popcll(K0) + __popcll(K1) + __popcll(K2) + __popcll(K3);
    };
    for (int base = 0; base < cnt; base += 2 * kStep) {
        step(std::integral_constant<int, 0>{}, base);
        if (base + kStep < cnt) step(std::integral_constant<int, 1>{}, base + kStep);
    }
    return out;
}

// Segment starts after an in-place stable filter of bkey[0..cnt) that keeps
// entry i iff key_i > gt, or key_i == eq and it is among the first eq_keep
// such entries: segs[j] (j = 1 .. nseg-1, a start position or INT_MAX when the
// segment has not been reached) becomes the number of kept entries before it.
// Reads the keys, so it runs before the filter.  Wave-level.
__device__ void seg_remap(const uint32_t *bkey, int cnt, int *segs, int nseg, uint32_t gt, uint32_t eq, int eq_keep,
                          int lane) {
    for (int j = 1; j < nseg; ++j) {
        const int pj = segs[j];
        if (pj == INT_MAX) break;   // later segments not reached either
        const int lim = min(pj, cnt);
        int ngt = 0, neq = 0;
        for (int base = 0; base < lim; base += kStep) {
            const int e0 = base + 4 * lane;
            const v4u kk = *reinterpret_cast<const v4u *>(bkey + e0);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bool in = e0 + t < lim;
                ngt += __popcll(ballot(in && kk[t] > gt));
                neq += __popcll(ballot(in && kk[t] == eq));
            }
        }
        const int np = ngt + min(neq, eq_keep);
        wave_lds_order();
        if (lane == 0) segs[j] = np;
        wave_lds_order();
    }
}

// Exact k-th largest key among bkey[0..cnt) (cnt >= k) by MSB-first radix
// select, then in-place stable compaction to the k best (ties: lowest index =
// earliest entry).  Wave-level; `hist` is this wave's 256-entry LDS scratch.
// Returns the k-th largest key.
template <typename IdxT>
__device__ uint32_t select_compact(uint32_t *bkey, IdxT *bidx, int &cnt, int k, uint32_t *hist, int lane,
                                   uint32_t *kept_max = nullptr, int *segs = nullptr, int nseg = 1) {
    // bits above `top` are common to every key (from the buffer's min and max)
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    for (int base = 0; base < cnt; base += kStep) {
        const int e0 = base + 4 * lane;
        const v4u kk = *reinterpret_cast<const v4u *>(bkey + e0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (e0 + j < cnt) { mn = min(mn, kk[j]); mx = max(mx, kk[j]); }
    }
    mn = ~wave_max_u32(~mn);
    mx = wave_max_u32(mx);
    int top = (mn == mx) ? 0 : 32 - __builtin_clz(mn ^ mx);
    uint32_t pmask = top == 32 ? 0u : ~((1u << top) - 1u);
    uint32_t prefix = mn & pmask;
    int need = k;
    while (top > 0) {
        const int width = top < 8 ? top : 8;
        const int shift = top - width;
        const uint32_t dmask = (1u << width) - 1u;
        for (int j = lane; j < kHistWords; j += kWave) hist[j] = 0;
        wave_lds_order();
        for (int base = 0; base < cnt; base += kStep) {
            const int e0 = base + 4 * lane;
            const v4u kk = *reinterpret_cast<const v4u *>(bkey + e0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool in = e0 + j < cnt && (kk[j] & pmask) == prefix;
                atomicAdd(&hist[in ? ((kk[j] >> shift) & dmask) : 256u + lane], 1u);
            }
        }
        wave_lds_order();
        int bin;
        uint32_t above;
        hist_find(hist, need, lane, bin, above);
        prefix |= (uint32_t)bin << shift;
        pmask |= dmask << shift;
        need -= (int)above;
        top = shift;
        wave_lds_order();
    }
    if (nseg > 1) seg_remap(bkey, cnt, segs, nseg, prefix, prefix, need, lane);
    cnt = filter4<true, IdxT>(bkey, bidx, cnt, prefix, prefix, need, lane, kept_max);
    return prefix;
}

// Binned-selection state of one row (wave-uniform, one row per wavefront).
// A compaction builds the wave's 256-bin histogram of the buffered keys by
// their bin above the base `lo` (log-spaced bins, see bin_of) and reads the
// cut off it.  (With a sampled starting threshold a row compacts only a few
// times, so building the histogram then is cheaper than keeping it current
// through every append.)
struct BinState {
    int cnt;          // entries in the buffer
    uint32_t thr;     // append filter: key > thr
    float thr_f;      // the same filter on scores: score > thr_f
    uint32_t lo;      // histogram base (<= every buffered key)
    int cur_seg;      // key segment of the last append (segment table)
};

// Largest float whose order-preserving key is <= thr: for every finite f,
// score_key(f) > thr  <=>  f > key_floor_float(thr).
__device__ __forceinline__ float key_floor_float(uint32_t thr) {
    if (thr >= 0x80000000u) return __uint_as_float(min(thr & 0x7FFFFFFFu, 0x7F800000u));
    if (thr >= 0x7FFFFFFEu) return __uint_as_float(0x80000001u);   // -denorm_min
    if (thr < 0x007FFFFFu) return -INFINITY;
    return __uint_as_float(~thr);
}

// Log-spaced bins of d = key - lo: d < 8 has its own bin; above that, eight
// bins per power of two (d's leading bit plus the next three bits), so the
// bins are finest just above the base, where the cut falls.  Bin order is
// key order; 8 + 8 * 29 bins cover every 32-bit d.
__device__ __forceinline__ uint32_t bin_of(uint32_t key, uint32_t lo) {
    const uint32_t d = key - lo;
    if (d < 8u) return d;
    const int e = 31 - __builtin_clz(d);
    return 8u * (uint32_t)(e - 2) + ((d >> (e - 3)) & 7u);
}

// smallest d of bin b
__device__ __forceinline__ uint32_t bin_floor(int b) {
    if (b < 8) return (uint32_t)b;
    const int e = b / 8 + 2;
    return (uint32_t)(8 + (b & 7)) << (e - 3);
}

// Histogram of the buffer above base lo.
template <typename IdxT>
__device__ void rebuild_hist(const uint32_t *bkey, BinState &st, uint32_t lo, uint32_t *hist, int lane) {
    st.lo = lo;
    for (int j = lane; j < kHistWords; j += kWave) hist[j] = 0;
    wave_lds_order();
    for (int base = 0; base < st.cnt; base += kStep) {
        const int e0 = base + 4 * lane;
        const v4u kk = *reinterpret_cast<const v4u *>(bkey + e0);
#pragma unroll
        for (int j = 0; j < 4; ++j) atomicAdd(&hist[e0 + j < st.cnt ? bin_of(kk[j], lo) : 256u + lane], 1u);
    }
    wave_lds_order();
}

template <typename IdxT>
__device__ uint32_t buffer_min(const uint32_t *bkey, int cnt, int lane) {
    uint32_t mn = 0xFFFFFFFFu;
    for (int base = 0; base < cnt; base += kStep) {
        const int e0 = base + 4 * lane;
        const v4u kk = *reinterpret_cast<const v4u *>(bkey + e0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (e0 + j < cnt) mn = min(mn, kk[j]);
    }
    return ~wave_max_u32(~mn);
}

template <typename IdxT>
__device__ void compact_exact(uint32_t *bkey, IdxT *bidx, BinState &st, int k, uint32_t *hist, int lane, int *segs,
                              int nseg) {
    const uint32_t theta = select_compact<IdxT>(bkey, bidx, st.cnt, k, hist, lane, nullptr, segs, nseg);
    st.thr = theta;
    st.thr_f = key_floor_float(theta);
}

// Shrink the buffer off a histogram of it: the bin holding the k-th largest
// key is read off it, every entry at or above that bin's lower edge is kept
// (at least k entries, all better than anything dropped), and the edge
// bounds the threshold.  Bins are log-spaced above the buffer's smallest key;
// when the cut's bin holds too many entries (too little room freed), exact
// selection takes over.
// Precondition: st.cnt >= k.
template <typename IdxT>
__device__ __forceinline__ void compact_binned(uint32_t *bkey, IdxT *bidx, BinState &st, int k, int cap, uint32_t *hist,
                               uint32_t *pad_k, IdxT *pad_i, int lane, int *segs, int nseg) {
    rebuild_hist<IdxT>(bkey, st, buffer_min<IdxT>(bkey, st.cnt, lane), hist, lane);
    int bstar;
    uint32_t above;
    hist_find(hist, k, lane, bstar, above);
    const uint32_t nkeep = above + hist[bstar];
    wave_lds_order();
    if (bstar > 0 && (int)nkeep <= cap - 2 * KB) {
        const uint32_t edge = st.lo + bin_floor(bstar);   // keep keys >= edge
        if (nseg > 1) seg_remap(bkey, st.cnt, segs, nseg, edge - 1u, 0u, 0, lane);
        st.cnt = filter_gt<IdxT>(bkey, bidx, st.cnt, edge - 1u, pad_k, pad_i, lane);
        st.thr = edge - 1u;
        st.thr_f = key_floor_float(st.thr);
        return;
    }
    compact_exact<IdxT>(bkey, bidx, st, k, hist, lane, segs, nseg);
}

struct PrefillParams {
    const unsigned char *q, *k;
    const void *w;
    int32_t *t_out;
    float *scores;
    int B, Lq, Lk, topk, cap;
    int nthreads;   // == blockDim.x, passed as an argument so it lives in an SGPR
    Enc w_enc;
    // serving batch over a paged key cache (the Paged kernels): sequence b owns
    // packed query rows query_start[b] .. query_start[b+1]-1, its last q_len
    // positions of seq_lens[b]; its keys live in pages block_table[b][s >> bs_log2]
    // of the pool k [num_blocks][1 << bs_log2][D]; its row blocks are
    // workgroups rb_start[b] .. rb_start[b+1]-1.  Lq and Lk above are then the
    // largest q_len and seq_len allowed.
    const int32_t *query_start, *seq_lens, *block_table, *rb_start;
    int num_seqs, bs_log2, max_blocks, num_blocks;
};

// LDS plan of the prefill kernel; identical on host and device.
struct PrefillLds {
    size_t ktile, stage, hist, flags, state, segs, bkey, bidx, total;
};

// `stage` holds one score per (row, key of a block): once for the staged
// kernels (H < 16), twice (by block parity) for the linear score terms of the
// pipelined 64-head kernel.
__host__ __device__ inline PrefillLds prefill_lds(int waves, int tw, int pitch, int cap, int idx_bytes, int stage_bufs,
                                                  int ktiles) {
    PrefillLds L;
    const int R = waves * tw;
    L.ktile = 0;
    size_t off = (size_t)ktiles * KB * pitch;
    L.stage = off;
    off += (size_t)stage_bufs * waves * tw * KB * 4;
    L.hist = off;
    off += (size_t)waves * kHistWords * 4;
    L.flags = off;
    off += 64;
    L.state = off;
    off += (size_t)R * 8;
    L.segs = off;
    off += (size_t)waves * kMaxSeg * 4;
    L.bkey = off;
    off += ((size_t)R * cap + kPadEntries) * 4;
    off = (off + 15) & ~(size_t)15;
    L.bidx = off;
    off += ((size_t)R * cap + kPadEntries) * idx_bytes;
    L.total = (off + 15) & ~(size_t)15;
    return L;
}

// Var: bit 0 set when a score row may be written for tests (p.scores), bit 1
// when keys may extend past 65,536 (segment table); launches without either
// run a body with those per-block checks compiled out.
template <Enc E, int D, int H, typename IdxT, bool Paged, int Var>
__global__ __launch_bounds__(kMaxThreads) __attribute__((amdgpu_waves_per_eu(1, 2))) void prefill_kernel(PrefillParams p) {
    using S = Shape<E, D>;
    constexpr int TW = 64 / H;              // query rows per wave
    constexpr bool kStaged = H < 16;        // scores go through LDS before selection
    constexpr bool kBinned = TW == 1;       // binned selection + batched compaction
    constexpr bool kMfma32 = E == Enc::FP8 && H == 64 && D == 128;
    // the pipelined sweep below needs kPipeWaves wavefronts, which the LDS
    // plan always gives with 16-bit candidate indices (keys up to 65536, or up
    // to kMaxSeg * 65536 with the segment table)
    constexpr bool kPipe = kMfma32 && sizeof(IdxT) == 2;
    constexpr bool kDbg = (Var & 1) != 0, kSeg = (Var & 2) != 0;
    const int waves = p.nthreads / kWave;
    const int R = waves * TW;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave, g = lane >> 4,
              n = lane & 15;

    extern __shared__ __align__(16) unsigned char smem[];
    const PrefillLds L =
        prefill_lds(waves, TW, S::PITCH, p.cap, (int)sizeof(IdxT), kStaged ? 1 : kPipe ? 2 : 0, kPipe ? kPipeTiles : 2);
    unsigned char *ktile = smem + L.ktile;
    float *stage = reinterpret_cast<float *>(smem + L.stage) + (size_t)wave * TW * KB;
    uint32_t *hist = reinterpret_cast<uint32_t *>(smem + L.hist) + wave * kHistWords;
    int *flags = reinterpret_cast<int *>(smem + L.flags);
    int *rcnt = reinterpret_cast<int *>(smem + L.state);
    uint32_t *rthr = reinterpret_cast<uint32_t *>(smem + L.state) + R;
    uint32_t *bkey_all = reinterpret_cast<uint32_t *>(smem + L.bkey);
    IdxT *bidx_all = reinterpret_cast<IdxT *>(smem + L.bidx);

    // This workgroup's sequence b, its query count Lq and key count Lk, the
    // packed index row0 of its query 0 in q, w and t_out, and its row block
    // rb.  Heaviest row blocks (largest positions) are dispatched first.
    int b, Lq, Lk, rb;
    size_t row0;
    if constexpr (Paged) {
        const int wg = (int)blockIdx.x;
        if (wg >= p.rb_start[p.num_seqs]) return;   // the grid is an upper bound on the row blocks
        int lo = 0, hi = p.num_seqs - 1;            // last sequence with rb_start <= wg
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.rb_start[mid] <= wg) lo = mid;
            else hi = mid - 1;
        }
        b = lo;
        // out-of-contract metadata is clamped (as the row-block count was) so
        // that every row lies in the packed rows (p.Lq = total_q), every key
        // in the pages the table can name and within the longest sequence
        const int q0 = min(max(p.query_start[b], 0), p.Lq);
        const int q1 = min(max(p.query_start[b + 1], q0), p.Lq);
        const int lk_cap = min(p.Lk, p.max_blocks << p.bs_log2);
        Lq = min(q1 - q0, lk_cap);
        Lk = min(max(p.seq_lens[b], Lq), lk_cap);
        row0 = (size_t)q0;
        rb = (Lq + R - 1) / R - 1 - (wg - p.rb_start[b]);
    } else {
        Lq = p.Lq;
        Lk = p.Lk;
        const int nrb = (Lq + R - 1) / R;
        rb = nrb - 1 - (int)(blockIdx.x / p.B);
        b = (int)(blockIdx.x % p.B);
        row0 = (size_t)b * Lq;
    }
    const int i0 = rb * R;
    const int off = Lk - Lq;
    const int pmax = off + min(i0 + R, Lq) - 1;
    const int nblk = pmax / KB + 1;
    // paged: the page of the 64-key block holding key s (pages hold a power of
    // two >= 64 keys, so a block lies in one page); pages are clamped to the
    // pool.  The table is read through the constant address space, so its
    // loads are uniform scalar loads, off the vector-memory counter.
    const __attribute__((address_space(4))) int32_t *btab =
        Paged ? (const __attribute__((address_space(4))) int32_t *)(p.block_table + (size_t)b * p.max_blocks) : nullptr;
    auto page_of = [&](int s) -> const unsigned char * {
        const int pg = min(max(btab[s >> p.bs_log2], 0), p.num_blocks - 1);
        return p.k + ((size_t)pg << p.bs_log2) * S::ROWB;
    };

    Q32 Q32f;
    if constexpr (kMfma32) {
        const int i = i0 + wave;
        if (i < Lq) {
            const size_t qi = row0 + i;
            load_q32(Q32f, p.q + qi * H * S::ROWB, [&](int h) { return load_w(p.w, p.w_enc, qi * H + h); }, lane);
        } else {
            load_q32(Q32f, p.q, [&](int h) { return 0.f; }, lane);
        }
        if constexpr (kPipe) {
#pragma unroll
            for (int rf = 0; rf < 2; ++rf)
#pragma unroll
                for (int r = 0; r < 16; ++r) Q32f.w[rf][r] *= 0.5f;   // ReLU split: w*|x|/2 + w*x/2
        }
    }
    // A fragments: fragment f, row r = 16f + n -> (t, h) = (r / H, r % H)
    Frag<E, D> A[4];
    float wv[4][4];
#pragma unroll
    for (int f = 0; f < 4 && !kMfma32; ++f) {
        const int r = 16 * f + n, t = r / H, h = r % H;
        const int i = i0 + wave * TW + t;
        if (i < Lq) {
            const size_t qrow = ((row0 + i) * H + h) * S::ROWB;
            load_frag<E, D>(A[f], p.q + qrow, g);
        } else {
            zero_frag<E, D>(A[f]);
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int ro = 16 * f + 4 * g + ii, to = ro / H, ho = ro % H;
            const int io = i0 + wave * TW + to;
            wv[f][ii] = io < Lq ? load_w(p.w, p.w_enc, (row0 + io) * H + ho) : 0.f;
        }
    }
    for (int t = lane; t < TW; t += kWave) {
        rcnt[wave * TW + t] = 0;
        rthr[wave * TW + t] = 0u;
    }
    if (tid < 4) flags[tid] = 0;   // words 0-2: compaction requests; word 3: the sample failed
    BinState st;
    st.cnt = 0; st.thr = 0u; st.thr_f = -INFINITY; st.lo = 0u; st.cur_seg = 0;
    const int want_level = p.topk + (p.cap - p.topk) / 4;   // past a quarter of the slack
    // segment table of this wave's row (pipelined sweep with keys beyond 65536)
    int *segs = reinterpret_cast<int *>(smem + L.segs) + wave * kMaxSeg;
    const int nseg = kPipe && kSeg ? (Lk + 65535) >> 16 : 1;
    auto seg_reset = [&]() {   // an empty buffer: every segment not reached yet
        if (nseg > 1) {
            wave_lds_order();
            if (lane < kMaxSeg) segs[lane] = lane == 0 ? 0 : INT_MAX;
            wave_lds_order();
        }
        st.cur_seg = 0;
    };
    seg_reset();

    // stage key block 0.  Thread tid stages 16-byte chunks tid + c*blockDim
    // (c < cpt).  Keys past Lk are clamped to the last key: their scores lie
    // beyond every query's position and are never used.
    constexpr int CPK = S::ROWB / 16;               // chunks per key
    const int nchunk = KB * CPK;
    const int cpt = (nchunk + p.nthreads - 1) / p.nthreads;
    const unsigned char *kseq = Paged ? p.k : p.k + (size_t)b * Lk * S::ROWB;
    v4i kreg[kChunkMax];
    auto fetch = [&](int blk) {
        // paged: the page of the block (of the last key for a block past it)
        const unsigned char *pb = nullptr;
        if constexpr (Paged) pb = page_of(min(blk * KB, Lk - 1));
#pragma unroll
        for (int c = 0; c < kChunkMax; ++c) {
            if (c < cpt) {
                const int ci = min(tid + c * p.nthreads, nchunk - 1);
                const int key = min(blk * KB + ci / CPK, Lk - 1);
                if constexpr (Paged)
                    kreg[c] = *reinterpret_cast<const v4i *>(
                        pb + (size_t)(key & ((1 << p.bs_log2) - 1)) * S::ROWB + (ci % CPK) * 16);
                else
                    kreg[c] = *reinterpret_cast<const v4i *>(kseq + (size_t)key * S::ROWB + (ci % CPK) * 16);
            }
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int c = 0; c < kChunkMax; ++c) {
            if (c < cpt) {
                const int ci = tid + c * p.nthreads;
                if (ci < nchunk)
                    *reinterpret_cast<v4i *>(ktile + (size_t)buf * KB * S::PITCH + (ci / CPK) * S::PITCH +
                                             (ci % CPK) * 16) = kreg[c];
            }
        }
    };
    // Streaming selection of one 64-key block (lane l: key base + l, score sc)
    // for the wave's row (one row per wavefront); returns whether the row's
    // buffer must be compacted before the next block.
    auto select_binned = [&](float sc, int base) -> bool {
        const int i = i0 + wave;
        const int pos = off + i;
        if (i >= Lq || base > pos) return false;
        const int s = base + lane;
        if (kDbg && p.scores) {   // the full score row, for tests only
            if (s < Lk) p.scores[(row0 + i) * Lk + s] = s <= pos ? sc : -INFINITY;
        }
        // one ballot per comparison (each compare writes its lane mask
        // directly), and the mask feeds the write predicate (inverse ballot),
        // so the candidate test is never kept as a per-lane value
        const uint64_t m = ballot(s <= pos) & ballot(sc > st.thr_f);
        if (m) {
            uint32_t *bk = bkey_all + (size_t)wave * p.cap;
            IdxT *bi = bidx_all + (size_t)wave * p.cap;
            if (nseg > 1) {
                // the first append in a later key segment starts it (blocks of
                // 64 keys never straddle a segment; appends come in index order)
                const int sg = base >> 16;
                if (sg > st.cur_seg) {
                    wave_lds_order();
                    if (lane > st.cur_seg && lane <= sg) segs[lane] = st.cnt;
                    wave_lds_order();
                    st.cur_seg = sg;
                }
            }
            const int at = st.cnt + lanes_below(m);
            const uint32_t key = score_key(sc);
            // the mask as an opaque scalar value: the compiler would otherwise
            // fold the inverse ballot back into the comparison and carry that
            // across the branch as a per-lane value
            uint64_t mw = m;
            asm volatile("" : "+s"(mw));
            if (__builtin_amdgcn_inverse_ballot_w64(mw)) {
                bk[at] = key;
                bi[at] = (IdxT)s;
            }
            st.cnt += __popcll(m);
        }
        return st.cnt > p.cap - KB;
    };
    // Compaction requests of iteration it: word it%3 collects them; word
    // (it+1)%3 was last read before the previous barrier and is next written
    // after this one.  After the barrier every requesting row compacts, and so
    // does every row past a quarter of its slack.
    auto raise_flags = [&](int it, bool need) {
        if constexpr (kBinned) {
            if (need && lane == 0) flags[it % 3] = 1;   // the words are only tested for nonzero
            if (wave == 0 && lane == 0) flags[(it + 1) % 3] = 0;
        }
    };
    auto compact_if_flagged = [&](int it) {
        if constexpr (kBinned) {
            if (st.cnt > want_level && flags[it % 3]) {
                compact_binned<IdxT>(bkey_all + (size_t)wave * p.cap, bidx_all + (size_t)wave * p.cap, st, p.topk,
                                     p.cap, hist, bkey_all + (size_t)R * p.cap, bidx_all + (size_t)R * p.cap, lane, segs,
                                     nseg);
            }
        }
    };

    // last position among this wave's valid rows (for skipping blocks)
    const int wlast = min(i0 + wave * TW + TW, Lq) - 1;
    const int wpmax = off + wlast;
    const bool wave_has_rows = wlast >= i0 + wave * TW;

    if constexpr (kPipe) {
        // Pipelined sweep (one query of 64 heads per wavefront, kPipeWaves
        // wavefronts; each thread stages CPT 16-byte chunks of every key block).
        // Iteration blk:
        //  * loads key block blk+2 into registers (stored to LDS an iteration later);
        //  * reads block blk's B operands from LDS;
        //  * phase 1: MFMAs of key fragment 0 of block blk, interleaved with the
        //    epilogue of key fragment 1 of block blk-1;
        //  * one key tile: barrier (every wave holds block blk's operands),
        //    then stores block blk+1 to the tile;
        //  * selection of block blk-1;
        //  * phase 2: MFMAs of key fragment 1 of block blk, interleaved with the
        //    epilogue of key fragment 0 of block blk;
        //  * two key tiles: stores block blk+1 to the idle tile;
        //  * barrier, batched compactions.
        // Every epilogue reads accumulators finished a phase earlier, fragment 1's
        // MFMAs run across the barrier, and the staging loads have two iterations
        // to land.  Waves past their row's last block keep computing (their scores
        // are masked by position), so the loop body has no branches around MFMAs.
        // With four wavefronts two workgroups share a compute unit, so each
        // SIMD runs one wavefront of each; their barriers are independent, and
        // one workgroup's selection, compactions, start and end overlap the
        // other's MFMAs.
        //
        // The epilogue uses the ReLU split w*relu(x) = w*|x|/2 + w*x/2: one FMA on
        // |x| per (head, key), while the linear half of every row's score,
        // qw.k per row (qw = sum_h (w_h/2) q_h), takes one 16x16x128 fp8 MFMA per
        // wavefront and block: wavefront v covers rows 4jq..4jq+3 and keys
        // 16sq..16sq+15 of the block (jq = v mod (kPipeWaves/4), sq = the
        // rest) and leaves them in LDS (by block parity) for the owning rows'
        // selection an iteration later.
        constexpr int RG = kPipeWaves / 4;
        const int jq = wave % RG, sq = wave / RG;
        float inv_s_lin;
        const v8i Alin = linear_terms_frag(p.q, p.w, p.w_enc, row0 + i0, Lq - i0, jq, lane, inv_s_lin);
        float *linbuf = reinterpret_cast<float *>(smem + L.stage);   // [2][kPipeWaves rows][64 keys]
        const int lin_put = (4 * jq + (lane >> 4)) * KB + 16 * sq + (lane & 15);
        const int lin_get = wave * KB + lane;
        constexpr int CPK = S::ROWB / 16;
        // CPT 16-byte chunks per thread and key block, rows krow + c * (rows per pass)
        constexpr int CPT = KB * CPK / (kPipeWaves * kWave);
        static_assert(CPT * kPipeWaves * kWave == KB * CPK, "whole 16-byte chunks per thread and key block");
        constexpr int KROWS = kPipeWaves * kWave / CPK;
        const int krow = tid / CPK, kcol = (tid % CPK) * 16;
        auto fetch1c = [&](int blk, int kr) {
            const int key = min(blk * KB + kr, Lk - 1);   // past Lk: clamped, never used
            // 32-bit offset from the block's page (one VALU add instead of
            // 64-bit address arithmetic)
            const unsigned char *pb = page_of(min(blk * KB, Lk - 1));
            const uint32_t o = (uint32_t)(key & ((1 << p.bs_log2) - 1)) * (uint32_t)S::ROWB + (uint32_t)kcol;
            return *reinterpret_cast<const v4i *>(pb + o);
        };
        struct KR { v4i c[CPT]; };
        // Contiguous keys: block blk is read through a buffer descriptor (scalar
        // registers) whose base is the block's first key and whose size ends at
        // the sequence's last key; the lane offsets are loop constants, and keys
        // past the sequence read as zero (the hardware's range check; their
        // scores are masked by position), so a block costs no address VALU.
        uint32_t voff[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) voff[c] = (uint32_t)(krow + c * KROWS) * (uint32_t)S::ROWB + (uint32_t)kcol;
        auto fetch1 = [&](int blk) {
            KR r;
            if constexpr (Paged) {
#pragma unroll
                for (int c = 0; c < CPT; ++c) r.c[c] = fetch1c(blk, krow + c * KROWS);
            } else {
                const int ub = __builtin_amdgcn_readfirstlane(blk);
                // bytes from the block on (this sweep covers at most kMaxSeg * 65536
                // keys of 128 bytes: 32-bit arithmetic)
                const int rem = (Lk - min(ub * KB, Lk)) * S::ROWB;
                const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<unsigned char *>(kseq) + (size_t)ub * (KB * S::ROWB), (short)0,
                    min(rem, KB * S::ROWB), kBufferWord3);
#pragma unroll
                for (int c = 0; c < CPT; ++c)
                    r.c[c] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[c], 0, 0));
            }
            return r;
        };
        // Key tile swizzle: the 32-byte half h of key row r (16-byte chunks
        // 2h, 2h+1) sits at half h ^ (r2 ^ r3 ^ r4).  A 16-byte LDS read
        // serves together the 16 lanes with one value of (l5, l2 ^ l3 ^ l4);
        // with the 144-byte pitch both operand reads below (32 rows x one
        // half, 16 rows x four halves) then cover all 64 banks in each cycle.
        auto kswz = [](int r) { return (__builtin_popcount(r & 28) & 1) << 5; };
        auto stash1 = [&](int buf, const KR &v) {
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                const int r = krow + c * KROWS;
                *reinterpret_cast<v4i *>(ktile + (size_t)buf * KB * S::PITCH + r * S::PITCH + (kcol ^ kswz(r))) = v.c[c];
            }
        };
        auto combine = [](float p0, float p1) {
            // lanes 0-31 hold key fragment 0 of their head half, lanes 32-63 the other half
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
            return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        };
        // Sampled start.  The sweep first visits the ns sampled blocks 0, 32,
        // 64, ... and then every block in order (iteration it -> block
        // bmap(it)).  After the sample's selection each row keeps only its
        // threshold tau, the r-th largest sampled key, and empties its buffer;
        // the full sweep then appends the keys above tau (the sampled blocks
        // again, so the buffer stays in index order).  If the row ends with
        // at least k entries, its k-th largest key is above tau and every
        // key that tau filtered out lies below it: the result is exact.  A
        // row left with fewer than k entries makes its workgroup sweep again
        // without the sample.  For i.i.d. scores r is about 7k/128 = 112: the
        // number of keys above tau is about 7k/4 with a relative spread of
        // 1/sqrt(r) (9.4 %), so a shortfall below k is a 4.5-sigma event
        // (about one row in 300,000); a row then appends about 7k/4 keys
        // instead of k(1 + ln(n/k)), and compacts once or twice instead of ~16.
        int ns = nblk >= kSampleMinBlocks ? (nblk - 1) / kSampleStride + 1 : 0;
        auto bmap = [&](int it) { return it < ns ? it * kSampleStride : it - ns; };
        auto tau_step = [&]() {
            const int i = i0 + wave;
            if (i >= Lq) return;
            const int pos = off + i;
            int nsk = 0;   // sampled keys at or before the row's position
            for (int j = 0; j < ns; ++j) {
                const int lo = j * kSampleStride * KB;
                if (lo <= pos) nsk += min(KB, pos + 1 - lo);
            }
            const long long den = (long long)kSampleMarginDen * (pos + 1);
            const int r = (int)(((long long)kSampleMarginNum * p.topk * nsk + den - 1) / den);
            uint32_t thr = 0u;   // 0: no filter
            if (r >= kSampleMinRank && r <= st.cnt) {
                int c = st.cnt;
                thr = select_compact<IdxT>(bkey_all + (size_t)wave * p.cap, bidx_all + (size_t)wave * p.cap, c, r, hist,
                                           lane);
            }
            st.cnt = 0;
            st.thr = thr;
            st.thr_f = key_floor_float(thr);
            st.lo = 0u;
            seg_reset();
        };
        for (;;) {
        const int niter = ns + nblk;
        KR kr[2];
        kr[0] = fetch1(bmap(0));
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // queries, weights and the first block
        stash1(0, kr[0]);
        kr[1] = fetch1(bmap(1));
        lds_barrier();

        const v16f z = {};
        v16f a1[2] = {z, z};   // key fragment 1 of the previous block
        float p0_prev = 0.f;   // epilogue of key fragment 0 of the previous block
        auto iter = [&](auto PAR_, int blk) {
            constexpr int PAR = decltype(PAR_)::value;   // == blk & 1 (blk: the iteration)
            kr[PAR] = fetch1(bmap(blk + 2));
            const unsigned char *kt = ktile + (kPipeTiles == 2 ? (size_t)PAR * KB * S::PITCH : 0);
            v8i B[2][2];
#pragma unroll
            for (int cf = 0; cf < 2; ++cf)
#pragma unroll
                for (int st2 = 0; st2 < 2; ++st2)
                    B[cf][st2] = load32(kt + (32 * cf + (lane & 31)) * S::PITCH + ((64 * st2 + 32 * (lane >> 5)) ^ kswz(lane)));
            const v8i Bl = load32(kt + (16 * sq + (lane & 15)) * S::PITCH + ((32 * (lane >> 4)) ^ kswz(16 * sq + (lane & 15))));
            const v4f dl = mfma_fp8_16x16x128(Alin, Bl, v4f{0.f, 0.f, 0.f, 0.f});
            v16f a0[2];
#pragma unroll
            for (int rf = 0; rf < 2; ++rf) a0[rf] = mfma_fp8_32x32x64(Q32f.a[rf][0], B[0][0], z);
#pragma unroll
            for (int rf = 0; rf < 2; ++rf) a0[rf] = mfma_fp8_32x32x64(Q32f.a[rf][1], B[0][1], a0[rf]);
            float p1 = epi32_abs(a1[0], a1[1], Q32f);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 10, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
            }
            keep_here(p1);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (kPipeTiles == 1) {
                // every wave holds block blk's operands: the tile takes block blk+1
                lds_barrier();
                stash1(0, kr[PAR ^ 1]);
            }
            // block blk-1's selection (none before block 0: a base past every position)
            const float lin_prev = linbuf[(PAR ^ 1) * (kPipeWaves * KB) + lin_get];
            const int bprev = __builtin_amdgcn_readfirstlane(blk) - 1;   // uniform: scalar arithmetic
            const bool need = select_binned(combine(p0_prev, p1) + lin_prev, bprev >= 0 ? bmap(bprev) * KB : Lk);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int rf = 0; rf < 2; ++rf) a1[rf] = mfma_fp8_32x32x64(Q32f.a[rf][0], B[1][0], z);
#pragma unroll
            for (int rf = 0; rf < 2; ++rf) a1[rf] = mfma_fp8_32x32x64(Q32f.a[rf][1], B[1][1], a1[rf]);
            p0_prev = epi32_abs(a0[0], a0[1], Q32f);
            // the four split terms, rescaled (exact powers of two) and summed
            const float lin = (((dl[3] * 0.0625f + dl[2]) * 0.0625f + dl[1]) * 0.0625f + dl[0]) * inv_s_lin;
            linbuf[PAR * (kPipeWaves * KB) + lin_put] = lin;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 9, 0);
            }
            keep_here(p0_prev);
            __builtin_amdgcn_sched_barrier(0);
            raise_flags(blk, need);
            // buffer PAR^1 last held block blk-1, read before the previous barrier
            if constexpr (kPipeTiles == 2) stash1(PAR ^ 1, kr[PAR ^ 1]);
            lds_barrier();
        };
        // unrolled by two: one copy of the body per register buffer of the staging loads
        for (int it = 0; it < niter; it += 2) {
            iter(std::integral_constant<int, 0>{}, it);
            compact_if_flagged(it);
            if (ns > 0 && it == ns) tau_step();
            if (it + 1 < niter) {
                iter(std::integral_constant<int, 1>{}, it + 1);
                compact_if_flagged(it + 1);
                if (ns > 0 && it + 1 == ns) tau_step();
            }
        }
        // the last block's fragment 1 and its selection (room for it was made
        // by the last iteration's compactions)
        (void)select_binned(combine(p0_prev, epi32_abs(a1[0], a1[1], Q32f)) + linbuf[((niter - 1) & 1) * (kPipeWaves * KB) + lin_get],
                            (nblk - 1) * KB);
        if (ns == 0) break;
        {
            const int i = i0 + wave;
            if (i < Lq && off + i + 1 > p.topk && st.cnt < p.topk && lane == 0) atomicOr(&flags[3], 1);
        }
        __syncthreads();
        const bool again = flags[3] != 0;
        __syncthreads();   // every wave has read the word
        if (!again) break;
        // sweep again without the sample, from empty buffers
        if (tid < 4) flags[tid] = 0;
        st.cnt = 0;
        st.thr = 0u;
        st.thr_f = -INFINITY;
        st.lo = 0u;
        seg_reset();
        ns = 0;
        __syncthreads();
        }
    } else {
    fetch(0);
    stash(0);
    // Every load issued so far (A fragments, head weights, block 0) has landed:
    // inside the loop only the next block's staging loads are in flight, and
    // the MFMAs never wait on them.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int blk = 0; blk < nblk; ++blk) {
        const int cur = blk & 1;
        if (blk + 1 < nblk) fetch(blk + 1);
        const int base = blk * KB;
        bool need = false;
        if (wave_has_rows && base <= wpmax) {
            const unsigned char *kt = ktile + (size_t)cur * KB * S::PITCH;
            float sc[TW];
            if constexpr (kMfma32) {
                sc[0] = score64_mfma32(Q32f, [&](int cf, int st) {
                    return load32(kt + (32 * cf + (lane & 31)) * S::PITCH + 64 * st + 32 * (lane >> 5));
                });
            } else if constexpr (!kStaged) {
                Frag<E, D> Bf[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) load_frag<E, D>(Bf[j], kt + (16 * j + n) * S::PITCH, g);
                v4f acc[4][4];
                // rows of fragment f all belong to query t = f * 16 / H
                float part[TW][4];
#pragma unroll
                for (int t = 0; t < TW; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j) part[t][j] = 0.f;
                // Software pipeline over the four sub-blocks: phase j issues the
                // MFMAs of sub-block j+1 interleaved (1 MFMA : 8 VALU) with the
                // epilogue of sub-block j, whose accumulators were produced a
                // whole phase earlier, so no VALU waits on an MFMA in flight.
#pragma unroll
                for (int f = 0; f < 4; ++f) acc[0][f] = frag_mma<E, D>(A[f], Bf[0]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (j + 1 < 4) {
#pragma unroll
                        for (int f = 0; f < 4; ++f) acc[j + 1][f] = frag_mma<E, D>(A[f], Bf[j + 1]);
                    }
                    float pf[4];
                    subblock_epilogue(acc[j], wv, pf);
#pragma unroll
                    for (int f = 0; f < 4; ++f) part[(16 * f) / H][j] += pf[f];
                    if (j + 1 < 4) {
#pragma unroll
                        for (int f = 0; f < 4; ++f) {
                            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int t = 0; t < TW; ++t) sc[t] = transpose_reduce4(part[t][0], part[t][1], part[t][2], part[t][3]);
            } else {
                Frag<E, D> Bf[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) load_frag<E, D>(Bf[j], kt + (16 * j + n) * S::PITCH, g);
                v4f acc[4][4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int f = 0; f < 4; ++f) acc[j][f] = frag_mma<E, D>(A[f], Bf[j]);
                // H = 4: lane group g holds all heads of query 4f+g;
                // H = 8: groups g and g^1 hold the two halves of query 2f+g/2.
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int f = 0; f < 4; ++f) {
                        float s = 0.f;
#pragma unroll
                        for (int ii = 0; ii < 4; ++ii) s += wv[f][ii] * relu(acc[j][f][ii]);
                        if constexpr (H == 8) {
                            s += shfl_xor(s, 16);
                            if ((g & 1) == 0) stage[(2 * f + (g >> 1)) * KB + 16 * j + n] = s;
                        } else {
                            stage[(4 * f + g) * KB + 16 * j + n] = s;
                        }
                    }
                wave_lds_sync();
#pragma unroll
                for (int t = 0; t < TW; ++t) sc[t] = stage[t * KB + lane];
                wave_lds_sync();
            }

            // selection
            if constexpr (kBinned) {
                need = select_binned(sc[0], base);
            } else {
#pragma unroll
                for (int t = 0; t < TW; ++t) {
                    const int i = i0 + wave * TW + t;
                    if (i >= Lq) continue;
                    const int pos = off + i;
                    if (base > pos) continue;
                    const int s = base + lane;
                    const int row = wave * TW + t;
                    if (kDbg && p.scores && s < Lk)
                        p.scores[(row0 + i) * Lk + s] = s <= pos ? sc[t] : -INFINITY;
                    int cnt = rcnt[row];
                    uint32_t thr = rthr[row];
                    const uint32_t key = score_key(sc[t]);
                    const bool cand = s <= pos && key > thr;
                    const uint64_t m = ballot(cand);
                    if (m) {
                        uint32_t *bk = bkey_all + (size_t)row * p.cap;
                        IdxT *bi = bidx_all + (size_t)row * p.cap;
                        const int at = cnt + lanes_below(m);
                        if (cand) { bk[at] = key; bi[at] = (IdxT)s; }
                        cnt += __popcll(m);
                        wave_lds_sync();
                        if (cnt > p.cap - KB) thr = select_compact<IdxT>(bk, bi, cnt, p.topk, hist, lane);
                        if (lane == 0) { rcnt[row] = cnt; rthr[row] = thr; }
                        wave_lds_sync();
                    }
                }
            }
        }
        raise_flags(blk, need);
        // The idle buffer was last read in block blk-1, which every wave has
        // left (barrier below); after this block's barrier it holds block blk+1.
        if (blk + 1 < nblk) stash(cur ^ 1);
        __syncthreads();
        compact_if_flagged(blk);
    }
    }

    // final selection and output
    for (int t = 0; t < TW; ++t) {
        const int i = i0 + wave * TW + t;
        if (i >= Lq) break;
        const int row = wave * TW + t;
        uint32_t *bk = bkey_all + (size_t)row * p.cap;
        IdxT *bi = bidx_all + (size_t)row * p.cap;
        int cnt = kBinned ? st.cnt : rcnt[row];
        if (cnt > p.topk) (void)select_compact<IdxT>(bk, bi, cnt, p.topk, hist, lane, nullptr, segs, nseg);
        int32_t *o = p.t_out + (row0 + i) * p.topk;
        for (int j = lane; j < p.topk; j += kWave) {
            int32_t v = -1;
            if (j < cnt) {
                v = (int32_t)bi[j];
                if (nseg > 1) {   // the index's segment: the last one starting at or before j
                    int sg = 0;
                    for (int b = 1; b < nseg; ++b) sg += segs[b] <= j ? 1 : 0;
                    v |= sg << 16;
                }
            }
            o[j] = v;
        }
        if (kDbg && p.scores) {
            const int pos = off + i;
            for (int s = (pos / KB + 1) * KB + lane; s < Lk; s += kWave)
                p.scores[(row0 + i) * Lk + s] = -INFINITY;
        }
    }
}

// ---------------------------------------------------------------- decode scores

struct ScoreParams {
    const unsigned char *q, *k;
    const void *w;
    float *scores;
    int B, Lq, Lk, split;
    Enc w_enc;
    // paged key cache (decode_scores_kernel<.., true>): k is the page pool
    // [num_blocks][block_size][row], block_table [B][max_blocks] maps a
    // sequence's key s to page block_table[b][s >> bs_log2], row s & (bs-1);
    // row_info [rows] gives each query row's (sequence, position); scores rows
    // are Lk apart (Lk = the longest sequence)
    const int32_t *block_table;
    const int2 *row_info;
    int bs_log2, max_blocks, num_blocks;
    // optional: each key range's top-k bound, bound[row][range] (split_bound)
    uint32_t *bound;
    int topk;
};

constexpr int kDecodeWaves = 4;
constexpr int kComputeUnits = 256;   // MI355X
// Score rows of key ranges up to this many keys are staged in LDS and written
// in one burst at the end of the workgroup (two workgroups per compute unit
// still fit): writes spread through the sweep cost far more than their bytes
// when they mix into the saturating read stream of the keys.
constexpr int kDecodeStageMaxKeys = 16384;

// 64 heads of one query against a contiguous key range; B operands are read
// straight from HBM (each key is used by exactly one query row here).
template <Enc E, int D, bool Paged, bool Stage = false>
__global__ __launch_bounds__(kDecodeWaves * kWave) __attribute__((amdgpu_waves_per_eu(2)))
void decode_scores_kernel(ScoreParams p) {
    using S = Shape<E, D>;
    constexpr int H = 64;
    __shared__ BoundShared bsh;
    extern __shared__ __align__(16) float sstage[];   // Stage: the range's scores
    uint32_t top[kLocal] = {0u, 0u, 0u, 0u};   // this thread's 4 largest keys (bound)
    const int tid = threadIdx.x, lane = tid % kWave, g = lane >> 4, n = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int row = blockIdx.y;
    int b, pos;
    if constexpr (Paged) {
        const int2 ri = p.row_info[row];
        b = __builtin_amdgcn_readfirstlane(ri.x);
        pos = __builtin_amdgcn_readfirstlane(ri.y);
    } else {
        b = row / p.Lq;
        pos = p.Lk - p.Lq + row % p.Lq;
    }
    const int s0 = blockIdx.x * p.split;
    const int s1 = min(s0 + p.split, p.Lk);
    float *out = p.scores + (size_t)row * p.Lk;
    // the key range's bound from every thread's top keys (whole block)
    auto write_bound = [&]() {
        if (!p.bound) return;
        const uint32_t bd = split_bound<kDecodeWaves * kWave>(bsh, top, pos + 1, p.split, (int)blockIdx.x, p.topk);
        if (threadIdx.x == 0) p.bound[(size_t)blockIdx.y * gridDim.x + blockIdx.x] = bd;
    };

    constexpr bool kMfma32 = E == Enc::FP8 && D == 128;
    Frag<E, D> A[4];
    float wv[4][4];
    Q32 Q32f;
    if constexpr (kMfma32) {
        load_q32(Q32f, p.q + (size_t)row * H * S::ROWB,
                 [&](int h) { return load_w(p.w, p.w_enc, (size_t)row * H + h); }, lane);
    } else {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            load_frag<E, D>(A[f], p.q + ((size_t)row * H + 16 * f + n) * S::ROWB, g);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) wv[f][ii] = load_w(p.w, p.w_enc, (size_t)row * H + 16 * f + 4 * g + ii);
        }
    }
    const unsigned char *kb = p.k + (size_t)b * p.Lk * S::ROWB;
    // paged: address of key s of this row's sequence (s <= pos); pages are
    // clamped to the pool so that no table value can address outside it
    // (the table is read through the constant address space: its loads are
    // uniform and go through the scalar cache, off the vector-memory counter
    // that the key loads are waited on)
    const __attribute__((address_space(4))) int32_t *bt =
        Paged ? (const __attribute__((address_space(4))) int32_t *)(p.block_table + (size_t)b * p.max_blocks) : nullptr;
    auto page_base = [&](int s) -> const unsigned char * {
        const int pg = min(max(bt[s >> p.bs_log2], 0), p.num_blocks - 1);
        return p.k + (((size_t)pg << p.bs_log2) + (s & ((1 << p.bs_log2) - 1))) * S::ROWB;
    };
    if constexpr (kMfma32) {
        // the keys of the next two blocks are loaded while the current one is
        // scored (three register buffers used in turn, so that no loaded value
        // is moved before use): two blocks (16 KB) of loads stay in flight per
        // wavefront through the scoring.  The prefetch is unconditional,
        // clamped to the last key, so that every iteration issues the same
        // loads and the compiler's waits stay exact.
        constexpr int STRIDE = kDecodeWaves * KB;
        // paged: a 64-key block lies in one page (pages hold a multiple of 64
        // keys); past the last valid key the last valid block is read again.
        // The page of a block is looked up (scalar load) one block before its
        // keys are loaded.
        auto block_page = [&](int base) -> const unsigned char * {
            if constexpr (Paged) return page_base(min(base, pos) & ~(KB - 1));
            else return nullptr;
        };
        auto load_block = [&](v8i (&B)[2][2], int base, const unsigned char *pb) {
            if constexpr (Paged) {
#pragma unroll
                for (int cf = 0; cf < 2; ++cf)
#pragma unroll
                    for (int st = 0; st < 2; ++st)
                        B[cf][st] = load32(pb + (size_t)(32 * cf + (lane & 31)) * S::ROWB + 64 * st + 32 * (lane >> 5));
            } else {
#pragma unroll
                for (int cf = 0; cf < 2; ++cf) {
                    const int key = min(base + 32 * cf + (lane & 31), p.Lk - 1);
#pragma unroll
                    for (int st = 0; st < 2; ++st) B[cf][st] = load32(kb + (size_t)key * S::ROWB + 64 * st + 32 * (lane >> 5));
                }
            }
        };
        auto put = [&](int s, float v) {   // s < s1
            if constexpr (Stage) sstage[s - s0] = v;
            else out[s] = v;
        };
        auto score_block = [&](const v8i (&B)[2][2], int base) {
            const float sc = score64_mfma32_b(Q32f, B);
            const int s = base + lane;
            if (s < s1) put(s, s <= pos ? sc : -INFINITY);
            if (s < s1 && s <= pos) keep_top4(top, score_key(sc));
        };
        const int last = min(s1, pos + 1);        // keys at or before the query position
        int base = s0 + wave * KB;
        if (base < last) {
            v8i B0[2][2], B1[2][2], B2[2][2];
            load_block(B0, base, block_page(base));
            load_block(B1, base + STRIDE, block_page(base + STRIDE));
            const unsigned char *pg = block_page(base + 2 * STRIDE);
            for (;;) {
                load_block(B2, base + 2 * STRIDE, pg);
                pg = block_page(base + 3 * STRIDE);
                score_block(B0, base);
                base += STRIDE;
                if (base >= last) break;
                load_block(B0, base + 2 * STRIDE, pg);
                pg = block_page(base + 3 * STRIDE);
                score_block(B1, base);
                base += STRIDE;
                if (base >= last) break;
                load_block(B1, base + 2 * STRIDE, pg);
                pg = block_page(base + 3 * STRIDE);
                score_block(B2, base);
                base += STRIDE;
                if (base >= last) break;
            }
        }
        for (; base < s1; base += STRIDE) {
            const int s = base + lane;
            if (s < s1) put(s, -INFINITY);
        }
        if constexpr (Stage) {
            // one burst of 16-byte stores (the score row stride and s0 are
            // multiples of 4 floats when staging is chosen)
            __syncthreads();
            const int len = s1 - s0;
            for (int i = 4 * (int)threadIdx.x; i < len; i += 4 * kDecodeWaves * kWave) {
                if (i + 4 <= len) *reinterpret_cast<v4f *>(out + s0 + i) = *reinterpret_cast<const v4f *>(sstage + i);
                else
                    for (int e = i; e < len; ++e) out[s0 + e] = sstage[e];
            }
        }
        write_bound();
        return;
    }
    for (int base = s0 + wave * KB; base < s1; base += kDecodeWaves * KB) {
        const int s = base + lane;
        if (base > pos) {
            if (s < s1) out[s] = -INFINITY;
            continue;
        }
        Frag<E, D> Bf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int key = base + 16 * j + n;
            if constexpr (Paged) {
                if (key <= pos) load_frag<E, D>(Bf[j], page_base(key), g);
                else zero_frag<E, D>(Bf[j]);
            } else {
                if (key < p.Lk) load_frag<E, D>(Bf[j], kb + (size_t)key * S::ROWB, g);
                else zero_frag<E, D>(Bf[j]);
            }
        }
        float part[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v4f a[4];
#pragma unroll
            for (int f = 0; f < 4; ++f) a[f] = frag_mma<E, D>(A[f], Bf[j]);
            float pf[4];
            subblock_epilogue(a, wv, pf);
            part[j] = 0.f;
#pragma unroll
            for (int f = 0; f < 4; ++f) part[j] += pf[f];
        }
        const float sc = transpose_reduce4(part[0], part[1], part[2], part[3]);
        if (s < s1) out[s] = s <= pos ? sc : -INFINITY;
        if (s < s1 && s <= pos) keep_top4(top, score_key(sc));
    }
    write_bound();
}

template <Enc E, int D, int H, typename IdxT, bool Paged, int Var>
hipError_t launch_prefill_v(const IndexerArgs &a, int waves, int cap, size_t lds, hipStream_t st,
                            const PagedPrefill *pp) {
    auto kern = prefill_kernel<E, D, H, IdxT, Paged, Var>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    PrefillParams p = {};
    p.q = static_cast<const unsigned char *>(a.q);
    p.k = static_cast<const unsigned char *>(a.k);
    p.w = a.w;
    p.t_out = a.t_out;
    p.scores = a.scores;
    p.B = a.B; p.Lq = a.Lq; p.Lk = a.Lk; p.topk = a.topk; p.cap = cap;
    p.nthreads = waves * kWave;
    p.w_enc = a.w_enc;
    const int R = waves * (64 / H);
    unsigned grid;
    if constexpr (Paged) {
        p.query_start = pp->query_start;
        p.seq_lens = pp->seq_lens;
        p.block_table = pp->block_table;
        p.rb_start = pp->rb_start;
        p.num_seqs = pp->num_seqs;
        p.bs_log2 = pp->bs_log2;
        p.max_blocks = pp->max_blocks;
        p.num_blocks = pp->num_blocks;
        // at most ceil(q_len / R) <= q_len / R + 1 row blocks per sequence
        grid = (unsigned)((pp->total_q + R - 1) / R + pp->num_seqs);
    } else {
        grid = (unsigned)(((a.Lq + R - 1) / R) * a.B);
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(waves * kWave), lds, st, p);
    return hipGetLastError();
}

// The pipelined sweep (fp8, 64 heads, 128 dims, 16-bit candidates) comes in
// four variants (score row for tests or not, keys past 65,536 or not); the
// other kernels keep one body that checks both at run time.
template <Enc E, int D, int H, typename IdxT, bool Paged = false>
hipError_t launch_prefill_t(const IndexerArgs &a, int waves, int cap, size_t lds, hipStream_t st,
                            const PagedPrefill *pp = nullptr) {
    if constexpr (E == Enc::FP8 && D == 128 && H == 64 && sizeof(IdxT) == 2) {
        const int var = (a.scores ? 1 : 0) | (a.Lk > 65536 ? 2 : 0);
        switch (var) {
        case 0: return launch_prefill_v<E, D, H, IdxT, Paged, 0>(a, waves, cap, lds, st, pp);
        case 1: return launch_prefill_v<E, D, H, IdxT, Paged, 1>(a, waves, cap, lds, st, pp);
        case 2: return launch_prefill_v<E, D, H, IdxT, Paged, 2>(a, waves, cap, lds, st, pp);
        default: return launch_prefill_v<E, D, H, IdxT, Paged, 3>(a, waves, cap, lds, st, pp);
        }
    } else {
        return launch_prefill_v<E, D, H, IdxT, Paged, 3>(a, waves, cap, lds, st, pp);
    }
}

struct PrefillPlan {
    int waves, cap, idx_bytes;
    size_t lds;
    bool ok;
};

constexpr size_t kLdsBudget = 160 * 1024;

PrefillPlan plan_prefill(const IndexerArgs &a) {
    PrefillPlan pl{0, 0, 0, 0, false};
    const int eb = a.qk_enc == Enc::FP8 ? 1 : 2;
    const int rowb = a.D * eb, pitch = rowb + 16;
    const int tw = 64 / a.H;
    const bool staged = a.H < 16;
    // 16-bit candidate indices: keys up to 65536, or (pipelined 64-head fp8
    // sweep, with its segment table) up to kMaxSeg * 65536
    const bool mfma32 = a.qk_enc == Enc::FP8 && a.H == 64 && a.D == 128;
    pl.idx_bytes = a.Lk <= 65536 || (mfma32 && (long long)a.Lk <= (long long)kMaxSeg * 65536) ? 2 : 4;
    const bool pipe = mfma32 && pl.idx_bytes == 2;
    const int stage_bufs = staged ? 1 : pipe ? 2 : 0;
    const int nchunk = KB * rowb / 16;
    int min_waves = (nchunk + kChunkMax * kWave - 1) / (kChunkMax * kWave);
    if (min_waves < 1) min_waves = 1;
    // the pipelined sweep runs kPipeWaves wavefronts per workgroup and
    // kPipeGroupsPerCU workgroups per compute unit, which share its LDS
    const int top_waves = pipe ? kPipeWaves : 8;
    if (pipe) min_waves = kPipeWaves;
    const size_t budget = pipe ? kLdsBudget / kPipeGroupsPerCU : kLdsBudget;
    for (int waves = top_waves; waves >= min_waves; waves /= 2) {
        // room beyond k: at least two blocks of appends; more room means fewer
        // compactions per row.  Take the most LDS allows (multiple of 64, <= 2048).
        const int ktiles = pipe ? kPipeTiles : 2;
        const PrefillLds base = prefill_lds(waves, tw, pitch, 0, pl.idx_bytes, stage_bufs, ktiles);
        if (base.total + 64 > budget) {
            if (waves == 1) break;
            continue;
        }
        const size_t per_entry = (size_t)waves * tw * (4 + pl.idx_bytes);
        long cap = (long)((budget - base.total - 32) / per_entry);
        cap = (cap / KB) * KB;
        if (cap > a.topk + 2048) cap = ((a.topk + 2048) / KB) * KB;
        if (cap >= a.topk + 2 * KB) {
            pl.waves = waves;
            pl.cap = (int)cap;
            pl.lds = prefill_lds(waves, tw, pitch, pl.cap, pl.idx_bytes, stage_bufs, ktiles).total;
            pl.ok = pl.lds <= budget;
            if (pl.ok) return pl;
        }
        if (waves == 1) break;
    }
    return pl;
}

template <Enc E, int D, int H>
hipError_t launch_prefill_h(const IndexerArgs &a, hipStream_t st) {
    const PrefillPlan pl = plan_prefill(a);
    if (!pl.ok) return hipErrorInvalidConfiguration;
    // the 64-head fp8 kernel with 16-bit indices runs its pipelined sweep with
    // exactly kPipeWaves wavefronts
    if (E == Enc::FP8 && H == 64 && D == 128 && pl.idx_bytes == 2 && pl.waves != kPipeWaves)
        return hipErrorInvalidConfiguration;
    if (pl.idx_bytes == 2) return launch_prefill_t<E, D, H, uint16_t>(a, pl.waves, pl.cap, pl.lds, st);
    return launch_prefill_t<E, D, H, uint32_t>(a, pl.waves, pl.cap, pl.lds, st);
}

template <Enc E, int D>
hipError_t launch_prefill_d(const IndexerArgs &a, hipStream_t st) {
    switch (a.H) {
    case 4: return launch_prefill_h<E, D, 4>(a, st);
    case 8: return launch_prefill_h<E, D, 8>(a, st);
    case 16: return launch_prefill_h<E, D, 16>(a, st);
    case 32: return launch_prefill_h<E, D, 32>(a, st);
    case 64: return launch_prefill_h<E, D, 64>(a, st);
    default: return hipErrorInvalidValue;
    }
}

template <Enc E, int D>
hipError_t launch_decode_d(const IndexerArgs &a, hipStream_t st, const PagedKeys *pk = nullptr) {
    ScoreParams p;
    p.q = static_cast<const unsigned char *>(a.q);
    p.k = static_cast<const unsigned char *>(a.k);
    p.w = a.w;
    p.scores = a.scores;
    p.B = a.B; p.Lq = a.Lq; p.Lk = a.Lk;
    p.w_enc = a.w_enc;
    // one round of workgroups: two per compute unit (the kernel's register
    // use allows two resident), each a contiguous key range of a multiple of
    // 256 keys (one 64-key block per wavefront and iteration)
    int nsplit;
    decode_split_geometry(a, &nsplit, &p.split);
    p.bound = a.split_bound;
    p.topk = a.topk;
    if constexpr (E == Enc::FP8 && D == 128) {
        if (p.split <= kDecodeStageMaxKeys && a.Lk % 4 == 0) {
            const size_t lds = (size_t)p.split * sizeof(float);
            if (pk) {
                p.block_table = pk->block_table;
                p.row_info = reinterpret_cast<const int2 *>(pk->row_info);
                p.bs_log2 = pk->bs_log2;
                p.max_blocks = pk->max_blocks;
                p.num_blocks = pk->num_blocks;
                auto kern = decode_scores_kernel<E, D, true, true>;
                hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
                if (e != hipSuccess) return e;
                hipLaunchKernelGGL(kern, dim3((unsigned)nsplit, (unsigned)(a.B * a.Lq)), dim3(kDecodeWaves * kWave), lds, st, p);
            } else {
                p.block_table = nullptr;
                p.row_info = nullptr;
                p.bs_log2 = p.max_blocks = p.num_blocks = 0;
                auto kern = decode_scores_kernel<E, D, false, true>;
                hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
                if (e != hipSuccess) return e;
                hipLaunchKernelGGL(kern, dim3((unsigned)nsplit, (unsigned)(a.B * a.Lq)), dim3(kDecodeWaves * kWave), lds, st, p);
            }
            return hipGetLastError();
        }
    }
    if (pk) {
        p.block_table = pk->block_table;
        p.row_info = reinterpret_cast<const int2 *>(pk->row_info);
        p.bs_log2 = pk->bs_log2;
        p.max_blocks = pk->max_blocks;
        p.num_blocks = pk->num_blocks;
        hipLaunchKernelGGL((decode_scores_kernel<E, D, true>), dim3((unsigned)nsplit, (unsigned)(a.B * a.Lq)),
                           dim3(kDecodeWaves * kWave), 0, st, p);
    } else {
        p.block_table = nullptr;
        p.row_info = nullptr;
        p.bs_log2 = p.max_blocks = p.num_blocks = 0;
        hipLaunchKernelGGL((decode_scores_kernel<E, D, false>), dim3((unsigned)nsplit, (unsigned)(a.B * a.Lq)),
                           dim3(kDecodeWaves * kWave), 0, st, p);
    }
    return hipGetLastError();
}

}  // namespace

bool prefill_fits(const IndexerArgs &a) { return plan_prefill(a).ok; }

int prefill_rows_per_workgroup(const IndexerArgs &a) {
    const PrefillPlan pl = plan_prefill(a);
    return pl.ok ? pl.waves * (64 / a.H) : 0;
}

bool paged_prefill_supported(const IndexerArgs &a) {
    return a.qk_enc == Enc::FP8 && a.D == 128 && a.H == 64 && prefill_fits(a);
}

hipError_t launch_indexer_prefill_paged(const IndexerArgs &a, const PagedPrefill &pp, hipStream_t st) {
    if (!paged_prefill_supported(a)) return hipErrorInvalidValue;
    const PrefillPlan pl = plan_prefill(a);
    if (pl.idx_bytes == 2) {
        if (pl.waves != kPipeWaves) return hipErrorInvalidConfiguration;
        return launch_prefill_t<Enc::FP8, 128, 64, uint16_t, true>(a, pl.waves, pl.cap, pl.lds, st, &pp);
    }
    return launch_prefill_t<Enc::FP8, 128, 64, uint32_t, true>(a, pl.waves, pl.cap, pl.lds, st, &pp);
}

hipError_t launch_indexer_prefill(const IndexerArgs &a, hipStream_t st) {
    if (a.qk_enc == Enc::FP8) {
        if (a.D == 128) return launch_prefill_d<Enc::FP8, 128>(a, st);
    } else if (a.qk_enc == Enc::BF16) {
        if (a.D == 32) return launch_prefill_d<Enc::BF16, 32>(a, st);
        if (a.D == 64) return launch_prefill_d<Enc::BF16, 64>(a, st);
        if (a.D == 128) return launch_prefill_d<Enc::BF16, 128>(a, st);
    }
    return hipErrorInvalidValue;
}

void decode_split_geometry(const IndexerArgs &a, int *nsplit, int *split) {
    const int rows = a.B * a.Lq;
    const int max_split = (a.Lk + 255) / 256;
    const int want = std::max(1, std::min(max_split, (2 * kComputeUnits + rows - 1) / rows));
    *split = ((a.Lk + want - 1) / want + 255) / 256 * 256;
    *nsplit = (a.Lk + *split - 1) / *split;
}

bool decode_supported(const IndexerArgs &a) {
    if (a.H != 64) return false;
    if (a.qk_enc == Enc::FP8) return a.D == 128;
    return a.D == 32 || a.D == 64 || a.D == 128;
}

hipError_t launch_indexer_scores(const IndexerArgs &a, hipStream_t st, const PagedKeys *pk) {
    if (a.qk_enc == Enc::FP8) {
        if (a.D == 128) return launch_decode_d<Enc::FP8, 128>(a, st, pk);
    } else if (a.qk_enc == Enc::BF16) {
        if (a.D == 32) return launch_decode_d<Enc::BF16, 32>(a, st, pk);
        if (a.D == 64) return launch_decode_d<Enc::BF16, 64>(a, st, pk);
        if (a.D == 128) return launch_decode_d<Enc::BF16, 128>(a, st, pk);
    }
    return hipErrorInvalidValue;
}

}  // namespace idxc
