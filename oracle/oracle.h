/*
 * oracle.h -- plain, slow CPU reference for the lightning indexer, its top-k,
 * the IndexCache routing rule and sparse MLA attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; the product path never calls it.
 *
 * Sources (cited by page title and section; the pages are web articles):
 *   [ITO]  itoverdose.com, "IndexCache: Wie DeepSeek O(NL²)-Kosten in Sparse
 *          Attention um 75% reduziert"
 *   [PPM]  parapluman.nl, Dutch article on IndexCache (sections "Het
 *          DSA-knelpunt", "Aandacht cachen met IndexCache")
 *   [AIB]  aiboss88.com, "IndexCache - 清華大学とZhipuが共同開発した、
 *          スパースアテンション高速化技術。 - AiBoss"
 *
 * All arithmetic is fp64; results are rounded once to the output type.
 */
#ifndef IDX_ORACLE_H
#define IDX_ORACLE_H
#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* input element encodings understood by the oracle */
enum { OR_BF16 = 1, OR_FP8_E4M3 = 2, OR_FP32 = 3 };

/* Exact decode of one element (OCP fp8 e4m3fn, bf16 or fp32) to double. */
double or_decode(int dtype, const void *base, size_t idx);

/* Round a double to fp32 (round-to-nearest-even). */
float or_round_f32(double x);

/* Round a double to bf16 bits (round-to-nearest-even, one rounding). */
uint16_t or_round_bf16(double x);

/*
 * Indexer scores for selected query rows.
 * q [B,Lq,H,D], k [B,Lk,D], w [B,Lq,H] in the given encodings.
 * rows[r] is a flat query row b*Lq+i; its position is p = Lk-Lq+i.
 * out [nrows, Lk] fp32: I[s] = sum_h w[h]*max(0, q[h].k[s]) for s <= p,
 * computed in double and rounded once to fp32 (-0 canonicalised to +0);
 * s > p holds -inf.
 */
int or_indexer_scores(int B, int Lq, int Lk, int H, int D,
                      int q_dtype, int k_dtype, int w_dtype,
                      const void *q, const void *k, const void *w,
                      int nrows, const int64_t *rows, float *out, int nthreads);

/*
 * Row top-k over fp32 scores.
 * scores [nrows, Lk]; pos[r] = last valid key index of row r (keys 0..pos[r]).
 * out [nrows, topk] int32: if pos+1 <= topk, 0..pos then -1 padding;
 * otherwise the topk keys largest by (score desc, index asc), emitted in
 * ascending index order.
 */
int or_topk(int nrows, int Lk, const float *scores, const int32_t *pos,
            int topk, int32_t *out, int nthreads);

/*
 * Sparse MLA attention (absorbed MLA / MQA over one shared latent row).
 * q bf16 [B,Lq,Hq,Dqk], kv bf16 [B,Lk,Dqk], t int32 [B,Lq,topk] (-1 = unused).
 * Only the flat query rows listed in rows[] are computed.
 * out bf16 [nrows, Hq, Dv]  (V = kv[..., :Dv]);  lse fp32 [nrows, Hq].
 * A row with no valid index yields O = 0 and lse = -inf.
 */
int or_sparse_mla(int B, int Lq, int Lk, int Hq, int Dqk, int Dv, int topk,
                  const uint16_t *q, const uint16_t *kv, const int32_t *t,
                  float sm_scale, int nrows, const int64_t *rows,
                  uint16_t *out, float *lse, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
