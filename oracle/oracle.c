/*
 * oracle.c -- plain fp64 CPU reference (TEST INFRASTRUCTURE ONLY).
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg load
 * this file's library.  It shares no code with the HIP path.  Every function
 * is the plain definition of what it computes: no blocking, no fusion, no
 * reordering beyond what the definition states.  Source legend in oracle.h.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ codecs */

/* OCP fp8 e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinity;
 * S.1111.111 is NaN; exponent field 0 encodes subnormals m/8 * 2^-6. */
static double dec_fp8_e4m3(uint8_t b) {
    int sign = (b >> 7) & 1;
    int e = (b >> 3) & 0xF;
    int m = b & 7;
    double v;
    if (e == 0xF && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);              /* (m/8) * 2^-6 */
    else v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

static double dec_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

double or_decode(int dtype, const void *base, size_t idx) {
    switch (dtype) {
    case OR_FP8_E4M3: return dec_fp8_e4m3(((const uint8_t *)base)[idx]);
    case OR_BF16: return dec_bf16(((const uint16_t *)base)[idx]);
    case OR_FP32: return (double)((const float *)base)[idx];
    default: return NAN;
    }
}

float or_round_f32(double x) { return (float)x; /* C conversion: nearest-even */ }

/* bf16 keeps 8 significant bits and fp32's exponent range.  Round x once:
 * normal range  -> nearbyint(x * 2^(8-e)) * 2^(e-8) with x = f*2^e, f in [.5,1)
 * subnormal     -> nearbyint(x * 2^133) * 2^-133 (spacing of bf16 subnormals). */
uint16_t or_round_bf16(double x) {
    if (isnan(x)) return 0x7FC0;
    double r;
    if (x == 0.0) {
        r = x;
    } else {
        int e;
        (void)frexp(x, &e);
        if (e - 1 >= -126) r = ldexp(nearbyint(ldexp(x, 8 - e)), e - 8);
        else r = ldexp(nearbyint(ldexp(x, 133)), -133);
    }
    float f = (float)r; /* exact: r is a bf16 value, or overflows to inf */
    if (fabs(r) >= ldexp(1.0, 128)) f = r > 0 ? INFINITY : -INFINITY;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------ thread pool */

typedef void (*row_fn)(void *ctx, int r);
typedef struct { row_fn fn; void *ctx; int n; int next; pthread_mutex_t mu; } par_t;

static void *par_worker(void *arg) {
    par_t *p = (par_t *)arg;
    for (;;) {
        pthread_mutex_lock(&p->mu);
        int r = p->next++;
        pthread_mutex_unlock(&p->mu);
        if (r >= p->n) break;
        p->fn(p->ctx, r);
    }
    return NULL;
}

static void par_for(int n, int nthreads, row_fn fn, void *ctx) {
    par_t p;
    p.fn = fn; p.ctx = ctx; p.n = n; p.next = 0;
    pthread_mutex_init(&p.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > n) nthreads = n > 0 ? n : 1;
    pthread_t th[256];
    int started = 0;
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[started], NULL, par_worker, &p) == 0) ++started;
    par_worker(&p);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&p.mu);
}

/* ------------------------------------------------------------ indexer */

/* [ITO] § "Wie der Indexer funktioniert und warum MLA entscheidend ist" and
 * [PPM] § "Het DSA-knelpunt": every preceding token s of query t gets a
 * score; scores pass through a ReLU before the top-k.  With H indexer heads
 * the score is I[t,s] = sum_h w[t,h] * max(0, q[t,h,:] . k[s,:]). */
typedef struct {
    int B, Lq, Lk, H, D, qdt, kdt, wdt;
    const void *q, *k, *w;
    const int64_t *rows;
    float *out;
} scores_ctx;

static void scores_row(void *vctx, int r) {
    scores_ctx *c = (scores_ctx *)vctx;
    int64_t flat = c->rows[r];
    int b = (int)(flat / c->Lq), i = (int)(flat % c->Lq);
    int p = c->Lk - c->Lq + i;                /* causal position of the query */
    int H = c->H, D = c->D;
    double *qd = (double *)malloc(sizeof(double) * (size_t)H * D);
    double *wd = (double *)malloc(sizeof(double) * (size_t)H);
    double *kd = (double *)malloc(sizeof(double) * (size_t)D);
    for (int h = 0; h < H; ++h) {
        wd[h] = or_decode(c->wdt, c->w, (size_t)flat * H + h);
        for (int d = 0; d < D; ++d)
            qd[h * D + d] = or_decode(c->qdt, c->q, ((size_t)flat * H + h) * D + d);
    }
    float *o = c->out + (size_t)r * c->Lk;
    for (int s = 0; s < c->Lk; ++s) {
        if (s > p) { o[s] = -INFINITY; continue; }
        for (int d = 0; d < D; ++d)
            kd[d] = or_decode(c->kdt, c->k, ((size_t)b * c->Lk + s) * D + d);
        double acc = 0.0;
        for (int h = 0; h < H; ++h) {
            double dot = 0.0;
            for (int d = 0; d < D; ++d) dot += qd[h * D + d] * kd[d];
            double relu = dot > 0.0 ? dot : 0.0;
            acc += wd[h] * relu;
        }
        float f = or_round_f32(acc);
        if (f == 0.0f) f = 0.0f;              /* -0 and +0 are the same score */
        o[s] = f;
    }
    free(qd); free(wd); free(kd);
}

int or_indexer_scores(int B, int Lq, int Lk, int H, int D, int q_dtype, int k_dtype,
                      int w_dtype, const void *q, const void *k, const void *w, int nrows,
                      const int64_t *rows, float *out, int nthreads) {
    if (B < 1 || Lq < 1 || Lk < Lq || H < 1 || D < 1 || !q || !k || !w || !out || nrows < 0)
        return -1;
    for (int r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= (int64_t)B * Lq) return -2;
    scores_ctx c = {B, Lq, Lk, H, D, q_dtype, k_dtype, w_dtype, q, k, w, rows, out};
    par_for(nrows, nthreads, scores_row, &c);
    return 0;
}

/* ------------------------------------------------------------ top-k */

/* [ITO] § "Einfache Implementierung, enorme Effizienzgewinne": the index set
 * is the top-k of the row's scores.  Ties go to the lower key index; the
 * set is emitted in ascending index order. */
typedef struct { float score; int32_t idx; } cand_t;

static int cand_cmp(const void *a, const void *b) {
    const cand_t *x = (const cand_t *)a, *y = (const cand_t *)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->idx > y->idx) - (x->idx < y->idx);
}

static int int_cmp(const void *a, const void *b) {
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

typedef struct {
    int Lk, topk;
    const float *scores;
    const int32_t *pos;
    int32_t *out;
} topk_ctx;

static void topk_row(void *vctx, int r) {
    topk_ctx *c = (topk_ctx *)vctx;
    int p = c->pos ? c->pos[r] : c->Lk - 1;
    int n = p + 1;
    int32_t *o = c->out + (size_t)r * c->topk;
    if (n <= 0) {
        for (int j = 0; j < c->topk; ++j) o[j] = -1;
        return;
    }
    if (n <= c->topk) {
        for (int j = 0; j < c->topk; ++j) o[j] = j < n ? j : -1;
        return;
    }
    const float *s = c->scores + (size_t)r * c->Lk;
    cand_t *v = (cand_t *)malloc(sizeof(cand_t) * (size_t)n);
    for (int j = 0; j < n; ++j) {
        v[j].score = s[j] == 0.0f ? 0.0f : s[j];
        v[j].idx = j;
    }
    qsort(v, (size_t)n, sizeof(cand_t), cand_cmp);
    for (int j = 0; j < c->topk; ++j) o[j] = v[j].idx;
    qsort(o, (size_t)c->topk, sizeof(int32_t), int_cmp);
    free(v);
}

int or_topk(int nrows, int Lk, const float *scores, const int32_t *pos, int topk,
            int32_t *out, int nthreads) {
    if (nrows < 0 || Lk < 1 || topk < 1 || !scores || !out) return -1;
    if (pos)
        for (int r = 0; r < nrows; ++r)
            if (pos[r] >= Lk) return -2;
    topk_ctx c = {Lk, topk, scores, pos, out};
    par_for(nrows, nthreads, topk_row, &c);
    return 0;
}

/* ------------------------------------------------------------ sparse MLA */

/* [ITO] introduction and § "Wie der Indexer funktioniert und warum MLA
 * entscheidend ist": attention runs only over the k selected tokens, whose
 * keys and values live in one compressed latent row shared by all heads.
 * Softmax attention over the selected rows:
 *   z_j = scale * q[h,:Dqk] . kv[T_j,:Dqk],  O[h,:] = sum_j softmax(z)_j kv[T_j,:Dv]. */
typedef struct {
    int B, Lq, Lk, Hq, Dqk, Dv, topk;
    const uint16_t *q, *kv;
    const int32_t *t;
    double scale;
    const int64_t *rows;
    uint16_t *out;
    float *lse;
} mla_ctx;

static void mla_row(void *vctx, int r) {
    mla_ctx *c = (mla_ctx *)vctx;
    int64_t flat = c->rows[r];
    int b = (int)(flat / c->Lq);
    const int32_t *t = c->t + (size_t)flat * c->topk;
    int nvalid = 0;
    for (int j = 0; j < c->topk; ++j)
        if (t[j] >= 0) ++nvalid;
    double *z = (double *)malloc(sizeof(double) * (size_t)(nvalid > 0 ? nvalid : 1));
    int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nvalid > 0 ? nvalid : 1));
    double *acc = (double *)malloc(sizeof(double) * (size_t)c->Dv);
    int n = 0;
    for (int j = 0; j < c->topk; ++j)
        if (t[j] >= 0) sel[n++] = t[j];
    for (int h = 0; h < c->Hq; ++h) {
        const uint16_t *qh = c->q + ((size_t)flat * c->Hq + h) * c->Dqk;
        uint16_t *oh = c->out + ((size_t)r * c->Hq + h) * c->Dv;
        if (n == 0) {
            for (int d = 0; d < c->Dv; ++d) oh[d] = 0;
            if (c->lse) c->lse[(size_t)r * c->Hq + h] = -INFINITY;
            continue;
        }
        double m = -INFINITY;
        for (int j = 0; j < n; ++j) {
            const uint16_t *kr = c->kv + ((size_t)b * c->Lk + sel[j]) * c->Dqk;
            double dot = 0.0;
            for (int d = 0; d < c->Dqk; ++d) dot += dec_bf16(qh[d]) * dec_bf16(kr[d]);
            z[j] = c->scale * dot;
            if (z[j] > m) m = z[j];
        }
        double l = 0.0;
        for (int d = 0; d < c->Dv; ++d) acc[d] = 0.0;
        for (int j = 0; j < n; ++j) {
            double e = exp(z[j] - m);
            l += e;
            const uint16_t *vr = c->kv + ((size_t)b * c->Lk + sel[j]) * c->Dqk;
            for (int d = 0; d < c->Dv; ++d) acc[d] += e * dec_bf16(vr[d]);
        }
        for (int d = 0; d < c->Dv; ++d) oh[d] = or_round_bf16(acc[d] / l);
        if (c->lse) c->lse[(size_t)r * c->Hq + h] = or_round_f32(m + log(l));
    }
    free(z); free(sel); free(acc);
}

int or_sparse_mla(int B, int Lq, int Lk, int Hq, int Dqk, int Dv, int topk,
                  const uint16_t *q, const uint16_t *kv, const int32_t *t, float sm_scale,
                  int nrows, const int64_t *rows, uint16_t *out, float *lse, int nthreads) {
    if (B < 1 || Lq < 1 || Lk < 1 || Hq < 1 || Dqk < 1 || Dv < 1 || Dv > Dqk || topk < 1 ||
        !q || !kv || !t || !out || nrows < 0)
        return -1;
    for (int r = 0; r < nrows; ++r) {
        if (rows[r] < 0 || rows[r] >= (int64_t)B * Lq) return -2;
        const int32_t *tr = t + (size_t)rows[r] * topk;
        for (int j = 0; j < topk; ++j)
            if (tr[j] >= Lk) return -3;
    }
    mla_ctx c = {B, Lq, Lk, Hq, Dqk, Dv, topk, q, kv, t, (double)sm_scale, rows, out, lse};
    par_for(nrows, nthreads, mla_row, &c);
    return 0;
}
