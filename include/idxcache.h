/*
 * idxcache.h -- C ABI of libidxcache.so: the DeepSeek-Sparse-Attention lightning
 * indexer with its per-row top-k, the IndexCache Full/Shared layer router, and
 * sparse MLA attention over the selected latent rows, for AMD MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *   [ITO] itoverdose.com, "IndexCache: Wie DeepSeek O(NL²)-Kosten in Sparse
 *         Attention um 75% reduziert"
 *   [PPM] parapluman.nl, Dutch article on IndexCache, sections "Het DSA-knelpunt",
 *         "Aandacht cachen met IndexCache", "Real-world versnellingen op
 *         productiemodellen" and "IndexCache in productie brengen"
 *   [AIB] aiboss88.com, "IndexCache - 清華大学とZhipuが共同開発した、
 *         スパースアテンション高速化技術。 - AiBoss", sections "IndexCacheの主な機能"
 *         and the comparison table "IndexCacheと類似の競合製品との比較"
 *   [SAI] setupai.cc, "IndexCache 加速長上下文推理 1.82 倍", comparison table
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or synchronises.  Scratch memory is passed in as a
 *     workspace whose size the matching *_workspace() call reports.
 *   - Tensors are dense, contiguous, row-major, in the shapes given below.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously on it; results are ready after the
 *     caller synchronises that stream.
 *   - Every argument is validated on the host before any HIP call; a failed
 *     check returns an error code and enqueues nothing.  Launch failures are
 *     reported as IDXC_ERR_HIP.  Faults inside kernels surface at the
 *     caller's next synchronisation.  No call aborts or throws.
 *   - Calls keep no state between invocations and may run concurrently on
 *     different streams with different buffers.
 */
#ifndef IDXCACHE_H
#define IDXCACHE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IDXC_ABI_VERSION 1

typedef enum {
    IDXC_OK = 0,
    IDXC_ERR_NULL = -1,        /* a required pointer is NULL */
    IDXC_ERR_SHAPE = -2,       /* a size is out of range or sizes disagree */
    IDXC_ERR_DTYPE = -3,       /* unknown encoding or unsupported encoding combination */
    IDXC_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
    IDXC_ERR_UNSUPPORTED = -5, /* valid request that no kernel of the library serves */
    IDXC_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than required */
    IDXC_ERR_PATTERN = -7,     /* layer pattern invalid (see idx_cache_route) */
    IDXC_ERR_HIP = -8,         /* the HIP runtime reported an error at launch */
    IDXC_ERR_SCRATCH = -9      /* idx_score_topk_noalloc: the request needs more than
                                  the library's static scratch (128 MiB per GPU) */
} idxc_status;

typedef enum {
    IDXC_BF16 = 1,
    IDXC_FP8_E4M3 = 2, /* OCP e4m3fn: bias 7, no infinity, max 448 */
    IDXC_FP32 = 3
} idxc_dtype;

/*
 * Lightning indexer problem ([ITO] § "Wie der Indexer funktioniert und warum MLA
 * entscheidend ist"; [PPM] § "Het DSA-knelpunt"):
 *   q [B, Lq, H, D]   indexer queries (q_dtype)
 *   k [B, Lk, D]      indexer keys (k_dtype), one row per cached token
 *   w [B, Lq, H]      per-query head weights (w_dtype)
 * Query i of sequence b sits at position p = Lk - Lq + i and scores every key
 * s <= p:   I[s] = sum_h w[h] * max(0, q[h,:] . k[s,:])   (fp32 accumulation).
 * Its index set T is the topk keys with the largest I (ties to the lower s),
 * written in ascending s; a query with p + 1 <= topk gets 0..p and -1 padding.
 *
 * Supported: (q,k,w) = (FP8_E4M3, FP8_E4M3, BF16) with D = 128, or
 * (BF16, BF16, FP32) with D in {32, 64, 128}; H in {4, 8, 16, 32, 64};
 * 1 <= topk <= 2048; 1 <= Lq <= Lk <= 2^24 - 1; B >= 1.
 */
typedef struct {
    int B, Lq, Lk, H, D, topk;
    idxc_dtype q_dtype, k_dtype, w_dtype;
} idxc_indexer_desc;

/* Workspace bytes idx_score_topk / idx_cache_route need for `desc` (may be 0). */
idxc_status idx_score_topk_workspace(const idxc_indexer_desc *desc, size_t *bytes);

/*
 * Fused indexer score + per-row top-k ([ITO] § "Einfache Implementierung, enorme
 * Effizienzgewinne": the Full-layer steps I = Indexer(X), T = top-k(I)).
 *   t_out      int32 [B, Lq, topk], ascending indices, -1 padded (output)
 *   scores_dbg optional fp32 [B, Lq, Lk]: if non-NULL, the scores are also
 *              written there (-inf beyond each query's position).  For tests
 *              only: it materialises the score matrix the fused path avoids.
 *   ws, ws_bytes  workspace, at least idx_score_topk_workspace() bytes
 *              (may be NULL when that size is 0).
 * Prefill-shaped problems (many queries per sequence) score and select in one
 * kernel and never store the score matrix; decode-shaped problems (Lq <= 4)
 * split each sequence's keys over many workgroups and select from the
 * workspace.  Both give the same T.
 */
idxc_status idx_score_topk(const idxc_indexer_desc *desc, const void *q, const void *k,
                           const void *w, int32_t *t_out, float *scores_dbg, void *ws,
                           size_t ws_bytes, void *stream);

/*
 * idx_score_topk without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, hosts that forbid allocation during a step.
 * Same descriptor, tensors, result and checks as idx_score_topk (no scores_dbg).
 * Where idx_score_topk would need a workspace, this call uses a static device
 * array of the library instead: 128 MiB per GPU, reserved when the library's
 * code object is loaded on that GPU and held until the process ends (its
 * address is looked up once per device, on the first call there).  A request
 * whose idx_score_topk_workspace() exceeds 128 MiB returns IDXC_ERR_SCRATCH
 * and enqueues nothing (the decode step of 32 sequences of 200,000 keys needs
 * about 77 MB: the score rows and the top-k's candidate regions).  All calls
 * on one GPU share the array: calls that may overlap on one GPU (different
 * streams without ordering) race and must not be issued.
 */
idxc_status idx_score_topk_noalloc(const idxc_indexer_desc *desc, const void *q, const void *k,
                                   const void *w, int32_t *t_out, void *stream);

/* Workspace bytes for idx_topk (may be 0: it is nonzero when few long rows
 * are each split over several workgroups). */
idxc_status idx_topk_workspace(int R, int Lk, int topk, size_t *bytes);

/*
 * Row top-k over given fp32 scores ([ITO] § "Einfache Implementierung, enorme
 * Effizienzgewinne", the top-k step on its own).
 *   scores  fp32 [R, Lk]
 *   row_pos int32 [R] last valid key of each row (keys 0..row_pos[r]); NULL
 *           means Lk - 1 for every row.  Values must lie in [-1, Lk - 1].
 *   t_out   int32 [R, topk]: if row_pos + 1 <= topk: 0..row_pos then -1;
 *           otherwise the topk keys by (score desc, index asc), ascending.
 *   ws      device scratch of ws_bytes >= idx_topk_workspace(R, Lk, topk)
 *           bytes, 16-byte aligned; may be NULL when that size is 0.  Its
 *           contents are overwritten; IDXC_ERR_WORKSPACE when too small.
 * -0 and +0 compare equal.  NaN scores are outside the contract.
 */
idxc_status idx_topk(const float *scores, const int32_t *row_pos, int R, int Lk, int topk,
                     int32_t *t_out, void *ws, size_t ws_bytes, void *stream);

/*
 * IndexCache layer router ([ITO] §§ "Der unsichtbare Datenstrom" and "Einfache
 * Implementierung, enorme Effizienzgewinne"; [PPM] § "Aandacht cachen met
 * IndexCache"; [AIB] comparison table: one branch, no extra GPU memory).
 *   pattern  NUL-terminated host string, one 'F' (Full) or 'S' (Shared) per
 *            layer; pattern[0] must be 'F' (the first layer fills the cache).
 *   layer    0 <= layer < strlen(pattern)
 *   t_cache  int32 [B, Lq, topk]: the one index buffer shared by all layers.
 * Full layer: exactly idx_score_topk(desc, q, k, w, t_cache, NULL, ws, ...);
 *   t_cache is overwritten in place and *computed = 1.
 * Shared layer: nothing is enqueued, t_cache is left as the nearest preceding
 *   Full layer wrote it (that layer's T is this layer's T), *computed = 0;
 *   q, k, w, ws may be NULL.
 * `computed` is a HOST pointer and may be NULL.
 */
idxc_status idx_cache_route(const char *pattern, int layer, const idxc_indexer_desc *desc,
                            const void *q, const void *k, const void *w, int32_t *t_cache,
                            void *ws, size_t ws_bytes, void *stream, int *computed);

/*
 * Sparse MLA attention over the selected rows ([ITO] introduction: attention
 * over the k selected tokens only; § "Wie der Indexer funktioniert und warum MLA
 * entscheidend ist": one compressed latent row per token, shared by all heads).
 *   q   bf16 [B, Lq, Hq, Dqk]
 *   kv  bf16 [B, Lk, Dqk]   latent rows; keys are the whole row, values are
 *                           its first Dv columns
 *   t   int32 [B, Lq, topk] row indices into kv (entries < 0 or >= Lk are
 *                           skipped: they select no row)
 *   out bf16 [B, Lq, Hq, Dv]:  out[h] = sum_j softmax_j(z) kv[t_j, :Dv],
 *                           z_j = sm_scale * q[h] . kv[t_j]   (fp32 math)
 *   lse optional fp32 [B, Lq, Hq]: log-sum-exp of z (-inf, with out = 0,
 *                           for a query whose index set is empty)
 * Supported: (Dqk, Dv) in {(32, 32), (576, 512)}; Hq a multiple of 4 up to
 * 128 (Dqk = 32) or a multiple of 16 (Dqk = 576); 1 <= topk <= 2048.
 */
typedef struct {
    int B, Lq, Lk, Hq, Dqk, Dv, topk;
} idxc_mla_desc;

idxc_status sparse_mla_attn_workspace(const idxc_mla_desc *desc, size_t *bytes);

idxc_status sparse_mla_attn(const idxc_mla_desc *desc, const void *q, const void *kv,
                            const int32_t *t, float sm_scale, void *out, float *lse, void *ws,
                            size_t ws_bytes, void *stream);

/*
 * Cross-layer overlap of two layers' index sets ([ITO] introduction and
 * § "Der unsichtbare Datenstrom": adjacent layers select largely the same
 * tokens; [PPM] § "Aandacht cachen met IndexCache"), the diagnostic behind
 * choosing Full and Shared layers.
 *   t_a, t_b int32 [R, topk]: rows as idx_score_topk writes them (ascending
 *            indices, then -1 padding); rows not in that form give
 *            unspecified counts.
 *   counts   int32 [R]: counts[r] = number of indices >= 0 present in both
 *            t_a[r] and t_b[r].
 * No workspace.  1 <= topk <= 2048; pointers 4-byte aligned.
 */
idxc_status idx_overlap(const int32_t *t_a, const int32_t *t_b, int R, int topk, int32_t *counts,
                        void *stream);

/*
 * Serving-shaped batches over paged caches ([PPM] §§ "Real-world versnellingen
 * op productiemodellen" (decode throughput of a saturated server) and
 * "IndexCache in productie brengen" (vLLM and SGLang patches); [SAI]
 * comparison table: paged memory allocation).
 *
 * A batch packs the query rows of num_seqs sequences one after another:
 * sequence b owns rows query_start[b] .. query_start[b+1]-1, which are its
 * last q_len_b = query_start[b+1] - query_start[b] positions, so row
 * query_start[b] + i sits at position seq_lens[b] - q_len_b + i.  Decode
 * tokens (q_len 1) and prefill chunks (q_len > 1) may be mixed freely.
 * Caches are pools of num_blocks pages of block_size rows; sequence b's
 * position s lives in page block_table[b][s / block_size], row
 * s % block_size.  The same table serves the indexer key cache and the
 * latent KV cache.
 *
 * query_start [num_seqs + 1], seq_lens [num_seqs] and block_table
 * [num_seqs, max_blocks] are DEVICE int32 arrays.  Their contents must satisfy
 * query_start[0] = 0, query_start nondecreasing with query_start[num_seqs] =
 * total_q, q_len_b <= seq_lens[b] <= max_seq_len, and every page of a
 * sequence's positions in [0, num_blocks).  The host cannot check them;
 * values outside this contract give unspecified results but no out-of-bounds
 * access (positions and pages are clamped).
 */
typedef struct {
    int num_seqs, total_q, max_seq_len;
    int num_blocks, block_size, max_blocks; /* block_size: power of two >= 64 */
    int H, D, topk;
    idxc_dtype q_dtype, k_dtype, w_dtype;
} idxc_paged_indexer_desc;

/* Workspace bytes of idx_score_topk_paged (scores of every row up to
 * max_seq_len, plus row metadata). */
idxc_status idx_score_topk_paged_workspace(const idxc_paged_indexer_desc *desc, size_t *bytes);

/*
 * idx_score_topk over a serving batch:
 *   q       [total_q, H, D]          packed query rows (q_dtype)
 *   k_cache [num_blocks, block_size, D] key pages (k_dtype)
 *   w       [total_q, H]             head weights (w_dtype)
 *   t_out   int32 [total_q, topk]    logical positions, as idx_score_topk
 * Every row is scored against its sequence's keys 0..position (split over
 * many workgroups, pages looked up per 64-key block) and its index set is
 * the row top-k of those scores.  Supported as the split-key decode path of
 * idx_score_topk: H = 64 with (FP8_E4M3, FP8_E4M3, BF16) D = 128 or
 * (BF16, BF16, FP32) D in {32, 64, 128}.
 */
idxc_status idx_score_topk_paged(const idxc_paged_indexer_desc *desc, const void *q, const void *k_cache,
                                 const int32_t *block_table, const int32_t *query_start, const int32_t *seq_lens,
                                 const void *w, int32_t *t_out, void *ws, size_t ws_bytes, void *stream);

/* The IndexCache router over a serving batch: as idx_cache_route with the
 * Full-layer step replaced by idx_score_topk_paged; t_cache [total_q, topk]. */
idxc_status idx_cache_route_paged(const char *pattern, int layer, const idxc_paged_indexer_desc *desc,
                                  const void *q, const void *k_cache, const int32_t *block_table,
                                  const int32_t *query_start, const int32_t *seq_lens, const void *w,
                                  int32_t *t_cache, void *ws, size_t ws_bytes, void *stream, int *computed);

typedef struct {
    int num_seqs, total_q;
    int num_blocks, block_size, max_blocks; /* block_size: power of two >= 1 */
    int Hq, Dqk, Dv, topk;
} idxc_paged_mla_desc;

idxc_status sparse_mla_attn_paged_workspace(const idxc_paged_mla_desc *desc, size_t *bytes);

/*
 * sparse_mla_attn over a serving batch:
 *   q        bf16 [total_q, Hq, Dqk]
 *   kv_cache bf16 [num_blocks, block_size, Dqk] latent pages
 *   t        int32 [total_q, topk] logical positions of the row's sequence
 *            (entries < 0 or >= seq_len are skipped)
 *   out      bf16 [total_q, Hq, Dv], lse optional fp32 [total_q, Hq]
 * The index sets are turned into page-pool rows, then the contiguous kernel
 * runs with the pool as one cache.  Same head/dimension support as
 * sparse_mla_attn.
 */
idxc_status sparse_mla_attn_paged(const idxc_paged_mla_desc *desc, const void *q, const void *kv_cache,
                                  const int32_t *block_table, const int32_t *query_start, const int32_t *seq_lens,
                                  const int32_t *t, float sm_scale, void *out, float *lse, void *ws,
                                  size_t ws_bytes, void *stream);

/* Static text for a status code. */
const char *idxc_status_str(idxc_status s);

/* IDXC_ABI_VERSION of the loaded library. */
int idxc_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* IDXCACHE_H */
