// abi.cpp -- the C ABI of libidxcache.so (declared in include/idxcache.h).
//
// Every entry point validates its arguments on the host before the first HIP
// call, so a rejected call enqueues nothing and needs no GPU.  Dispatch:
//   idx_score_topk  -> fused prefill kernel (scores never stored), or, for
//                      decode-shaped problems, split-key scoring into the
//                      workspace followed by the row top-k kernel;
//   idx_topk        -> row top-k kernel;
//   idx_cache_route -> the IndexCache branch (itoverdose.com, "IndexCache: Wie
//                      DeepSeek O(NL²)-Kosten in Sparse Attention um 75%
//                      reduziert", section "Einfache Implementierung, enorme
//                      Effizienzgewinne"): Full layers run idx_score_topk into
//                      the cache buffer, Shared layers enqueue nothing;
//   sparse_mla_attn -> sparse MLA kernel;
//   idx_overlap     -> per-row index-set overlap of two layers' T.
#include <hip/hip_runtime.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/idxcache.h"
#include "kernels.h"

using idxc::Enc;

namespace {

constexpr int kMaxTopk = 2048;
constexpr int kMaxLen = (1 << 24) - 1;
constexpr int kDecodeMaxLq = 4;

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool known_dtype(int d) { return d == IDXC_BF16 || d == IDXC_FP8_E4M3 || d == IDXC_FP32; }

bool h_supported(int H) { return H == 4 || H == 8 || H == 16 || H == 32 || H == 64; }

// Shape/encoding checks shared by idx_score_topk and idx_cache_route.
idxc_status check_indexer_desc(const idxc_indexer_desc *d) {
    if (!d) return IDXC_ERR_NULL;
    if (!known_dtype(d->q_dtype) || !known_dtype(d->k_dtype) || !known_dtype(d->w_dtype)) return IDXC_ERR_DTYPE;
    const bool fp8 = d->q_dtype == IDXC_FP8_E4M3 && d->k_dtype == IDXC_FP8_E4M3 && d->w_dtype == IDXC_BF16;
    const bool bf16 = d->q_dtype == IDXC_BF16 && d->k_dtype == IDXC_BF16 && d->w_dtype == IDXC_FP32;
    if (!fp8 && !bf16) return IDXC_ERR_DTYPE;
    if (d->B < 1 || d->Lq < 1 || d->Lk < 1 || d->Lq > d->Lk || d->H < 1 || d->D < 1 || d->topk < 1)
        return IDXC_ERR_SHAPE;
    if (d->Lk > kMaxLen) return IDXC_ERR_SHAPE;
    if ((size_t)d->B * (size_t)d->Lk > (size_t)INT32_MAX) return IDXC_ERR_SHAPE;
    if (!h_supported(d->H) || d->topk > kMaxTopk) return IDXC_ERR_UNSUPPORTED;
    if (fp8 && d->D != 128) return IDXC_ERR_UNSUPPORTED;
    if (bf16 && d->D != 32 && d->D != 64 && d->D != 128) return IDXC_ERR_UNSUPPORTED;
    return IDXC_OK;
}

idxc::IndexerArgs make_args(const idxc_indexer_desc *d, const void *q, const void *k, const void *w,
                            int32_t *t, float *scores) {
    idxc::IndexerArgs a;
    a.q = q; a.k = k; a.w = w; a.t_out = t; a.scores = scores;
    a.B = d->B; a.Lq = d->Lq; a.Lk = d->Lk; a.H = d->H; a.D = d->D; a.topk = d->topk;
    a.qk_enc = d->q_dtype == IDXC_FP8_E4M3 ? Enc::FP8 : Enc::BF16;
    a.w_enc = d->w_dtype == IDXC_BF16 ? Enc::BF16 : Enc::FP32;
    return a;
}

enum class Path { Fused, Decode, None };

Path choose_path(const idxc::IndexerArgs &a) {
    if (a.Lq <= kDecodeMaxLq && idxc::decode_supported(a)) return Path::Decode;
    if (idxc::prefill_fits(a)) return Path::Fused;
    if (idxc::decode_supported(a)) return Path::Decode;
    return Path::None;
}

// Decode workspace: the score rows, then the row top-k's own workspace.
size_t decode_scores_bytes(const idxc_indexer_desc *d) {
    return ((size_t)d->B * d->Lq * d->Lk * sizeof(float) + 255) & ~(size_t)255;
}

size_t decode_ws_bytes(const idxc_indexer_desc *d) {
    return decode_scores_bytes(d) + idxc::row_topk_ws_bytes(d->B * d->Lq, d->Lk);
}

idxc_status from_hip(hipError_t e) { return e == hipSuccess ? IDXC_OK : IDXC_ERR_HIP; }

// Descriptor, tensor pointers and the path an F-layer call takes.
idxc_status check_indexer_tensors(const idxc_indexer_desc *d, const void *q, const void *k, const void *w,
                                  const int32_t *t, const float *scores_dbg, Path *path) {
    idxc_status st = check_indexer_desc(d);
    if (st != IDXC_OK) return st;
    if (!q || !k || !w || !t) return IDXC_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(t, 16) || !aligned(w, 4)) return IDXC_ERR_ALIGN;
    if (scores_dbg && !aligned(scores_dbg, 16)) return IDXC_ERR_ALIGN;
    const idxc::IndexerArgs a = make_args(d, q, k, w, nullptr, nullptr);
    *path = choose_path(a);
    if (*path == Path::None) return IDXC_ERR_UNSUPPORTED;
    return IDXC_OK;
}

// Validation of the tensors of an F-layer call; shared by score_topk and route.
idxc_status check_indexer_call(const idxc_indexer_desc *d, const void *q, const void *k, const void *w,
                               const int32_t *t, const float *scores_dbg, const void *ws, size_t ws_bytes,
                               Path *path) {
    const idxc_status st = check_indexer_tensors(d, q, k, w, t, scores_dbg, path);
    if (st != IDXC_OK) return st;
    if (*path == Path::Decode) {
        if (!ws || ws_bytes < decode_ws_bytes(d)) return IDXC_ERR_WORKSPACE;
        if (!aligned(ws, 16)) return IDXC_ERR_ALIGN;
    }
    return IDXC_OK;
}

// When the row top-k takes its split path over exactly the score kernel's key
// ranges, the score kernel writes the per-split bounds itself (one pass over
// the scores fewer).  Sets a.split_bound and returns whether it did.
int fuse_split_bounds(idxc::IndexerArgs &a, const idxc::TopkArgs &ta) {
    int S, N, ns, sp;
    if (!idxc::row_topk_split_geometry(ta.R, ta.Lk, &S, &N)) return 0;
    idxc::decode_split_geometry(a, &ns, &sp);
    if (ns != S || sp != N) return 0;
    a.split_bound = idxc::row_topk_split_bounds(ta.ws, ta.R, ta.Lk);
    return 1;
}

idxc_status run_indexer(const idxc_indexer_desc *d, const void *q, const void *k, const void *w, int32_t *t,
                        float *scores_dbg, void *ws, Path path, hipStream_t stream) {
    if (path == Path::Fused) {
        idxc::IndexerArgs a = make_args(d, q, k, w, t, scores_dbg);
        return from_hip(idxc::launch_indexer_prefill(a, stream));
    }
    float *scores = static_cast<float *>(ws);
    idxc::IndexerArgs a = make_args(d, q, k, w, t, scores);
    idxc::TopkArgs ta;
    ta.scores = scores;
    ta.row_pos = nullptr;
    ta.R = d->B * d->Lq;
    ta.Lk = d->Lk;
    ta.topk = d->topk;
    ta.pos_Lq = d->Lq;
    ta.t_out = t;
    ta.ws = static_cast<unsigned char *>(ws) + decode_scores_bytes(d);
    ta.ws_bytes = idxc::row_topk_ws_bytes(ta.R, ta.Lk);
    ta.bounds_given = fuse_split_bounds(a, ta);
    hipError_t e = idxc::launch_indexer_scores(a, stream);
    if (e != hipSuccess) return IDXC_ERR_HIP;
    e = idxc::launch_row_topk(ta, stream);
    if (e != hipSuccess) return IDXC_ERR_HIP;
    if (scores_dbg)
        e = hipMemcpyAsync(scores_dbg, scores, (size_t)d->B * d->Lq * d->Lk * sizeof(float), hipMemcpyDeviceToDevice,
                           stream);
    return from_hip(e);
}

// Pattern validation shared by both routers; returns IDXC_OK and sets *full.
idxc_status check_route(const char *pattern, int layer, bool *full) {
    if (!pattern) return IDXC_ERR_NULL;
    const size_t n = strlen(pattern);
    if (n == 0 || pattern[0] != 'F') return IDXC_ERR_PATTERN;
    for (size_t i = 0; i < n; ++i)
        if (pattern[i] != 'F' && pattern[i] != 'S') return IDXC_ERR_PATTERN;
    if (layer < 0 || (size_t)layer >= n) return IDXC_ERR_PATTERN;
    *full = pattern[layer] == 'F';
    return IDXC_OK;
}

// sparse_mla_attn after the null check; the paged entry point calls it with
// the page pool as one cache (Lk = num_blocks * block_size).
// validate_only: return after the checks, before any launch.
idxc_status run_mla(const idxc_mla_desc *desc, const void *q, const void *kv, const int32_t *t, float sm_scale,
                    void *out, float *lse, void *ws, size_t ws_bytes, void *stream, bool validate_only = false) {
    const idxc_mla_desc &d = *desc;
    if (d.B < 1 || d.Lq < 1 || d.Lk < 1 || d.Hq < 1 || d.Dqk < 1 || d.Dv < 1 || d.topk < 1 || d.Dv > d.Dqk)
        return IDXC_ERR_SHAPE;
    if ((size_t)d.B * d.Lq > (size_t)INT32_MAX / 2) return IDXC_ERR_SHAPE;
    const bool small = d.Dqk == 32 && d.Dv == 32;
    const bool mla = d.Dqk == 576 && d.Dv == 512;
    if (!small && !mla) return IDXC_ERR_UNSUPPORTED;
    if (small && (d.Hq % 4 != 0 || d.Hq > 128)) return IDXC_ERR_UNSUPPORTED;
    if (mla && d.Hq % 16 != 0) return IDXC_ERR_UNSUPPORTED;
    if (d.topk > kMaxTopk) return IDXC_ERR_UNSUPPORTED;
    if (!(sm_scale > 0.f) || sm_scale > 1e30f) return IDXC_ERR_SHAPE;
    if (!q || !kv || !t || !out) return IDXC_ERR_NULL;
    if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(t, 4) || !aligned(out, 4) || (lse && !aligned(lse, 4)))
        return IDXC_ERR_ALIGN;
    const idxc::MlaWidePlan plan = idxc::mla_wide_plan(d.B, d.Lq, d.Hq, d.Dqk, d.Dv, d.topk);
    if (plan.ok) {
        if (plan.ws_bytes > 0 && !validate_only) {
            if (!ws || ws_bytes < plan.ws_bytes) return IDXC_ERR_WORKSPACE;
            if (!aligned(ws, 16)) return IDXC_ERR_ALIGN;
        }
        if (validate_only) return IDXC_OK;
        idxc::MlaWideArgs w;
        w.q = q; w.kv = kv; w.t = t; w.out = out; w.lse = lse; w.sm_scale = sm_scale;
        w.B = d.B; w.Lq = d.Lq; w.Lk = d.Lk; w.Hq = d.Hq; w.topk = d.topk;
        w.nchunk = plan.nchunk; w.chunk_rows = plan.chunk_rows;
        w.part_o = ws;
        w.part_lse = plan.ws_bytes > 0
                         ? reinterpret_cast<float *>(static_cast<unsigned char *>(ws) +
                                                     (size_t)d.B * d.Lq * d.Hq * plan.nchunk * d.Dv * 2)
                         : nullptr;
        return from_hip(idxc::launch_sparse_mla_wide(w, static_cast<hipStream_t>(stream)));
    }
    if (validate_only) return IDXC_OK;
    idxc::MlaArgs a;
    a.q = q; a.kv = kv; a.t = t; a.out = out; a.lse = lse; a.sm_scale = sm_scale;
    a.B = d.B; a.Lq = d.Lq; a.Lk = d.Lk; a.Hq = d.Hq; a.Dqk = d.Dqk; a.Dv = d.Dv; a.topk = d.topk;
    return from_hip(idxc::launch_sparse_mla(a, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- paged

bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
int log2i(int v) {
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// The dense descriptor that the split-key scoring path sees for a serving
// batch: total_q rows of one "sequence" whose score rows are max_seq_len long.
idxc_indexer_desc paged_as_dense(const idxc_paged_indexer_desc *d);

// Two ways to score a serving batch, chosen from the descriptor alone:
//  * fused: the prefill kernel with page lookups per 64-key block scores and
//    selects every row without storing scores (one workgroup per 4-8 rows of
//    a sequence, so it pays off when the batch holds prefill chunks: more
//    than 4 rows per sequence on average, fp8 with 64 heads of 128);
//  * split: every row's keys split over many workgroups into score rows of
//    max_seq_len, then the row top-k (decode tokens).
bool paged_fused(const idxc_paged_indexer_desc *d) {
    if ((long long)d->total_q <= 4LL * d->num_seqs) return false;
    const idxc_indexer_desc e = paged_as_dense(d);
    idxc::IndexerArgs a;
    a.B = 1; a.Lq = 1; a.Lk = d->max_seq_len; a.H = d->H; a.D = d->D; a.topk = d->topk;
    a.qk_enc = e.q_dtype == IDXC_FP8_E4M3 ? Enc::FP8 : Enc::BF16;
    a.w_enc = e.w_dtype == IDXC_BF16 ? Enc::BF16 : Enc::FP32;
    return e.q_dtype == IDXC_FP8_E4M3 && idxc::paged_prefill_supported(a);
}

// Paged indexer workspace.  Split: row (sequence, position) pairs, row
// positions, score rows of max_seq_len, then the row top-k's workspace.
// Fused: the row-block prefix over sequences only.
struct PagedIdxWs {
    size_t info, pos, scores, topk, rb, total;
};
PagedIdxWs paged_idx_ws(const idxc_paged_indexer_desc *d) {
    PagedIdxWs w = {};
    if (paged_fused(d)) {
        w.rb = 0;
        w.total = align256((size_t)(d->num_seqs + 1) * 4);
        return w;
    }
    w.info = 0;
    w.pos = align256((size_t)d->total_q * 8);
    w.scores = w.pos + align256((size_t)d->total_q * 4);
    w.topk = w.scores + align256((size_t)d->total_q * d->max_seq_len * sizeof(float));
    w.total = w.topk + idxc::row_topk_ws_bytes(d->total_q, d->max_seq_len);
    return w;
}

idxc_indexer_desc paged_as_dense(const idxc_paged_indexer_desc *d) {
    idxc_indexer_desc e;
    e.B = 1;
    e.Lq = d->total_q;
    e.Lk = d->max_seq_len;
    e.H = d->H;
    e.D = d->D;
    e.topk = d->topk;
    e.q_dtype = d->q_dtype;
    e.k_dtype = d->k_dtype;
    e.w_dtype = d->w_dtype;
    return e;
}

idxc_status check_paged_indexer_desc(const idxc_paged_indexer_desc *d) {
    if (!d) return IDXC_ERR_NULL;
    if (d->num_seqs < 1 || d->total_q < 1 || d->max_seq_len < 1 || d->num_blocks < 1 || d->max_blocks < 1 ||
        d->H < 1 || d->D < 1 || d->topk < 1)
        return IDXC_ERR_SHAPE;
    if (!pow2(d->block_size) || d->block_size < 64) return IDXC_ERR_SHAPE;
    if (d->max_seq_len > kMaxLen || (long long)d->max_blocks * d->block_size < d->max_seq_len) return IDXC_ERR_SHAPE;
    if ((long long)d->num_blocks * d->block_size > (long long)INT32_MAX) return IDXC_ERR_SHAPE;
    if ((long long)d->total_q * d->max_seq_len > ((long long)1 << 40)) return IDXC_ERR_SHAPE;
    const idxc_indexer_desc e = paged_as_dense(d);
    idxc_status st = check_indexer_desc(&e);
    if (st != IDXC_OK && st != IDXC_ERR_SHAPE) return st;   // encodings, heads, topk
    const idxc::IndexerArgs a = make_args(&e, nullptr, nullptr, nullptr, nullptr, nullptr);
    if (!idxc::decode_supported(a)) return IDXC_ERR_UNSUPPORTED;
    return IDXC_OK;
}

idxc_status run_indexer_paged(const idxc_paged_indexer_desc *d, const void *q, const void *k_cache,
                              const int32_t *block_table, const int32_t *query_start, const int32_t *seq_lens,
                              const void *w, int32_t *t, void *ws, hipStream_t stream) {
    const PagedIdxWs lay = paged_idx_ws(d);
    unsigned char *wsb = static_cast<unsigned char *>(ws);
    if (paged_fused(d)) {
        const idxc_indexer_desc dd = paged_as_dense(d);
        idxc::IndexerArgs a = make_args(&dd, q, k_cache, w, t, nullptr);
        idxc::PagedPrefill pp;
        pp.query_start = query_start;
        pp.seq_lens = seq_lens;
        pp.block_table = block_table;
        pp.rb_start = reinterpret_cast<int32_t *>(wsb + lay.rb);
        pp.num_seqs = d->num_seqs;
        pp.total_q = d->total_q;
        pp.bs_log2 = log2i(d->block_size);
        pp.max_blocks = d->max_blocks;
        pp.num_blocks = d->num_blocks;
        const long long cap = std::min<long long>(d->max_seq_len, (long long)d->max_blocks << pp.bs_log2);
        hipError_t e = idxc::launch_row_blocks(query_start, d->num_seqs, d->total_q,
                                               idxc::prefill_rows_per_workgroup(a), (int)cap,
                                               reinterpret_cast<int32_t *>(wsb + lay.rb), stream);
        if (e != hipSuccess) return IDXC_ERR_HIP;
        return from_hip(idxc::launch_indexer_prefill_paged(a, pp, stream));
    }
    int32_t *info = reinterpret_cast<int32_t *>(wsb + lay.info);
    int32_t *pos = reinterpret_cast<int32_t *>(wsb + lay.pos);
    float *scores = reinterpret_cast<float *>(wsb + lay.scores);
    hipError_t e = idxc::launch_row_info(query_start, seq_lens, d->num_seqs, d->total_q, d->max_seq_len - 1, info,
                                         pos, stream);
    if (e != hipSuccess) return IDXC_ERR_HIP;
    const idxc_indexer_desc dd = paged_as_dense(d);
    idxc::IndexerArgs a = make_args(&dd, q, k_cache, w, t, scores);
    idxc::PagedKeys pk;
    pk.block_table = block_table;
    pk.row_info = info;
    pk.bs_log2 = log2i(d->block_size);
    pk.max_blocks = d->max_blocks;
    pk.num_blocks = d->num_blocks;
    idxc::TopkArgs ta;
    ta.scores = scores;
    ta.row_pos = pos;
    ta.R = d->total_q;
    ta.Lk = d->max_seq_len;
    ta.topk = d->topk;
    ta.pos_Lq = 0;
    ta.t_out = t;
    ta.ws = wsb + lay.topk;
    ta.ws_bytes = lay.total - lay.topk;
    ta.bounds_given = fuse_split_bounds(a, ta);
    e = idxc::launch_indexer_scores(a, stream, &pk);
    if (e != hipSuccess) return IDXC_ERR_HIP;
    return from_hip(idxc::launch_row_topk(ta, stream));
}

idxc_status check_paged_indexer_call(const idxc_paged_indexer_desc *d, const void *q, const void *k_cache,
                                     const int32_t *block_table, const int32_t *query_start,
                                     const int32_t *seq_lens, const void *w, const int32_t *t, const void *ws,
                                     size_t ws_bytes) {
    idxc_status st = check_paged_indexer_desc(d);
    if (st != IDXC_OK) return st;
    if (!q || !k_cache || !block_table || !query_start || !seq_lens || !w || !t) return IDXC_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(t, 16) || !aligned(w, 4) || !aligned(block_table, 4) ||
        !aligned(query_start, 4) || !aligned(seq_lens, 4))
        return IDXC_ERR_ALIGN;
    if (!ws || ws_bytes < paged_idx_ws(d).total) return IDXC_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return IDXC_ERR_ALIGN;
    return IDXC_OK;
}

// Paged sparse MLA workspace: row metadata, pool-row index sets, then the
// workspace of the contiguous kernel for total_q rows.
struct PagedMlaWs {
    size_t info, tphys, mla, total;
};
idxc_mla_desc paged_mla_as_dense(const idxc_paged_mla_desc *d) {
    idxc_mla_desc m;
    m.B = 1;
    m.Lq = d->total_q;
    m.Lk = (int)((long long)d->num_blocks * d->block_size);
    m.Hq = d->Hq;
    m.Dqk = d->Dqk;
    m.Dv = d->Dv;
    m.topk = d->topk;
    return m;
}
PagedMlaWs paged_mla_ws(const idxc_paged_mla_desc *d, size_t mla_bytes) {
    PagedMlaWs w;
    w.info = 0;
    w.tphys = align256((size_t)d->total_q * 8);
    w.mla = w.tphys + align256((size_t)d->total_q * d->topk * 4);
    w.total = w.mla + mla_bytes;
    return w;
}

// ---------------------------------------------------------------- static scratch
//
// Device memory of idx_score_topk_noalloc: one array per GPU, loaded with the
// library's code object and held until the process ends.  Host code never
// uses the array's name as an address (on the host it is only a stand-in):
// the device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (resolved on its first use).
idxc_status scratch_for_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return IDXC_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return IDXC_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return IDXC_OK;
}

}  // namespace

extern "C" {

int idxc_abi_version(void) { return IDXC_ABI_VERSION; }

const char *idxc_status_str(idxc_status s) {
    switch (s) {
    case IDXC_OK: return "ok";
    case IDXC_ERR_NULL: return "a required pointer is NULL";
    case IDXC_ERR_SHAPE: return "a size is out of range or sizes disagree";
    case IDXC_ERR_DTYPE: return "unknown or unsupported element encoding combination";
    case IDXC_ERR_ALIGN: return "a pointer is not suitably aligned";
    case IDXC_ERR_UNSUPPORTED: return "no kernel for this valid request";
    case IDXC_ERR_WORKSPACE: return "workspace missing or too small";
    case IDXC_ERR_PATTERN: return "invalid layer pattern or layer index";
    case IDXC_ERR_HIP: return "HIP runtime error at launch";
    case IDXC_ERR_SCRATCH: return "request needs more device scratch than the library's static array holds";
    }
    return "unknown status";
}

idxc_status idx_score_topk_workspace(const idxc_indexer_desc *desc, size_t *bytes) {
    if (!bytes) return IDXC_ERR_NULL;
    idxc_status st = check_indexer_desc(desc);
    if (st != IDXC_OK) return st;
    const idxc::IndexerArgs a = make_args(desc, nullptr, nullptr, nullptr, nullptr, nullptr);
    const Path p = choose_path(a);
    if (p == Path::None) return IDXC_ERR_UNSUPPORTED;
    *bytes = p == Path::Decode ? decode_ws_bytes(desc) : 0;
    return IDXC_OK;
}

idxc_status idx_score_topk(const idxc_indexer_desc *desc, const void *q, const void *k, const void *w,
                           int32_t *t_out, float *scores_dbg, void *ws, size_t ws_bytes, void *stream) {
    Path path;
    idxc_status st = check_indexer_call(desc, q, k, w, t_out, scores_dbg, ws, ws_bytes, &path);
    if (st != IDXC_OK) return st;
    return run_indexer(desc, q, k, w, t_out, scores_dbg, ws, path, static_cast<hipStream_t>(stream));
}

idxc_status idx_score_topk_noalloc(const idxc_indexer_desc *desc, const void *q, const void *k, const void *w,
                                   int32_t *t_out, void *stream) {
    // the same checks and kernels as idx_score_topk, with the static scratch as
    // the workspace; nothing in it needs to start at zero (every word a call
    // reads was written earlier in the same call).  All checks run before the
    // first HIP call.
    Path path;
    idxc_status st = check_indexer_tensors(desc, q, k, w, t_out, nullptr, &path);
    if (st != IDXC_OK) return st;
    const size_t need = path == Path::Decode ? decode_ws_bytes(desc) : 0;
    if (need > kScratchBytes) return IDXC_ERR_SCRATCH;
    void *ws = nullptr;
    if (need > 0) {
        st = scratch_for_current_device(&ws);
        if (st != IDXC_OK) return st;
    }
    return run_indexer(desc, q, k, w, t_out, nullptr, ws, path, static_cast<hipStream_t>(stream));
}

idxc_status idx_topk_workspace(int R, int Lk, int topk, size_t *bytes) {
    if (!bytes) return IDXC_ERR_NULL;
    if (R < 0 || Lk < 1 || topk < 1 || Lk > kMaxLen) return IDXC_ERR_SHAPE;
    if (topk > kMaxTopk) return IDXC_ERR_UNSUPPORTED;
    *bytes = idxc::row_topk_ws_bytes(R, Lk);
    return IDXC_OK;
}

idxc_status idx_topk(const float *scores, const int32_t *row_pos, int R, int Lk, int topk, int32_t *t_out,
                     void *ws, size_t ws_bytes, void *stream) {
    if (R < 0 || Lk < 1 || topk < 1 || Lk > kMaxLen) return IDXC_ERR_SHAPE;
    if (topk > kMaxTopk) return IDXC_ERR_UNSUPPORTED;
    if (R == 0) return IDXC_OK;
    if (!scores || !t_out) return IDXC_ERR_NULL;
    if (!aligned(scores, 4) || !aligned(t_out, 4) || (row_pos && !aligned(row_pos, 4))) return IDXC_ERR_ALIGN;
    const size_t need = idxc::row_topk_ws_bytes(R, Lk);
    if (need > 0) {
        if (!ws || ws_bytes < need) return IDXC_ERR_WORKSPACE;
        if (!aligned(ws, 16)) return IDXC_ERR_ALIGN;
    }
    idxc::TopkArgs a;
    a.scores = scores;
    a.row_pos = row_pos;
    a.R = R;
    a.Lk = Lk;
    a.topk = topk;
    a.pos_Lq = 0;
    a.t_out = t_out;
    a.ws = ws;
    a.ws_bytes = ws_bytes;
    return from_hip(idxc::launch_row_topk(a, static_cast<hipStream_t>(stream)));
}

idxc_status idx_cache_route(const char *pattern, int layer, const idxc_indexer_desc *desc, const void *q,
                            const void *k, const void *w, int32_t *t_cache, void *ws, size_t ws_bytes,
                            void *stream, int *computed) {
    if (!pattern || !t_cache) return IDXC_ERR_NULL;
    bool full;
    const idxc_status pst = check_route(pattern, layer, &full);
    if (pst != IDXC_OK) return pst;
    if (!full) {
        // T of this layer is the cache as the nearest preceding Full layer left it.
        if (computed) *computed = 0;
        return IDXC_OK;
    }
    Path path;
    idxc_status st = check_indexer_call(desc, q, k, w, t_cache, nullptr, ws, ws_bytes, &path);
    if (st != IDXC_OK) return st;
    st = run_indexer(desc, q, k, w, t_cache, nullptr, ws, path, static_cast<hipStream_t>(stream));
    if (st == IDXC_OK && computed) *computed = 1;
    return st;
}

idxc_status idx_overlap(const int32_t *t_a, const int32_t *t_b, int R, int topk, int32_t *counts, void *stream) {
    if (R < 0 || topk < 1 || topk > kMaxTopk) return IDXC_ERR_SHAPE;
    if (R == 0) return IDXC_OK;
    if (!t_a || !t_b || !counts) return IDXC_ERR_NULL;
    if (!aligned(t_a, 4) || !aligned(t_b, 4) || !aligned(counts, 4)) return IDXC_ERR_ALIGN;
    idxc::OverlapArgs a;
    a.t_a = t_a;
    a.t_b = t_b;
    a.R = R;
    a.topk = topk;
    a.counts = counts;
    return from_hip(idxc::launch_overlap(a, static_cast<hipStream_t>(stream)));
}

idxc_status sparse_mla_attn_workspace(const idxc_mla_desc *desc, size_t *bytes) {
    if (!desc || !bytes) return IDXC_ERR_NULL;
    const idxc_mla_desc &d = *desc;
    const idxc::MlaWidePlan p = idxc::mla_wide_plan(d.B, d.Lq, d.Hq, d.Dqk, d.Dv, d.topk);
    *bytes = p.ok ? p.ws_bytes : 0;
    return IDXC_OK;
}

idxc_status sparse_mla_attn(const idxc_mla_desc *desc, const void *q, const void *kv, const int32_t *t,
                            float sm_scale, void *out, float *lse, void *ws, size_t ws_bytes, void *stream) {
    if (!desc) return IDXC_ERR_NULL;
    if (desc->Lk > kMaxLen) return IDXC_ERR_SHAPE;
    return run_mla(desc, q, kv, t, sm_scale, out, lse, ws, ws_bytes, stream);
}
idxc_status idx_score_topk_paged_workspace(const idxc_paged_indexer_desc *desc, size_t *bytes) {
    if (!bytes) return IDXC_ERR_NULL;
    const idxc_status st = check_paged_indexer_desc(desc);
    if (st != IDXC_OK) return st;
    *bytes = paged_idx_ws(desc).total;
    return IDXC_OK;
}

idxc_status idx_score_topk_paged(const idxc_paged_indexer_desc *desc, const void *q, const void *k_cache,
                                 const int32_t *block_table, const int32_t *query_start, const int32_t *seq_lens,
                                 const void *w, int32_t *t_out, void *ws, size_t ws_bytes, void *stream) {
    const idxc_status st = check_paged_indexer_call(desc, q, k_cache, block_table, query_start, seq_lens, w, t_out,
                                                    ws, ws_bytes);
    if (st != IDXC_OK) return st;
    return run_indexer_paged(desc, q, k_cache, block_table, query_start, seq_lens, w, t_out, ws,
                             static_cast<hipStream_t>(stream));
}

idxc_status idx_cache_route_paged(const char *pattern, int layer, const idxc_paged_indexer_desc *desc,
                                  const void *q, const void *k_cache, const int32_t *block_table,
                                  const int32_t *query_start, const int32_t *seq_lens, const void *w,
                                  int32_t *t_cache, void *ws, size_t ws_bytes, void *stream, int *computed) {
    if (!pattern || !t_cache) return IDXC_ERR_NULL;
    bool full;
    idxc_status st = check_route(pattern, layer, &full);
    if (st != IDXC_OK) return st;
    if (!full) {
        if (computed) *computed = 0;
        return IDXC_OK;
    }
    st = check_paged_indexer_call(desc, q, k_cache, block_table, query_start, seq_lens, w, t_cache, ws, ws_bytes);
    if (st != IDXC_OK) return st;
    st = run_indexer_paged(desc, q, k_cache, block_table, query_start, seq_lens, w, t_cache, ws,
                           static_cast<hipStream_t>(stream));
    if (st == IDXC_OK && computed) *computed = 1;
    return st;
}

idxc_status sparse_mla_attn_paged_workspace(const idxc_paged_mla_desc *desc, size_t *bytes) {
    if (!desc || !bytes) return IDXC_ERR_NULL;
    if (desc->total_q < 1 || desc->topk < 1 || desc->num_blocks < 1 || desc->max_blocks < 1 ||
        !pow2(desc->block_size))
        return IDXC_ERR_SHAPE;
    if ((long long)desc->num_blocks * desc->block_size > (long long)INT32_MAX) return IDXC_ERR_SHAPE;
    const idxc_mla_desc m = paged_mla_as_dense(desc);
    size_t mla = 0;
    const idxc_status st = sparse_mla_attn_workspace(&m, &mla);
    if (st != IDXC_OK) return st;
    *bytes = paged_mla_ws(desc, mla).total;
    return IDXC_OK;
}

idxc_status sparse_mla_attn_paged(const idxc_paged_mla_desc *desc, const void *q, const void *kv_cache,
                                  const int32_t *block_table, const int32_t *query_start, const int32_t *seq_lens,
                                  const int32_t *t, float sm_scale, void *out, float *lse, void *ws,
                                  size_t ws_bytes, void *stream) {
    if (!desc) return IDXC_ERR_NULL;
    const idxc_paged_mla_desc &d = *desc;
    if (d.num_seqs < 1 || d.total_q < 1 || d.topk < 1 || d.num_blocks < 1 || d.max_blocks < 1 ||
        !pow2(d.block_size))
        return IDXC_ERR_SHAPE;
    if ((long long)d.num_blocks * d.block_size > (long long)INT32_MAX) return IDXC_ERR_SHAPE;
    if (!block_table || !query_start || !seq_lens || !t) return IDXC_ERR_NULL;
    if (!aligned(block_table, 4) || !aligned(query_start, 4) || !aligned(seq_lens, 4) || !aligned(t, 4))
        return IDXC_ERR_ALIGN;
    const idxc_mla_desc m = paged_mla_as_dense(desc);
    size_t mla = 0;
    idxc_status st = sparse_mla_attn_workspace(&m, &mla);
    if (st != IDXC_OK) return st;
    const PagedMlaWs lay = paged_mla_ws(desc, mla);
    if (!ws || ws_bytes < lay.total) return IDXC_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return IDXC_ERR_ALIGN;
    // the contiguous kernel's own checks run before anything is enqueued
    unsigned char *wsb = static_cast<unsigned char *>(ws);
    int32_t *info = reinterpret_cast<int32_t *>(wsb + lay.info);
    int32_t *tphys = reinterpret_cast<int32_t *>(wsb + lay.tphys);
    st = run_mla(&m, q, kv_cache, tphys, sm_scale, out, lse, wsb + lay.mla, lay.total - lay.mla, stream, true);
    if (st != IDXC_OK) return st;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    const int bs_log2 = log2i(d.block_size);
    hipError_t e = idxc::launch_row_info(query_start, seq_lens, d.num_seqs, d.total_q,
                                         (int)(((long long)d.max_blocks << bs_log2) - 1 < INT32_MAX
                                                   ? ((long long)d.max_blocks << bs_log2) - 1
                                                   : INT32_MAX),
                                         info, nullptr, hs);
    if (e != hipSuccess) return IDXC_ERR_HIP;
    e = idxc::launch_translate_index(t, info, seq_lens, block_table, d.total_q, d.topk, bs_log2, d.max_blocks,
                                     d.num_blocks, tphys, hs);
    if (e != hipSuccess) return IDXC_ERR_HIP;
    return run_mla(&m, q, kv_cache, tphys, sm_scale, out, lse, wsb + lay.mla, lay.total - lay.mla, stream);
}

}  // extern "C"
