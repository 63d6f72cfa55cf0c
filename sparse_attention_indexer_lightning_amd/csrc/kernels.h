// kernels.h -- internal launch interface between the C ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace idxc {

enum class Enc : int { BF16 = 1, FP8 = 2, FP32 = 3 };

struct IndexerArgs {
    const void *q, *k, *w;
    int32_t *t_out;
    float *scores;   // prefill: optional debug copy; decode: required score rows
    int B, Lq, Lk, H, D, topk;
    Enc qk_enc, w_enc;
    // decode: when set, the score kernel also writes every key range's top-k
    // bound here ([rows][ranges], as the row top-k's split bounds)
    uint32_t *split_bound = nullptr;
};

// Fused score + streaming top-k for prefill-shaped problems.  Returns
// hipErrorInvalidConfiguration when the shape does not fit the kernel's LDS
// plan (the caller then takes the two-step path).
bool prefill_fits(const IndexerArgs &a);
hipError_t launch_indexer_prefill(const IndexerArgs &a, hipStream_t s);

// Paged key cache for launch_indexer_scores: k is the page pool
// [num_blocks][1 << bs_log2][row] (bs_log2 >= 6), block_table [B][max_blocks]
// holds each sequence's pages in order, row_info [B*Lq] (int2) each query
// row's (sequence, position).  a.B * a.Lq is then the number of query rows
// and a.Lk the score row stride (>= every position + 1).
struct PagedKeys {
    const int32_t *block_table;
    const int32_t *row_info;
    int bs_log2, max_blocks, num_blocks;
};

// Fused score + top-k of a serving batch over a paged key cache (fp8, 64
// heads, d 128): a.q / a.w / a.t_out are packed rows [total_q, ...], a.k the
// page pool, a.Lk the longest sequence; rb_start [num_seqs + 1] (from
// launch_row_blocks with the same rows per workgroup) maps workgroups to
// (sequence, row block).  Rows of a sequence are its last q_len positions.
struct PagedPrefill {
    const int32_t *query_start, *seq_lens, *block_table;
    const int32_t *rb_start;
    int num_seqs, total_q, bs_log2, max_blocks, num_blocks;
};
bool paged_prefill_supported(const IndexerArgs &a);
int prefill_rows_per_workgroup(const IndexerArgs &a);
hipError_t launch_indexer_prefill_paged(const IndexerArgs &a, const PagedPrefill &pp, hipStream_t s);
// rb_start[b] = sum over sequences b' < b of ceil(q_len_b' / rows), with the
// query starts clamped to [0, total_q] and q_len to lk_cap as the paged
// prefill kernel clamps them; one workgroup.
hipError_t launch_row_blocks(const int32_t *query_start, int B, int total_q, int rows, int lk_cap,
                             int32_t *rb_start, hipStream_t s);

// Scores of every (query, key <= position) into a.scores [B*Lq, Lk], keys
// split over many workgroups; -inf beyond each query's position.
bool decode_supported(const IndexerArgs &a);
// Key ranges of the decode score kernel: nsplit ranges of `split` keys per row.
void decode_split_geometry(const IndexerArgs &a, int *nsplit, int *split);
hipError_t launch_indexer_scores(const IndexerArgs &a, hipStream_t s, const PagedKeys *paged = nullptr);

// Serving metadata: row_info[r] = (sequence, position) of query row r from
// query_start [B+1] (rows of sequence b are query_start[b]..[b+1]-1, the last
// ones of that sequence) and seq_lens [B]; row_pos [rows] (optional) gets the
// positions alone.  Values are clamped so that every row maps to a valid
// sequence and a position in [0, max_pos].
hipError_t launch_row_info(const int32_t *query_start, const int32_t *seq_lens, int B, int rows, int max_pos,
                           int32_t *row_info, int32_t *row_pos, hipStream_t s);
// Logical -> pool row indices of a paged latent cache: out[r][j] =
// page(t[r][j]) * bs + t[r][j] % bs for 0 <= t < seq_len of row r's
// sequence, -1 otherwise.
hipError_t launch_translate_index(const int32_t *t, const int32_t *row_info, const int32_t *seq_lens,
                                  const int32_t *block_table, int rows, int topk, int bs_log2, int max_blocks,
                                  int num_blocks, int32_t *out, hipStream_t s);

// Exact per-row top-k of fp32 scores [R, Lk] (ties to the lower index,
// ascending output, -1 padding).  row_pos may be NULL (all Lk keys valid).
// pos_from_query != 0 derives the position of row r as (Lk - Lq + r % Lq).
// Long rows that are few in number are split over several workgroups; that
// needs row_topk_ws_bytes(R, Lk) bytes of workspace (0 when not split).
struct TopkArgs {
    const float *scores;
    const int32_t *row_pos;
    int R, Lk, topk;
    int pos_Lq;       // > 0: row position = Lk - pos_Lq + r % pos_Lq (row_pos unused)
    int32_t *t_out;
    void *ws;         // device workspace of ws_bytes bytes (16-byte aligned), may be NULL if not needed
    size_t ws_bytes;
    int bounds_given = 0;   // split path: the per-split bounds in ws were written by the score kernel
};
size_t row_topk_ws_bytes(int R, int Lk);
// The split path's geometry (S splits of N keys per row; false: one workgroup
// per row) and the address of its per-split bounds [R][S] in a workspace.
bool row_topk_split_geometry(int R, int Lk, int *S, int *N);
uint32_t *row_topk_split_bounds(void *ws, int R, int Lk);
hipError_t launch_row_topk(const TopkArgs &a, hipStream_t s);

// counts[r] = |{t_a[r][j] >= 0} intersected with {t_b[r][j] >= 0}|; rows
// ascending with -1 padding.
struct OverlapArgs {
    const int32_t *t_a, *t_b;
    int R, topk;
    int32_t *counts;
};
hipError_t launch_overlap(const OverlapArgs &a, hipStream_t s);

struct MlaArgs {
    const void *q, *kv;
    const int32_t *t;
    void *out;
    float *lse;
    float sm_scale;
    int B, Lq, Lk, Hq, Dqk, Dv, topk;
};
hipError_t launch_sparse_mla(const MlaArgs &a, hipStream_t s);

// Sparse MLA with 64 heads of a query per workgroup (Dqk 576, Dv 512,
// Hq a multiple of 64).  With nchunk > 1 each query's index set is split
// into chunks of chunk_rows positions; every chunk writes its normalised
// output (bf16 [B*Lq][nchunk][Hq][512]) and log2-sum-exp (fp32
// [B*Lq][nchunk][Hq]) to part_o / part_lse and a merge kernel combines them.
struct MlaWideArgs {
    const void *q, *kv;
    const int32_t *t;
    void *out;
    float *lse;
    float sm_scale;
    int B, Lq, Lk, Hq, topk;
    int nchunk, chunk_rows;
    void *part_o;
    float *part_lse;
};
struct MlaWidePlan {
    bool ok;            // the shape is served by the wide kernel
    int nchunk, chunk_rows;
    size_t ws_bytes;    // partial outputs, 0 when nchunk == 1
};
constexpr int kMlaTargetWorkgroups = 256;   // one per compute unit of MI355X
MlaWidePlan mla_wide_plan(int B, int Lq, int Hq, int Dqk, int Dv, int topk);
hipError_t launch_sparse_mla_wide(const MlaWideArgs &a, hipStream_t s);

}  // namespace idxc
