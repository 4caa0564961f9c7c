/*
 * fp8idx — paged FP8-E4M3 decode indexer for MI355X (gfx950).  C ABI.
 *
 * The operation is the long-context decode indexer launch described on the
 * sglang pull request page "sgl-project/sglang#48224" (the sgl-amd-mono #86
 * commit body, Motivation): every cached key of each query row is scored and
 * each row's exact top-2048 keys are selected.  The score of logical key s for
 * row r is
 *
 *     score(r, s) = k_scale(s) * sum_{h<64} w[r][h] * max(q[r][h] . k(s), 0)
 *
 * with 64 index heads of 128 dims, q in bf16, k(s) the key's 128 E4M3 codes
 * (decoded exactly) and k_scale(s) its fp32 scale (the same page, Modifications
 * row 2: four 8-byte loads and the scale per 16-key group, i.e. 128 code bytes
 * plus one scale per key).  Keys at or past a row's bound are neither scored
 * nor selected (Modifications row 2: the store's mask drops them), so the
 * bound is exclusive.
 *
 * Layouts (all row-major and contiguous unless a stride is given):
 *   q           [rows][64][128]         bf16 (raw 16-bit patterns), 16-B aligned
 *   w           [rows][64]              fp32, 16-B aligned
 *   k_e4m3      [num_pages][64][128]    uint8 OCP E4M3FN codes, 16-B aligned
 *   k_scale     [num_pages][64]         fp32
 *   page_table  [pt_rows][pt_stride]    int32 physical page ids
 *   row_pt      [rows]                  int32 page-table row of each query row
 *   row_bound   [rows]                  int32 exclusive key bound, 0..max_bound
 *   scores      [rows][score_stride]    fp32; entry s written only for s < bound
 *   out_idx     [rows][topk]            int32 logical key indices
 * Logical key s of row r lives in page page_table[row_pt[r]][s / 64], slot
 * s % 64.  Only page-table entries below ceil(bound / 64) are read.
 *
 * Memory and ownership: every pointer argument except `p` is DEVICE memory
 * owned by the caller.  The library allocates nothing, frees nothing and never
 * synchronises; work is enqueued on `stream` (a hipStream_t; NULL = the
 * default stream) and the call returns without waiting.  The workspace must
 * be zero-filled once before first use (fp8idx_workspace_init does that on the
 * stream); every launch leaves it zero-filled again, so it can be reused by
 * later launches on the same stream, also for other problem shapes as long as
 * rows <= 256 (above that, re-initialise it when the row count grows).
 * Concurrent launches must not share one workspace.
 *
 * Device arrays are trusted for sizes: row_bound[r] must be <= max_bound and
 * row_pt[r] < pt_rows; values outside are clamped (bound) or make the row
 * produce NaN scores (page-table row).  A page id outside [0, num_pages) is
 * never dereferenced: the keys it covers score NaN.
 *
 * Errors: every call returns 0 on success or a negative FP8IDX_E* code.  All
 * argument checks happen on the host before any device work is enqueued; an
 * error return means nothing was enqueued (except FP8IDX_ELAUNCH, reported by
 * the HIP runtime after an enqueue was attempted).  No exception crosses the
 * ABI.
 */
#ifndef FP8IDX_H
#define FP8IDX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8IDX_ABI_VERSION 1
#define FP8IDX_HEADS 64
#define FP8IDX_HEAD_DIM 128
#define FP8IDX_PAGE 64
#define FP8IDX_MAX_TOPK 2048
/* Limits of indexer_launch_static's scratch (one per GPU): at most this many
 * rows, and a workspace layout of at most this many bytes. */
#define FP8IDX_STATIC_MAX_ROWS 256
#define FP8IDX_STATIC_SCRATCH_BYTES (64u << 20)

enum {
    FP8IDX_OK = 0,
    FP8IDX_EINVAL = -1,     /* invalid argument (null pointer, size, alignment) */
    FP8IDX_EWORKSPACE = -2, /* workspace null or smaller than fp8idx_workspace_size */
    FP8IDX_ELAUNCH = -3,    /* the HIP runtime reported an error for a launch */
    FP8IDX_EDEVICE = -4,    /* current device is not gfx950 / no device */
    FP8IDX_ESCRATCH = -5    /* problem larger than indexer_launch_static's scratch */
};

/* Problem descriptor (plain data, passed by host pointer).
 *   rows         query rows (>= 1, <= 65535)
 *   num_pages    pages in the key pool (>= 1)
 *   pt_rows      rows of the page table (>= 1)
 *   pt_stride    entries per page-table row (>= 1)
 *   max_bound    upper bound of every row_bound (0 .. pt_stride*64)
 *   topk         keys selected per row (1 .. 2048)
 *   score_stride elements between score rows (>= max_bound when scores are
 *                passed; ignored when they are not) */
typedef struct fp8idx_problem {
    int32_t rows;
    int32_t num_pages;
    int32_t pt_rows;
    int32_t pt_stride;
    int32_t max_bound;
    int32_t topk;
    int64_t score_stride;
} fp8idx_problem_t;

/* ABI version of the loaded library (FP8IDX_ABI_VERSION it was built with). */
int fp8idx_abi_version(void);

/* Static message for an error code (never NULL). */
const char *fp8idx_strerror(int code);

/* Bytes of device workspace for `p` (written to *bytes).  With
 * scores_in_workspace != 0 the size includes room for the scores
 * (indexer_launch with scores == NULL); with 0 it covers indexer_topk and
 * indexer_launch with caller-provided scores.  The workspace pointer must be
 * 256-byte aligned.  Host-only; touches no device. */
int fp8idx_workspace_size(const fp8idx_problem_t *p, int scores_in_workspace, size_t *bytes);

/* Zero-fills `ws_bytes` bytes (a multiple of 4) of workspace with a fill
 * kernel on `stream`. */
int fp8idx_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Scoring only (the same page, Motivation: every cached key is scored;
 * Modifications rows 1-2: FP8 -> bf16 conversion, the head reduction, the
 * per-key scale loaded with each 16-key group, the mask at the store):
 * scores[r][s] for every s < row_bound[r] (the causal mask at
 * the store); entries at or past the bound are left untouched.  Rows that
 * share a page-table row and sit next to each other in the launch are scored
 * together (each key is read from HBM once for the group).
 * score_stride must be >= max_bound.  No workspace. */
int indexer_score(const fp8idx_problem_t *p,
                  const void *q_bf16, const float *w,
                  const uint8_t *k_e4m3, const float *k_scale,
                  const int32_t *page_table, const int32_t *row_pt,
                  const int32_t *row_bound,
                  float *scores, void *stream);

/* Selection only (the same page, Motivation: the exact top-2048 per row;
 * Modifications row 4: a radix select whose first digit is radix_key >> 26):
 * for each row, the exact top-topk of scores[r][0..bound)
 * (descending value; equal values go to the lower key index; NaN ranks below
 * every number; -0 equals +0).  out_idx[r] receives the selected logical
 * indices in ascending index order; with fewer than topk keys all of them
 * are returned and the remaining slots hold -1.  Uses p->rows, max_bound,
 * topk and score_stride. */
int indexer_topk(const fp8idx_problem_t *p,
                 const float *scores, const int32_t *row_bound,
                 int32_t *out_idx, void *ws, size_t ws_bytes, void *stream);

/* The fused launch (the same page, Motivation and Modifications rows 1-4:
 * scoring with the selection's first radix digit counted in the scoring
 * pass, then the exact top-k): scoring followed by selection.  `scores` may be NULL (then the
 * scores live in the workspace); when given, it receives exactly what
 * indexer_score writes.  out_idx as for indexer_topk. */
int indexer_launch(const fp8idx_problem_t *p,
                   const void *q_bf16, const float *w,
                   const uint8_t *k_e4m3, const float *k_scale,
                   const int32_t *page_table, const int32_t *row_pt,
                   const int32_t *row_bound,
                   float *scores, int32_t *out_idx,
                   void *ws, size_t ws_bytes, void *stream);

/* The two stages of indexer_launch as separate calls (indexer_launch is
 * exactly indexer_launch_score followed by indexer_launch_select on one
 * stream and workspace).  For callers that put work between the stages or
 * time them apart.
 *
 * indexer_launch_score: the scoring pass of the fused launch (the same page,
 * Motivation and Modifications rows 1-2 for the scoring; row 4 for counting
 * the selection's first radix digit while scoring): scores as indexer_score
 * writes them (into the workspace when `scores` is NULL) and the per-row
 * radix-digit counts the selection reads, added into the workspace's zero
 * block.  Arguments as for indexer_launch without out_idx.
 *
 * indexer_launch_select: the selection from those scores and counts: out_idx
 * as for indexer_topk; the counts are consumed and the zero block left zero.
 * `scores` must be the pointer (or NULL, for scores in the workspace) and
 * p->score_stride the stride given to indexer_launch_score; p, row_bound and
 * the workspace must be the same.
 *
 * Exactly one indexer_launch_select must follow each indexer_launch_score on
 * a workspace before the workspace is used again (two scoring passes in a row
 * add their counts together; fp8idx_workspace_init restores a workspace).
 * Errors as for indexer_launch. */
int indexer_launch_score(const fp8idx_problem_t *p,
                         const void *q_bf16, const float *w,
                         const uint8_t *k_e4m3, const float *k_scale,
                         const int32_t *page_table, const int32_t *row_pt,
                         const int32_t *row_bound,
                         float *scores, void *ws, size_t ws_bytes, void *stream);

int indexer_launch_select(const fp8idx_problem_t *p,
                          const float *scores, const int32_t *row_bound,
                          int32_t *out_idx, void *ws, size_t ws_bytes, void *stream);

/* indexer_launch without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors as
 * indexer_launch; the workspace is the library's own static scratch of
 * FP8IDX_STATIC_SCRATCH_BYTES (64 MiB) of device memory per GPU, held by each
 * GPU the library runs on until the process ends.  The call allocates
 * nothing.  Its first call on a GPU looks up that GPU's scratch and clears
 * its counters with a fill kernel on `stream`; every call leaves them clear.
 *
 * Limits: p->rows <= FP8IDX_STATIC_MAX_ROWS and the workspace the problem
 * needs (fp8idx_workspace_size, with the counters laid out for 256 rows; with
 * scores == NULL the scores live there too) at most 64 MiB; a larger problem
 * returns FP8IDX_ESCRATCH before anything is enqueued.  All calls on one GPU
 * share its scratch: calls that may overlap on the GPU (on different streams
 * without ordering between them, or from several threads) race and give
 * undefined results; order them on one stream. */
int indexer_launch_static(const fp8idx_problem_t *p,
                          const void *q_bf16, const float *w,
                          const uint8_t *k_e4m3, const float *k_scale,
                          const int32_t *page_table, const int32_t *row_pt,
                          const int32_t *row_bound,
                          float *scores, int32_t *out_idx, void *stream);

/* Checks the device arrays the calls above trust and writes a status word to
 * `status` (one device uint32, 4-byte aligned; zeroed by this call first, then
 * OR-ed): bit 0 (1) some row_bound outside [0, max_bound]; bit 1 (2) some
 * row_pt outside [0, pt_rows); bit 2 (4) some page id a row would read (its
 * page-table entries below ceil(min(bound, max_bound) / 64)) outside
 * [0, num_pages).  0 = every array is within range.  The launches stay safe
 * on such values (bounds clamped, bad page-table rows or page ids score NaN);
 * this call reports them, in place of a separate debug build.  Uses p->rows,
 * num_pages, pt_rows, pt_stride, max_bound.  Errors: -1 for a null or
 * misaligned pointer or the problem checks of indexer_score.  No workspace. */
int indexer_validate(const fp8idx_problem_t *p, const int32_t *page_table,
                     const int32_t *row_pt, const int32_t *row_bound,
                     uint32_t *status, void *stream);

/* ---- New keys (the same page, Modifications row 2 and the Reviewer notes
 * on new keys: the launch writes keys into the cache and every row of the
 * request scores them).  Row r's own key k_new[r] (128 bf16 elements) is
 * quantized and written at logical position bound[r] - 1 of its page-table
 * row: page page_table[row_pt[r]][(bound - 1) / 64], slot (bound - 1) % 64,
 * 128 codes into k_e4m3 and one scale into k_scale.  Quantization (the pages
 * give none; the plain per-key rule): scale = amax / 448 in fp32 with amax
 * the key's largest magnitude (scale 1 and all codes 0 for an all-zero key),
 * code = the OCP E4M3FN value nearest to the fp32 quotient k / scale, ties to
 * the even code.  k_new elements must be finite.
 *
 * Layout: k_new [rows][128] bf16, 4-byte aligned.  A row with bound 0 (after
 * clamping to [0, max_bound]), a page-table row outside [0, pt_rows) or a
 * page id outside [0, num_pages) writes nothing.  When two rows name the same
 * slot, which of their keys lands there is unspecified.  Errors: -1 for a
 * null or misaligned pointer, or the problem checks of indexer_score. */
int indexer_write_keys(const fp8idx_problem_t *p, const void *k_new_bf16,
                       uint8_t *k_e4m3, float *k_scale,
                       const int32_t *page_table, const int32_t *row_pt,
                       const int32_t *row_bound, void *stream);

/* indexer_write_keys followed by indexer_launch on the same stream: the rows
 * score the cache with the launch's new keys in it (each row's own key and
 * those of the rows before it in the request).  Arguments as for the two
 * calls; every check of both happens before anything is enqueued. */
int indexer_launch_new_keys(const fp8idx_problem_t *p,
                            const void *q_bf16, const float *w, const void *k_new_bf16,
                            uint8_t *k_e4m3, float *k_scale,
                            const int32_t *page_table, const int32_t *row_pt,
                            const int32_t *row_bound,
                            float *scores, int32_t *out_idx,
                            void *ws, size_t ws_bytes, void *stream);

/* ---- Key-sharded selection (the context split over G shards by page).
 * Shard g of G (0 <= g < G) holds pages g, g+G, g+2G, ... of every request
 * in its own page table and runs indexer_launch (with `scores`) on them; its
 * logical key s is global key 64 * (g + G * (s / 64)) + s % 64 (the release
 * test-suite page for GLM-5.2: 64-key pages interleaved over ranks, a
 * top-k owner merge).  Every key scores the same in any shard, so the exact
 * top-k of the union of the shards' top-k sets is the row's global top-k. */

/* Step 1, per shard: turns shard g's selection out_idx [rows][topk] (its
 * logical indices, -1 padded) and its scores [rows][score_stride] into
 * (score, global index) candidates at cand_score / cand_idx
 * [rows][shards][topk], block g; empty slots get index -1.  Uses p->rows,
 * max_bound, topk, score_stride of the shard's problem.  Errors: -1 for a
 * null or misaligned pointer, shard outside [0, shards), shards * topk above
 * 16384, or global indices that would not fit in int32
 * (shards * (max_bound + 64) >= 2^31).  No workspace. */
int indexer_shard_candidates(const fp8idx_problem_t *p, int shard, int shards,
                             const float *scores, const int32_t *out_idx,
                             float *cand_score, int32_t *cand_idx, void *stream);

/* Step 2, once the candidates of all shards are in one place: out_idx
 * [rows][topk] receives each row's exact top-topk of its shards * topk
 * candidates (descending score, equal scores to the lower global index, NaN
 * below every number) as global indices in candidate-slot order (grouped by
 * shard, shard 0 first; ascending within a shard for the candidates step 1
 * writes), -1 padded when fewer than topk candidates exist.  Uses p->rows and
 * p->topk.  cand_score and cand_idx must be 16-byte aligned and shards * topk
 * a multiple of 16.  Errors as for step 1 (-1 also for those).  No
 * workspace. */
int indexer_merge_topk(const fp8idx_problem_t *p, int shards,
                       const float *cand_score, const int32_t *cand_idx,
                       int32_t *out_idx, void *stream);

/* ---- Sparse attention over each row's selected keys: the step the indexer
 * feeds (the same sglang page, Motivation: the exact top-2048 keys of each
 * row are picked for the attention after it; the release test-suite page for
 * GLM-5.2 runs that step as MLA sparse attention over a DeepSeek-style latent
 * cache).  The pages give no formula or shapes; the reading is absorbed
 * multi-head latent attention at decode:
 *   kv          [num_pages][64][576]   bf16 latent cache (512 latent + 64
 *                                      rotary values per key), 16-B aligned,
 *                                      paged by the same page_table / row_pt
 *                                      as the index keys
 *   q_bf16      [rows][16][576]        bf16 absorbed queries, 16-B aligned
 *   sel         [rows][topk]           int32 logical key positions (the
 *                                      indexer's out_idx); -1 = none
 *   out         [rows][16][512]        fp32
 *   lse         [rows][16]             fp32
 * For row r and head h, over the selected positions j (an entry is skipped
 * when it is negative, at or past max_bound, or on a page id outside
 * [0, num_pages); a repeated position counts each time):
 *   l_j = sm_scale * q[r][h] . kv(j),   out[r][h] = sum_j e^{l_j} kv(j)[0..512) / sum_j e^{l_j},
 *   lse[r][h] = log sum_j e^{l_j};  nothing selected: out 0, lse -inf.
 * Logits are fp32 sums of exact bf16 products; the softmax weights enter the
 * value sum with about 16 significant bits; sums are fp32.
 *
 * Bytes of workspace for indexer_sparse_attention with p->rows and p->topk
 * (per-split partial outputs); host-only. */
int fp8idx_attention_workspace_size(const fp8idx_problem_t *p, size_t *bytes);

/* Enqueues the attention on `stream`.  Uses every field of `p` but
 * score_stride (rows, topk = entries per row of sel; num_pages, pt_rows,
 * pt_stride, max_bound as for the indexer).  `ws` (256-byte aligned, at least
 * fp8idx_attention_workspace_size bytes) is scratch: no initialisation is
 * needed and its contents are overwritten.  Errors: -1 for a null or
 * misaligned pointer, a non-finite sm_scale or a bad problem; -2 for a
 * missing or short workspace; row_pt entries outside [0, pt_rows) select
 * nothing. */
int indexer_sparse_attention(const fp8idx_problem_t *p, const void *q_bf16, const void *kv_bf16,
                             const int32_t *page_table, const int32_t *row_pt, const int32_t *sel,
                             float sm_scale, float *out, float *lse, void *ws, size_t ws_bytes,
                             void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8IDX_H */
