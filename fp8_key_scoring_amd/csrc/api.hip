// C ABI of libfp8idx (declared in include/fp8idx.h): host-side argument
// checks, workspace layout and the kernel launch sequence.  Everything is
// enqueued on the caller's stream; nothing is allocated or synchronised.
#include "fp8idx.h"
#include "common.h"

#include <atomic>
#include <cstring>
#include <mutex>

using namespace fp8idx;

namespace {

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_problem(const fp8idx_problem_t *p) {
    if (!p) return FP8IDX_EINVAL;
    if (p->rows < 1 || p->rows > 65535) return FP8IDX_EINVAL;
    if (p->topk < 1 || p->topk > FP8IDX_MAX_TOPK) return FP8IDX_EINVAL;
    if (p->max_bound < 0) return FP8IDX_EINVAL;
    return FP8IDX_OK;
}

int check_score_inputs(const fp8idx_problem_t *p, const void *q, const float *w,
                       const uint8_t *k8, const float *ks, const int32_t *pt,
                       const int32_t *row_pt, const int32_t *row_bound) {
    if (p->num_pages < 1 || p->pt_rows < 1 || p->pt_stride < 1) return FP8IDX_EINVAL;
    if ((int64_t)p->max_bound > (int64_t)p->pt_stride * FP8IDX_PAGE) return FP8IDX_EINVAL;
    if (!q || !w || !k8 || !ks || !pt || !row_pt || !row_bound) return FP8IDX_EINVAL;
    if (!aligned(q, 16) || !aligned(w, 16) || !aligned(k8, 16) || !aligned(ks, 4) ||
        !aligned(pt, 4) || !aligned(row_pt, 4) || !aligned(row_bound, 4))
        return FP8IDX_EINVAL;
    return FP8IDX_OK;
}

// gfx950 check, cached per device id.
std::atomic<int> g_dev_ok[64];

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FP8IDX_EDEVICE;
    if (dev < 64) {
        int c = g_dev_ok[dev].load(std::memory_order_relaxed);
        if (c == 1) return FP8IDX_OK;
        if (c == 2) return FP8IDX_EDEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FP8IDX_EDEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) g_dev_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? FP8IDX_OK : FP8IDX_EDEVICE;
}

int score_chunk(const fp8idx_problem_t *p) {
    // aim at about one workgroup per CU (256 CUs) on the longest request group
    const int64_t groups = (p->rows + kGroupRows - 1) / kGroupRows;
    int64_t ch = groups * (int64_t)p->max_bound / 256;
    ch = (ch + 63) / 64 * 64;
    if (ch < 256) ch = 256;
    if (ch > 4096) ch = 4096;   // the score kernel keeps a chunk's <= 64 page ids in one VGPR
    return (int)ch;
}

ScoreArgs make_score_args(const fp8idx_problem_t *p, const void *q, const float *w,
                          const uint8_t *k8, const float *ks, const int32_t *pt,
                          const int32_t *row_pt, const int32_t *row_bound, float *scores,
                          int64_t sstride, uint32_t *hist1) {
    ScoreArgs a;
    a.q = (const uint16_t *)q;
    a.w = w;
    a.k8 = k8;
    a.kscale = ks;
    a.page_table = pt;
    a.row_pt = row_pt;
    a.row_bound = row_bound;
    a.scores = scores;
    a.hist1 = hist1;
    a.sstride = sstride;
    a.rows = p->rows;
    a.num_pages = p->num_pages;
    a.pt_rows = p->pt_rows;
    a.pt_stride = p->pt_stride;
    a.max_bound = p->max_bound;
    a.chunk = score_chunk(p);
    return a;
}

int to_code(hipError_t e) { return e == hipSuccess ? FP8IDX_OK : FP8IDX_ELAUNCH; }

int run_select(const fp8idx_problem_t *p, const float *scores, int64_t sstride,
               const int32_t *row_bound, int32_t *out_idx, unsigned char *ws,
               const WsLayout &L, bool need_hist1, hipStream_t st) {
    SelectArgs a;
    a.scores = scores;
    a.row_bound = row_bound;
    a.out_idx = out_idx;
    a.ws = ws;
    a.L = L;
    a.sstride = sstride;
    a.rows = p->rows;
    a.max_bound = p->max_bound;
    a.topk = p->topk;
    hipError_t e = hipSuccess;
    // short rows: one kernel, one workgroup per row
    if (p->max_bound <= kSmallMax) return to_code(launch_select_small(a, need_hist1, st));
    if (need_hist1 && (e = launch_hist1(a, st)) != hipSuccess) return to_code(e);
    if ((e = launch_refine(a, st)) != hipSuccess) return to_code(e);
    if ((e = launch_gather(a, st)) != hipSuccess) return to_code(e);
    return to_code(launch_finalize(a, st));
}

constexpr int kStageScore = 1, kStageSelect = 2;

// Scoring with the selection's digit counts into the workspace (kStageScore)
// and/or the selection from those counts (kStageSelect); every check before
// anything is enqueued.  zero_rows: the workspace's zero-block layout (0 for
// a caller's workspace).
int launch_checked(const fp8idx_problem_t *p, const void *q_bf16, const float *w, const uint8_t *k_e4m3,
                   const float *k_scale, const int32_t *page_table, const int32_t *row_pt,
                   const int32_t *row_bound, float *scores, int32_t *out_idx, void *ws, size_t ws_bytes,
                   int zero_rows, int stages, hipStream_t st) {
    int rc = check_problem(p);
    if (rc) return rc;
    rc = check_score_inputs(p, q_bf16, w, k_e4m3, k_scale, page_table, row_pt, row_bound);
    if (rc) return rc;
    if ((stages & kStageSelect) && (!out_idx || !aligned(out_idx, 4))) return FP8IDX_EINVAL;
    if (scores && (!aligned(scores, 4) || p->score_stride < p->max_bound)) return FP8IDX_EINVAL;
    const WsLayout L = ws_layout(p->rows, p->max_bound, scores == nullptr, zero_rows);
    if (!ws || !aligned(ws, 256) || ws_bytes < L.total) return FP8IDX_EWORKSPACE;
    rc = check_device();
    if (rc) return rc;
    unsigned char *wsb = (unsigned char *)ws;
    float *sc = scores ? scores : (float *)(wsb + L.scores);
    const int64_t sstride = scores ? p->score_stride : L.sstride;
    if (stages & kStageScore) {
        ScoreArgs a = make_score_args(p, q_bf16, w, k_e4m3, k_scale, page_table, row_pt, row_bound,
                                      sc, sstride, (uint32_t *)(wsb + L.hist1));
        rc = to_code(launch_score(a, st));
        if (rc) return rc;
    }
    if (stages & kStageSelect) return run_select(p, sc, sstride, row_bound, out_idx, wsb, L, false, st);
    return FP8IDX_OK;
}

}  // namespace

extern "C" {

int fp8idx_abi_version(void) { return FP8IDX_ABI_VERSION; }

const char *fp8idx_strerror(int code) {
    switch (code) {
    case FP8IDX_OK: return "ok";
    case FP8IDX_EINVAL: return "invalid argument";
    case FP8IDX_EWORKSPACE: return "workspace missing or too small";
    case FP8IDX_ELAUNCH: return "kernel launch failed";
    case FP8IDX_EDEVICE: return "no gfx950 device is current";
    case FP8IDX_ESCRATCH: return "problem larger than the static scratch of indexer_launch_static";
    default: return "unknown error";
    }
}

int fp8idx_workspace_size(const fp8idx_problem_t *p, int scores_in_workspace, size_t *bytes) {
    int rc = check_problem(p);
    if (rc) return rc;
    if (!bytes) return FP8IDX_EINVAL;
    *bytes = ws_layout(p->rows, p->max_bound, scores_in_workspace != 0).total;
    return FP8IDX_OK;
}

int fp8idx_workspace_init(void *ws, size_t ws_bytes, void *stream) {
    if (!ws || !aligned(ws, 256) || ws_bytes % 4) return FP8IDX_EINVAL;
    int rc = check_device();
    if (rc) return rc;
    return to_code(launch_fill_zero(ws, ws_bytes, (hipStream_t)stream));
}

int indexer_score(const fp8idx_problem_t *p, const void *q_bf16, const float *w,
                  const uint8_t *k_e4m3, const float *k_scale, const int32_t *page_table,
                  const int32_t *row_pt, const int32_t *row_bound, float *scores,
                  void *stream) {
    int rc = check_problem(p);
    if (rc) return rc;
    rc = check_score_inputs(p, q_bf16, w, k_e4m3, k_scale, page_table, row_pt, row_bound);
    if (rc) return rc;
    if (!scores || !aligned(scores, 4) || p->score_stride < p->max_bound) return FP8IDX_EINVAL;
    rc = check_device();
    if (rc) return rc;
    ScoreArgs a = make_score_args(p, q_bf16, w, k_e4m3, k_scale, page_table, row_pt, row_bound,
                                  scores, p->score_stride, nullptr);
    return to_code(launch_score(a, (hipStream_t)stream));
}

int indexer_topk(const fp8idx_problem_t *p, const float *scores, const int32_t *row_bound,
                 int32_t *out_idx, void *ws, size_t ws_bytes, void *stream) {
    int rc = check_problem(p);
    if (rc) return rc;
    if (!scores || !row_bound || !out_idx) return FP8IDX_EINVAL;
    if (!aligned(scores, 4) || !aligned(row_bound, 4) || !aligned(out_idx, 4)) return FP8IDX_EINVAL;
    if (p->score_stride < p->max_bound) return FP8IDX_EINVAL;
    const WsLayout L = ws_layout(p->rows, p->max_bound, false);
    if (!ws || !aligned(ws, 256) || ws_bytes < L.total) return FP8IDX_EWORKSPACE;
    rc = check_device();
    if (rc) return rc;
    return run_select(p, scores, p->score_stride, row_bound, out_idx, (unsigned char *)ws, L,
                      true, (hipStream_t)stream);
}

int indexer_launch(const fp8idx_problem_t *p, const void *q_bf16, const float *w,
                   const uint8_t *k_e4m3, const float *k_scale, const int32_t *page_table,
                   const int32_t *row_pt, const int32_t *row_bound, float *scores,
                   int32_t *out_idx, void *ws, size_t ws_bytes, void *stream) {
    return launch_checked(p, q_bf16, w, k_e4m3, k_scale, page_table, row_pt, row_bound, scores, out_idx, ws,
                          ws_bytes, 0, kStageScore | kStageSelect, (hipStream_t)stream);
}

int indexer_launch_score(const fp8idx_problem_t *p, const void *q_bf16, const float *w,
                         const uint8_t *k_e4m3, const float *k_scale, const int32_t *page_table,
                         const int32_t *row_pt, const int32_t *row_bound, float *scores,
                         void *ws, size_t ws_bytes, void *stream) {
    return launch_checked(p, q_bf16, w, k_e4m3, k_scale, page_table, row_pt, row_bound, scores, nullptr, ws,
                          ws_bytes, 0, kStageScore, (hipStream_t)stream);
}

int indexer_launch_select(const fp8idx_problem_t *p, const float *scores, const int32_t *row_bound,
                          int32_t *out_idx, void *ws, size_t ws_bytes, void *stream) {
    int rc = check_problem(p);
    if (rc) return rc;
    if (!row_bound || !aligned(row_bound, 4) || !out_idx || !aligned(out_idx, 4)) return FP8IDX_EINVAL;
    if (scores && (!aligned(scores, 4) || p->score_stride < p->max_bound)) return FP8IDX_EINVAL;
    const WsLayout L = ws_layout(p->rows, p->max_bound, scores == nullptr);
    if (!ws || !aligned(ws, 256) || ws_bytes < L.total) return FP8IDX_EWORKSPACE;
    rc = check_device();
    if (rc) return rc;
    unsigned char *wsb = (unsigned char *)ws;
    const float *sc = scores ? scores : (const float *)(wsb + L.scores);
    const int64_t sstride = scores ? p->score_stride : L.sstride;
    return run_select(p, sc, sstride, row_bound, out_idx, wsb, L, false, (hipStream_t)stream);
}

// ---- The launch with the library's own scratch in place of a workspace.
// scratch: file-scope device memory, one copy per GPU the library runs on
// (the runtime places it when the code object is loaded and keeps it until
// the process ends).  Its host-side name is not a device address: host code
// uses only the per-device address hipGetSymbolAddress returns.
constexpr size_t kScratchBytes = (size_t)FP8IDX_STATIC_SCRATCH_BYTES;
constexpr int kScratchRows = FP8IDX_STATIC_MAX_ROWS;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
unsigned char *g_scratch_ptr[64];   // per device: the scratch's device address (null: not set up)
bool g_scratch_dirty[64];           // per device: a call failed after enqueueing work; clear again
}  // namespace

int indexer_launch_static(const fp8idx_problem_t *p, const void *q_bf16, const float *w,
                          const uint8_t *k_e4m3, const float *k_scale, const int32_t *page_table,
                          const int32_t *row_pt, const int32_t *row_bound, float *scores,
                          int32_t *out_idx, void *stream) {
    int rc = check_problem(p);
    if (rc) return rc;
    if (p->rows > kScratchRows) return FP8IDX_ESCRATCH;
    if (ws_layout(p->rows, p->max_bound, scores == nullptr, kScratchRows).total > kScratchBytes)
        return FP8IDX_ESCRATCH;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return FP8IDX_EDEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    unsigned char *ws = g_scratch_ptr[dev];
    const size_t zero_bytes = ws_layout(1, 1, false, kScratchRows).state;
    if (!ws) {
        // set-up, once per device with that device current: the scratch's
        // address on this device, and its zero block cleared (a fill
        // kernel) ahead of the first launch on the caller's stream
        rc = check_device();
        if (rc) return rc;
        void *addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return FP8IDX_ELAUNCH;
        g_scratch_ptr[dev] = ws = (unsigned char *)addr;
        g_scratch_dirty[dev] = true;
    }
    if (g_scratch_dirty[dev]) {
        if (launch_fill_zero(ws, zero_bytes, (hipStream_t)stream) != hipSuccess) return FP8IDX_ELAUNCH;
        g_scratch_dirty[dev] = false;
    }
    rc = launch_checked(p, q_bf16, w, k_e4m3, k_scale, page_table, row_pt, row_bound, scores, out_idx, ws,
                        kScratchBytes, kScratchRows, kStageScore | kStageSelect, (hipStream_t)stream);
    // a launch error after the scoring pass was enqueued can leave counts in
    // the zero block: the next call clears it first
    if (rc == FP8IDX_ELAUNCH) g_scratch_dirty[dev] = true;
    return rc;
}

int fp8idx_attention_workspace_size(const fp8idx_problem_t *p, size_t *bytes) {
    int rc = check_problem(p);
    if (rc) return rc;
    if (!bytes) return FP8IDX_EINVAL;
    *bytes = attn_workspace_bytes(p->rows, p->topk);
    return FP8IDX_OK;
}

int indexer_sparse_attention(const fp8idx_problem_t *p, const void *q_bf16, const void *kv_bf16,
                             const int32_t *page_table, const int32_t *row_pt, const int32_t *sel,
                             float sm_scale, float *out, float *lse, void *ws, size_t ws_bytes, void *stream) {
    int rc = check_problem(p);
    if (rc) return rc;
    if (p->num_pages < 1 || p->pt_rows < 1 || p->pt_stride < 1) return FP8IDX_EINVAL;
    if ((int64_t)p->max_bound > (int64_t)p->pt_stride * FP8IDX_PAGE) return FP8IDX_EINVAL;
    if (!q_bf16 || !kv_bf16 || !page_table || !row_pt || !sel || !out || !lse) return FP8IDX_EINVAL;
    if (!aligned(q_bf16, 16) || !aligned(kv_bf16, 16) || !aligned(page_table, 4) || !aligned(row_pt, 4) ||
        !aligned(sel, 4) || !aligned(out, 4) || !aligned(lse, 4))
        return FP8IDX_EINVAL;
    if (!(sm_scale == sm_scale) || sm_scale == INFINITY || sm_scale == -INFINITY) return FP8IDX_EINVAL;
    if ((int64_t)p->num_pages * FP8IDX_PAGE > INT32_MAX) return FP8IDX_EINVAL;   // cache rows as int32
    const size_t need = attn_workspace_bytes(p->rows, p->topk);
    if (!ws || !aligned(ws, 256) || ws_bytes < need) return FP8IDX_EWORKSPACE;
    rc = check_device();
    if (rc) return rc;
    AttnArgs a;
    a.q = (const uint16_t *)q_bf16;
    a.kv = (const uint16_t *)kv_bf16;
    a.page_table = page_table;
    a.row_pt = row_pt;
    a.sel = sel;
    a.out = out;
    a.lse = lse;
    int n, sp;
    attn_split(p->rows, p->topk, &n, &sp);
    a.part_o = (float *)ws;
    a.part_ml = (float *)((unsigned char *)ws + align_up((size_t)p->rows * n * kAttnHeads * kAttnVDim * 4, 256));
    a.sm_scale = sm_scale;
    a.rows = p->rows;
    a.topk = p->topk;
    a.span = sp;
    a.nsplit = n;
    a.num_pages = p->num_pages;
    a.pt_rows = p->pt_rows;
    a.pt_stride = p->pt_stride;
    a.max_bound = p->max_bound;
    return to_code(launch_attention(a, (hipStream_t)stream));
}

int indexer_validate(const fp8idx_problem_t *p, const int32_t *page_table, const int32_t *row_pt,
                     const int32_t *row_bound, uint32_t *status, void *stream) {
    int rc = check_problem(p);
    if (rc) return rc;
    if (p->num_pages < 1 || p->pt_rows < 1 || p->pt_stride < 1) return FP8IDX_EINVAL;
    if ((int64_t)p->max_bound > (int64_t)p->pt_stride * FP8IDX_PAGE) return FP8IDX_EINVAL;
    if (!page_table || !row_pt || !row_bound || !status) return FP8IDX_EINVAL;
    if (!aligned(page_table, 4) || !aligned(row_pt, 4) || !aligned(row_bound, 4) || !aligned(status, 4))
        return FP8IDX_EINVAL;
    rc = check_device();
    if (rc) return rc;
    return to_code(launch_validate(page_table, row_pt, row_bound, status, p->rows, p->num_pages, p->pt_rows,
                                   p->pt_stride, p->max_bound, (hipStream_t)stream));
}

int indexer_write_keys(const fp8idx_problem_t *p, const void *k_new_bf16, uint8_t *k_e4m3,
                       float *k_scale, const int32_t *page_table, const int32_t *row_pt,
                       const int32_t *row_bound, void *stream) {
    int rc = check_problem(p);
    if (rc) return rc;
    if (p->num_pages < 1 || p->pt_rows < 1 || p->pt_stride < 1) return FP8IDX_EINVAL;
    if ((int64_t)p->max_bound > (int64_t)p->pt_stride * FP8IDX_PAGE) return FP8IDX_EINVAL;
    if (!k_new_bf16 || !k_e4m3 || !k_scale || !page_table || !row_pt || !row_bound) return FP8IDX_EINVAL;
    if (!aligned(k_new_bf16, 4) || !aligned(k_e4m3, 16) || !aligned(k_scale, 4) || !aligned(page_table, 4) ||
        !aligned(row_pt, 4) || !aligned(row_bound, 4))
        return FP8IDX_EINVAL;
    rc = check_device();
    if (rc) return rc;
    return to_code(launch_write_keys((const uint16_t *)k_new_bf16, k_e4m3, k_scale, page_table, row_pt,
                                     row_bound, p->rows, p->num_pages, p->pt_rows, p->pt_stride,
                                     p->max_bound, (hipStream_t)stream));
}

int indexer_launch_new_keys(const fp8idx_problem_t *p, const void *q_bf16, const float *w,
                            const void *k_new_bf16, uint8_t *k_e4m3, float *k_scale,
                            const int32_t *page_table, const int32_t *row_pt, const int32_t *row_bound,
                            float *scores, int32_t *out_idx, void *ws, size_t ws_bytes, void *stream) {
    // every check of both steps before anything is enqueued
    int rc = check_problem(p);
    if (rc) return rc;
    rc = check_score_inputs(p, q_bf16, w, k_e4m3, k_scale, page_table, row_pt, row_bound);
    if (rc) return rc;
    if (!k_new_bf16 || !aligned(k_new_bf16, 4)) return FP8IDX_EINVAL;
    if (!out_idx || !aligned(out_idx, 4)) return FP8IDX_EINVAL;
    if (scores && (!aligned(scores, 4) || p->score_stride < p->max_bound)) return FP8IDX_EINVAL;
    const WsLayout L = ws_layout(p->rows, p->max_bound, scores == nullptr);
    if (!ws || !aligned(ws, 256) || ws_bytes < L.total) return FP8IDX_EWORKSPACE;
    rc = indexer_write_keys(p, k_new_bf16, k_e4m3, k_scale, page_table, row_pt, row_bound, stream);
    if (rc) return rc;
    return indexer_launch(p, q_bf16, w, k_e4m3, k_scale, page_table, row_pt, row_bound, scores, out_idx,
                          ws, ws_bytes, stream);
}

static int check_shards(const fp8idx_problem_t *p, int shards) {
    if (shards < 1 || (int64_t)shards * p->topk > kMergeMaxCand) return FP8IDX_EINVAL;
    if ((int64_t)shards * ((int64_t)p->max_bound + FP8IDX_PAGE) >= ((int64_t)1 << 31)) return FP8IDX_EINVAL;
    return FP8IDX_OK;
}

int indexer_shard_candidates(const fp8idx_problem_t *p, int shard, int shards,
                             const float *scores, const int32_t *out_idx,
                             float *cand_score, int32_t *cand_idx, void *stream) {
    int rc = check_problem(p);
    if (rc) return rc;
    if ((rc = check_shards(p, shards))) return rc;
    if (shard < 0 || shard >= shards) return FP8IDX_EINVAL;
    if (!scores || !out_idx || !cand_score || !cand_idx) return FP8IDX_EINVAL;
    if (!aligned(scores, 4) || !aligned(out_idx, 4) || !aligned(cand_score, 4) || !aligned(cand_idx, 4))
        return FP8IDX_EINVAL;
    if (p->score_stride < p->max_bound) return FP8IDX_EINVAL;
    rc = check_device();
    if (rc) return rc;
    return to_code(launch_shard_cand(scores, p->score_stride, out_idx, p->rows, p->topk, shard, shards,
                                     cand_score, cand_idx, (hipStream_t)stream));
}

int indexer_merge_topk(const fp8idx_problem_t *p, int shards,
                       const float *cand_score, const int32_t *cand_idx,
                       int32_t *out_idx, void *stream) {
    int rc = check_problem(p);
    if (rc) return rc;
    if ((rc = check_shards(p, shards))) return rc;
    if (!cand_score || !cand_idx || !out_idx) return FP8IDX_EINVAL;
    if (!aligned(cand_score, 16) || !aligned(cand_idx, 16) || !aligned(out_idx, 4)) return FP8IDX_EINVAL;
    if ((shards * p->topk) % 16) return FP8IDX_EINVAL;
    rc = check_device();
    if (rc) return rc;
    return to_code(launch_merge(p->rows, shards * p->topk, p->topk, cand_score, cand_idx, out_idx,
                                (hipStream_t)stream));
}

}  // extern "C"
