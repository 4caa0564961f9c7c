// Internal definitions shared by the HIP translation units of libfp8idx.
// Not part of the public ABI (include/fp8idx.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8idx {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kHeads = 64;
constexpr int kDim = 128;
constexpr int kPage = 64;
constexpr int kMaxTopk = 2048;

// Scoring: one workgroup = 4 waves; up to 4 rows that share a page-table row
// are scored together (each wave scores all of them on every fourth 16-key
// group, so each key is read from HBM once and converted once).
constexpr int kScoreThreads = 256;
constexpr int kGroupRows = 4;
constexpr int kKeysPerMfma = 16;   // one 16x16x32 MFMA column block = 16 keys

// Selection.
constexpr int kSelThreads = 1024;                   // 16 waves: 4 per SIMD hide LDS latency
constexpr int kSelUnroll = 8;                       // scores in flight per thread
constexpr int kSelTile = kSelThreads * kSelUnroll;  // keys per workgroup step
constexpr int kSelMaxWgs = 64;                      // selection workgroups per row (at most)
constexpr int kCandSlice = 1024;                    // candidates one gather workgroup keeps
constexpr int kSliceCap = kMaxTopk + kCandSlice;    // entries (sure keys + candidates) per gather workgroup
constexpr int kCandCap = 4096;                      // candidates one row may have (else fallback)
constexpr int kEntCap = kMaxTopk + kCandCap;        // entries of one row finalize holds
constexpr int kTieCap = 1024;                       // keys in the third-digit bin finalize ranks
// Launches whose rows all have at most this many keys select with one
// workgroup per row that holds the row's keys in registers (16 per thread);
// past it the multi-workgroup chain is faster (4 rows x 32,768 keys: 27.3
// against 32.6 us per launch).
constexpr int kSmallMax = 16384;
// Heavy ties (the threshold's third-digit bin holds more keys than finalize
// ranks): the last 10 bits of the keys in that bin are counted by up to
// kFbMaxWgs workgroups per row, each over its share of the row
constexpr int kFbBits = 10;
constexpr int kFbBins = 1 << kFbBits;
constexpr int kFbMaxWgs = 8;
constexpr int64_t kFbKeysPerWg = 65536;
constexpr int kZeroRows = 256;     // rows the zero block is laid out for (at least)
constexpr int kDigit1Bits = 6;      // first radix digit (counted while scoring)
constexpr int kDigit2Bits = 8;      // second radix digit
constexpr int kDigit1Shift = 32 - kDigit1Bits;               // 26
constexpr int kDigit2Shift = kDigit1Shift - kDigit2Bits;     // 18
constexpr int kDigit3Bits = 8;      // third radix digit (counted over the candidates)
constexpr int kDigit3Shift = kDigit2Shift - kDigit3Bits;     // 10
constexpr int kBins1 = 1 << kDigit1Bits;                     // 64
constexpr int kBins2 = 1 << kDigit2Bits;                     // 256
constexpr int kBins3 = 1 << kDigit3Bits;                     // 256
// A row's first-digit counts are spread over kHist1Slots copies (workgroup x
// adds into copy x % kHist1Slots): a row's scores fall into one or two bins,
// and hundreds of workgroups adding into one word would queue behind each
// other.  Readers sum the copies.
constexpr int kHist1Slots = 16;
// The same for the second-digit counts: the 64 refine workgroups of a row add
// ~a hundred bins each into the row's 256, and each bin would take one atomic
// per workgroup in turn; workgroup x adds into copy x % kHist2Slots.
constexpr int kHist2Slots = 8;

// Per-row selection state: b1 and above1 written by the first refine
// workgroup of a row, the rest by the first gather workgroup.
struct RowState {
    uint32_t b1;      // first-digit bin holding the k-th largest key
    uint32_t b2;      // second-digit bin inside b1 holding it
    uint32_t sure;    // keys whose top 14 bits exceed (b1, b2): all selected
    uint32_t need;    // keys still to take from the (b1, b2) bin
    uint32_t cand;    // keys in the (b1, b2) bin
    uint32_t above1;  // keys in first-digit bins above b1 (written with b1 by refine)
    uint32_t pad[2];
};

// Workspace layout.  The histograms must be zero before a launch; every
// launch leaves them zero again.  They sit in one block at the start, laid out
// for max(rows, kZeroRows) rows, so the block has the same offsets for every
// problem of up to kZeroRows rows and a workspace can be reused across problem
// shapes; the rest of the workspace is scratch that each launch writes before
// it reads.
struct WsLayout {
    size_t hist1;      // u32 [rz][kHist1Slots][64]  first-digit counts
    size_t hist2;      // u32 [rz][kHist2Slots][256]  second-digit counts inside the first-digit bin
    size_t hist3;      // u32 [rz][256]     third-digit counts of the candidates
    size_t fb_hist;    // u32 [rz][1024]    heavy-tie fallback: last-10-bit counts of the threshold bin
    size_t fb_cnt;     // u32 [rz]          finalize workgroups of the row that are done
    size_t state;      // RowState [rows]
    size_t ent_cnt;    // u32 [rows][sel_wgs]              entries (sure keys + candidates) per gather workgroup
    size_t cand_cnt;   // u32 [rows][sel_wgs]              candidates among them
    size_t ent_list;   // u64 [rows][sel_wgs][kSliceCap]   entries in ascending index: key << 32 | sure << 31 | index
    size_t scores;     // f32 [rows][sstride]  (only when the caller gives none)
    size_t total;
    int sel_wgs;
    int fb_wgs;        // finalize workgroups per row (1 .. kFbMaxWgs)
    int64_t sel_chunk;
    int64_t sstride;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// zero_rows: rows the zero block is laid out for; 0 means max(rows,
// kZeroRows) (a caller's workspace), a fixed value gives every problem of up
// to that many rows the same zero block (the library's static scratch).
inline WsLayout ws_layout(int rows, int max_bound, bool own_scores, int zero_rows = 0) {
    WsLayout L{};
    const int64_t mb = max_bound > 0 ? max_bound : 1;
    int n = (int)((mb + kSelTile - 1) / kSelTile);
    if (n < 1) n = 1;
    if (n > kSelMaxWgs) n = kSelMaxWgs;
    const int64_t ch = (mb + n - 1) / n;
    L.sel_wgs = n;
    L.sel_chunk = (ch + kSelTile - 1) / kSelTile * kSelTile;   // whole scan steps
    L.sstride = (int64_t)align_up((size_t)mb, 64);
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
    const size_t rz = zero_rows > 0 ? (size_t)zero_rows : (size_t)(rows > kZeroRows ? rows : kZeroRows);
    L.hist1 = take(rz * kHist1Slots * kBins1 * 4);
    L.hist2 = take(rz * kHist2Slots * kBins2 * 4);
    L.hist3 = take(rz * kBins3 * 4);
    L.fb_hist = take(rz * kFbBins * 4);
    L.fb_cnt = take(rz * 4);
    // finalize workgroups per row: one per 64K keys, at most kFbMaxWgs, and
    // about 256 in all (more would need a second round on the chip, and only
    // rows with heavy ties use them)
    int64_t fw = (mb + kFbKeysPerWg - 1) / kFbKeysPerWg;
    const int64_t cap = rows > 0 ? 256 / rows : 1;
    if (fw > cap) fw = cap;
    L.fb_wgs = (int)(fw < 1 ? 1 : (fw > kFbMaxWgs ? kFbMaxWgs : fw));
    L.state = take((size_t)rows * sizeof(RowState));
    L.ent_cnt = take((size_t)rows * n * 4);
    L.cand_cnt = take((size_t)rows * n * 4);
    L.ent_list = take((size_t)rows * n * kSliceCap * 8);
    L.scores = own_scores ? take((size_t)rows * (size_t)L.sstride * 4) : off;
    L.total = off;
    return L;
}

// Inclusive prefix sum over the wave's lanes with DPP row shifts (VALU only;
// a shuffle goes through the LDS crossbar at LDS latency per step): a
// Hillis-Steele scan inside each row of 16 lanes, then each row adds the
// totals of the rows before it.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int lane) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);   // row_shr:8
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
    const int row = lane >> 4;
    return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Wave-wide maximum and sum of a float, every lane getting the result: DPP
// rotations within each 16-lane row (1, 2, 4, 8), then the four rows through
// the two permlane swaps (each lane combines its value with the one 32, then
// 16, lanes away).
__device__ __forceinline__ float wave_max_f32(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false)));
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
    v = fmaxf(__int_as_float(a[0]), __int_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
    return fmaxf(__int_as_float(b[0]), __int_as_float(b[1]));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
    v = __int_as_float(a[0]) + __int_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
    return __int_as_float(b[0]) + __int_as_float(b[1]);
}

// Order-preserving map fp32 -> u32 used as the radix key: larger float ->
// larger key; -0 and +0 map to the same key; every NaN maps to 0, below -inf.
__device__ __forceinline__ uint32_t radix_key(float f) {
    uint32_t u = __float_as_uint(f);
    u = (u == 0x80000000u) ? 0u : u;
    uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (f != f) ? 0u : k;
}

struct ScoreArgs {
    const uint16_t *q;
    const float *w;
    const uint8_t *k8;
    const float *kscale;
    const int32_t *page_table;
    const int32_t *row_pt;
    const int32_t *row_bound;
    float *scores;
    uint32_t *hist1;   // null: no first-digit counting
    int64_t sstride;
    int rows, num_pages, pt_rows, pt_stride, max_bound, chunk;
};

struct SelectArgs {
    const float *scores;
    const int32_t *row_bound;
    int32_t *out_idx;
    unsigned char *ws;
    WsLayout L;
    int64_t sstride;
    int rows, max_bound, topk;
};

// ---- sparse attention over the selected keys (attn.hip)
constexpr int kAttnHeads = 16;    // query heads per row
constexpr int kAttnDim = 576;     // latent (512) + rotary (64) dims of a cache row and a query head
constexpr int kAttnVDim = 512;    // value dims (the latent part)
constexpr int kAttnMaxSplit = 32;     // workgroups one row's index list is split over (at most)
constexpr int kAttnWaveChunk = 16;    // index-list entries one wave takes at a time

struct AttnArgs {
    const uint16_t *q;        // [rows][16][576] bf16
    const uint16_t *kv;       // [num_pages][64][576] bf16
    const int32_t *page_table;
    const int32_t *row_pt;
    const int32_t *sel;       // [rows][topk] logical positions, -1 none
    float *out;               // [rows][16][512]
    float *lse;               // [rows][16]
    float *part_o;            // [rows][nsplit][16][512]  (workspace)
    float *part_ml;           // [rows][nsplit][2][16]    (workspace)
    float sm_scale;
    int rows, topk, span, nsplit, num_pages, pt_rows, pt_stride, max_bound;
};

// A row's index list is split over nsplit workgroups of span entries (a
// multiple of 64) so that rows * nsplit reaches about 256 workgroups.
inline void attn_split(int rows, int topk, int *nsplit, int *span) {
    // about 256 workgroups in all; a workgroup (4 waves) takes at least one
    // chunk of kAttnWaveChunk entries per wave
    int n = (256 + rows - 1) / rows;
    const int units = (topk + 4 * kAttnWaveChunk - 1) / (4 * kAttnWaveChunk);
    if (n > units) n = units;
    if (n > kAttnMaxSplit) n = kAttnMaxSplit;
    if (n < 1) n = 1;
    int sp = (topk + n - 1) / n;
    sp = (sp + kAttnWaveChunk - 1) / kAttnWaveChunk * kAttnWaveChunk;
    *span = sp;
    *nsplit = (topk + sp - 1) / sp > 0 ? (topk + sp - 1) / sp : 1;
}

inline size_t attn_workspace_bytes(int rows, int topk) {
    int n, sp;
    attn_split(rows, topk, &n, &sp);
    const size_t o = align_up((size_t)rows * n * kAttnHeads * kAttnVDim * 4, 256);
    return o + (size_t)rows * n * 2 * kAttnHeads * 4;
}

hipError_t launch_attention(const AttnArgs &a, hipStream_t st);

hipError_t launch_score(const ScoreArgs &a, hipStream_t st);
hipError_t launch_hist1(const SelectArgs &a, hipStream_t st);
hipError_t launch_refine(const SelectArgs &a, hipStream_t st);
hipError_t launch_gather(const SelectArgs &a, hipStream_t st);
hipError_t launch_finalize(const SelectArgs &a, hipStream_t st);
// rows of at most kSmallMax keys: one workgroup per row (with_hist1: it counts
// the first digit itself; else it takes, and clears, the scoring pass's counts)
hipError_t launch_select_small(const SelectArgs &a, bool with_hist1, hipStream_t st);
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t st);
hipError_t launch_shard_cand(const float *scores, int64_t sstride, const int32_t *out_idx, int rows, int k,
                             int g, int G, float *cand_score, int32_t *cand_idx, hipStream_t st);
hipError_t launch_merge(int rows, int n, int k, const float *cand_score, const int32_t *cand_idx,
                        int32_t *out_idx, hipStream_t st);
constexpr int kMergeMaxCand = 16384;   // shards * topk the merge holds per row
hipError_t launch_validate(const int32_t *page_table, const int32_t *row_pt, const int32_t *row_bound,
                           uint32_t *status, int rows, int num_pages, int pt_rows, int pt_stride, int max_bound,
                           hipStream_t st);
hipError_t launch_write_keys(const uint16_t *k_new, uint8_t *k8, float *kscale, const int32_t *page_table,
                             const int32_t *row_pt, const int32_t *row_bound, int rows, int num_pages,
                             int pt_rows, int pt_stride, int max_bound, hipStream_t st);

}  // namespace fp8idx
