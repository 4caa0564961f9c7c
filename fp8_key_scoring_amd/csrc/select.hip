// Exact top-k selection of the paged FP8 decode indexer (gfx950).
//
// Each row's exact top-k (k <= 2048) of its fp32 scores below the row's bound:
// descending value, equal values to the lower key index, NaN below every
// number, -0 equal to +0 (sglang pull request page "sgl-project/sglang#48224",
// sgl-amd-mono #86 commit body: Motivation for the exact top-2048 and the
// first radix digit; Modifications row 4 for taking the first digit,
// radix_key >> 26 in 64 bins, from the scoring pass).
//
// Radix key: the order-preserving fp32 -> u32 map (common.h).  Digits:
//   d1 = bits 31..26 (64 bins)   counted by the scoring pass, or by hist1_kernel
//   d2 = bits 25..18 (256 bins)  counted by refine_kernel inside the d1 bin
// The 14-bit prefix (d1, d2) of the k-th largest key splits a row into
//   "sure" keys (prefix above it: all selected) and
//   candidates (prefix equal: the remaining `need` are chosen among them).
// Kernels, one after the other on the stream (a kernel boundary is the only
// hand-off between workgroups: an agent-scope release inside a kernel writes
// back the whole L2 of an XCD, which costs far more than a dependent launch):
//   hist1    (only for indexer_topk) first-digit counts of stored scores;
//   refine   second-digit counts inside the first-digit bin, added to the
//            row's histogram with one atomic per non-empty bin per workgroup;
//   gather   every workgroup derives the same split from the two histograms,
//            writes its sure keys in index order to its own slice of the
//            workspace (ballot prefix sums, no atomics) and appends its
//            candidates to the row's list (one slot reservation);
//   finalize one workgroup per row sorts the candidates by (key desc, index
//            asc), takes `need`, and merges them with the concatenated sure
//            slices by binary search, so the row's output comes out in
//            ascending index order (deterministic bytes) without a full sort.
// Each scan step keeps 32 loads in flight per thread (8192 keys per
// workgroup), so a workgroup's pass over its chunk is one memory round trip.
// If a row has more than kCandCap candidates (heavy ties) finalize resolves
// the remaining 18 bits itself with three more digit passes over the row and
// takes exact ties in index order.
#include "common.h"

namespace fp8idx {

static_assert(kSelThreads == kBins2, "one thread per second-digit bin");
static_assert(kSelThreads / 64 * kSelUnroll == 128, "gather prefix: two entries per lane");

__device__ __forceinline__ uint32_t lane_prefix(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Executed by one full wave.  h: 64 * per bins in LDS.  Finds the largest bin
// B with sum_{b >= B} h[b] >= need (need >= 1) and the count strictly above
// B.  Results land in *outB / *outAbove (LDS), written by one lane.
__device__ void wave_find_bin(const uint32_t *h, int per, uint32_t need, int lane,
                              int *outB, uint32_t *outAbove) {
    uint32_t mine = 0;
    for (int j = 0; j < per; ++j) mine += h[lane * per + j];
    uint32_t incl = mine;   // sum over lanes >= lane
    for (int off = 1; off < 64; off <<= 1) {
        uint32_t v = __shfl_down(incl, off);
        if (lane + off < 64) incl += v;
    }
    const uint32_t excl = incl - mine;
    const uint64_t m = __ballot(excl < need && need <= incl);
    const int L = m ? (__ffsll((unsigned long long)m) - 1) : -1;
    if (lane == L) {
        uint32_t cum = excl;
        for (int j = per - 1; j >= 0; --j) {
            const uint32_t c = h[L * per + j];
            if (cum + c >= need) { *outB = L * per + j; *outAbove = cum; break; }
            cum += c;
        }
    }
}

// One scan step: thread t gets the radix keys of keys base + j*256 + t for
// j < kSelUnroll; all loads are issued before any is used.  Keys at or past
// s1 are not read (their slot gets key 0; callers test s < s1).
__device__ __forceinline__ void load_tile(const float *row, int64_t base, int64_t s1,
                                          uint32_t (&u)[kSelUnroll]) {
    const int t = threadIdx.x;
    float v[kSelUnroll];
#pragma unroll
    for (int j = 0; j < kSelUnroll; ++j) {
        const int64_t s = base + j * kSelThreads + t;
        v[j] = s < s1 ? row[s] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kSelUnroll; ++j) u[j] = radix_key(v[j]);
}

template <typename T>
__device__ __forceinline__ T tmin(T a, T b) { return a < b ? a : b; }
template <typename T>
__device__ __forceinline__ T tmax(T a, T b) { return a < b ? b : a; }

// Bitonic sort of n = kSelThreads * EPT values, thread t holding elements
// t*EPT + e in x[e].  Partners inside a thread are compared in registers,
// partners inside a wave are fetched with a lane shuffle, and only partners
// in another wave go through LDS (`lds`: n values of scratch).
template <typename T, int EPT, bool kAsc>
__device__ void block_sort(T (&x)[EPT], T *lds) {
    const int t = threadIdx.x;
    constexpr int n = kSelThreads * EPT;
#pragma unroll
    for (int kk = 2; kk <= n; kk <<= 1) {
#pragma unroll
        for (int j = kk >> 1; j > 0; j >>= 1) {
            if (j < EPT) {
#pragma unroll
                for (int e = 0; e < EPT; ++e) {
                    const int e2 = e ^ j;
                    if (e2 > e) {
                        const int i = t * EPT + e;
                        const bool up = ((i & kk) == 0) == kAsc;
                        const T a = x[e], b = x[e2];
                        x[e] = up ? tmin(a, b) : tmax(a, b);
                        x[e2] = up ? tmax(a, b) : tmin(a, b);
                    }
                }
            } else if (j < EPT * 64) {
#pragma unroll
                for (int e = 0; e < EPT; ++e) {
                    const int i = t * EPT + e;
                    const T y = __shfl_xor(x[e], j / EPT);
                    const bool keep_min = (((i & j) == 0) == (((i & kk) == 0) == kAsc));
                    x[e] = keep_min ? tmin(x[e], y) : tmax(x[e], y);
                }
            } else {
                __syncthreads();
#pragma unroll
                for (int e = 0; e < EPT; ++e) lds[t * EPT + e] = x[e];
                __syncthreads();
#pragma unroll
                for (int e = 0; e < EPT; ++e) {
                    const int i = t * EPT + e;
                    const T y = lds[i ^ j];
                    const bool keep_min = (((i & j) == 0) == (((i & kk) == 0) == kAsc));
                    x[e] = keep_min ? tmin(x[e], y) : tmax(x[e], y);
                }
            }
        }
    }
    __syncthreads();
}


// The `need` largest candidates (key << 32 | ~index, so equal keys order by
// lower index): their indices land in ch[0..need) in no particular order.
template <int EPT>
__device__ void take_candidates(const unsigned long long *cand, uint32_t n_cand, uint32_t need,
                                int32_t *ch, unsigned long long *lds) {
    const int t = threadIdx.x;
    unsigned long long x[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const uint32_t i = t * EPT + e;
        x[e] = i < n_cand ? cand[i] : 0ull;
    }
    block_sort<unsigned long long, EPT, false>(x, lds);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const uint32_t i = t * EPT + e;
        if (i < need) ch[i] = (int32_t)(0xFFFFFFFFu - (uint32_t)(x[e] & 0xFFFFFFFFull));
    }
    __syncthreads();
}

// v[0..n) sorted ascending in place (n <= kSelThreads * EPT).
template <int EPT>
__device__ void sort_small(int32_t *v, int n, int32_t *lds) {
    const int t = threadIdx.x;
    int32_t x[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int i = t * EPT + e;
        x[e] = i < n ? v[i] : 0x7FFFFFFF;
    }
    block_sort<int32_t, EPT, true>(x, lds);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int i = t * EPT + e;
        if (i < n) v[i] = x[e];
    }
    __syncthreads();
}

__device__ __forceinline__ int lower_bound(const int32_t *a, int n, int32_t v) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] < v) lo = mid + 1; else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ int clamp_bound(int b, int max_bound) {
    return b < 0 ? 0 : (b > max_bound ? max_bound : b);
}

// ---------------------------------------------------------------- hist1
// First-digit histogram of stored scores (used when the scores were not
// produced by this launch's scoring pass).
__global__ __launch_bounds__(kSelThreads) void hist1_kernel(SelectArgs a) {
    __shared__ uint32_t h[kBins1];
    const int r = blockIdx.y, t = threadIdx.x;
    const int b = clamp_bound(a.row_bound[r], a.max_bound);
    const int64_t s0 = (int64_t)blockIdx.x * a.L.sel_chunk;
    if (s0 >= b) return;
    const int64_t s1 = min(s0 + a.L.sel_chunk, (int64_t)b);
    if (t < kBins1) h[t] = 0;
    __syncthreads();
    const float *row = a.scores + (int64_t)r * a.sstride;
    for (int64_t base = s0; base < s1; base += kSelTile) {
        uint32_t u[kSelUnroll];
        load_tile(row, base, s1, u);
#pragma unroll
        for (int j = 0; j < kSelUnroll; ++j)
            if (base + j * kSelThreads + t < s1) atomicAdd(&h[u[j] >> kDigit1Shift], 1u);
    }
    __syncthreads();
    uint32_t *hist1 = (uint32_t *)(a.ws + a.L.hist1);
    if (t < kBins1 && h[t]) atomicAdd(hist1 + (int64_t)r * kBins1 + t, h[t]);
}

// ---------------------------------------------------------------- refine
// Second-digit counts inside the first-digit bin of the k-th largest key.
__global__ __launch_bounds__(kSelThreads) void refine_kernel(SelectArgs a) {
    __shared__ uint32_t h1[kBins1];
    __shared__ uint32_t h2[kBins2];
    __shared__ int sb1;
    __shared__ uint32_t sabove1;
    const int r = blockIdx.y, x = blockIdx.x, t = threadIdx.x, lane = t & 63;
    const int b = clamp_bound(a.row_bound[r], a.max_bound);
    const uint32_t k = (uint32_t)a.topk;
    const int64_t s0 = (int64_t)x * a.L.sel_chunk;
    if ((uint32_t)b <= k || s0 >= b) return;   // all selected, or nothing here
    const int64_t s1 = min(s0 + a.L.sel_chunk, (int64_t)b);
    const uint32_t *hist1 = (const uint32_t *)(a.ws + a.L.hist1) + (int64_t)r * kBins1;
    uint32_t *hist2 = (uint32_t *)(a.ws + a.L.hist2) + (int64_t)r * kBins2;
    const float *row = a.scores + (int64_t)r * a.sstride;

    uint32_t u[kSelUnroll];
    load_tile(row, s0, s1, u);   // first step's loads overlap the digit search
    if (t < kBins1) h1[t] = hist1[t];
    h2[t] = 0;
    if (t == 0) { sb1 = 0; sabove1 = 0; }
    __syncthreads();
    if (t < 64) wave_find_bin(h1, 1, k, lane, &sb1, &sabove1);
    __syncthreads();
    const uint32_t b1 = (uint32_t)sb1;
    for (int64_t base = s0; base < s1; base += kSelTile) {
        if (base != s0) load_tile(row, base, s1, u);
#pragma unroll
        for (int j = 0; j < kSelUnroll; ++j)
            if (base + j * kSelThreads + t < s1 && (u[j] >> kDigit1Shift) == b1)
                atomicAdd(&h2[(u[j] >> kDigit2Shift) & (kBins2 - 1)], 1u);
    }
    __syncthreads();
    if (h2[t]) atomicAdd(hist2 + t, h2[t]);
}

// ------------------------------------------------------------- fallback
// Exact resolution inside the 14-bit prefix bin by one workgroup, used when
// the bin holds more than kCandCap keys: three more digit passes fix the
// threshold key T, then keys above T and the first `need - above` ties at T
// in index order go to ch[0..need) (in no particular order).
__device__ void fallback_select(const float *row, int b, uint32_t T14, uint32_t need, int32_t *ch,
                                uint32_t *h, int *sB, uint32_t *sAbove, uint32_t *wtot, uint32_t *spos) {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int shifts[3] = {10, 2, 0};
    const int widths[3] = {8, 8, 2};
    uint32_t prefix = T14;
    int pshift = kDigit2Shift;
    uint32_t need_cur = need;
    for (int d = 0; d < 3; ++d) {
        h[t] = 0;
        if (t == 0) { *sB = 0; *sAbove = 0; }
        __syncthreads();
        const uint32_t mask = (1u << widths[d]) - 1u;
        const int sh = shifts[d];
        for (int64_t base = 0; base < b; base += kSelTile) {
            uint32_t u[kSelUnroll];
            load_tile(row, base, b, u);
#pragma unroll
            for (int j = 0; j < kSelUnroll; ++j)
                if (base + j * kSelThreads + t < b && (u[j] >> pshift) == prefix)
                    atomicAdd(&h[(u[j] >> sh) & mask], 1u);
        }
        __syncthreads();
        if (t < 64) wave_find_bin(h, kBins2 / 64, need_cur, lane, sB, sAbove);
        __syncthreads();
        need_cur -= *sAbove;
        prefix = (prefix << widths[d]) | (uint32_t)(*sB);
        pshift = shifts[d];
        __syncthreads();
    }
    const uint32_t T = prefix;   // the k-th largest key; need_cur ties at T to take
    if (t == 0) *spos = 0;
    __syncthreads();
    uint32_t tie_run = 0;
    for (int base = 0; base < b; base += kSelThreads) {
        const int s = base + t;
        const uint32_t u = s < b ? radix_key(row[s]) : 0u;
        const bool in = s < b && (u >> kDigit2Shift) == T14;
        const bool gt = in && u > T;
        const bool tie = in && u == T;
        const uint64_t m = __ballot(tie);
        if (lane == 0) wtot[wave] = (uint32_t)__popcll(m);
        __syncthreads();
        uint32_t woff = 0, all = 0;
        for (int wv = 0; wv < kSelThreads / 64; ++wv) {
            if (wv < wave) woff += wtot[wv];
            all += wtot[wv];
        }
        const uint32_t rank = tie_run + woff + lane_prefix(m);
        if (gt || (tie && rank < need_cur)) {
            const uint32_t p = atomicAdd(spos, 1u);
            if (p < need) ch[p] = s;
        }
        tie_run += all;
        __syncthreads();
    }
}

// ---------------------------------------------------------------- gather
// Every workgroup of a row derives the same split from the two histograms,
// writes its sure keys (ascending) to its own slice and appends candidates.
__global__ __launch_bounds__(kSelThreads) void gather_kernel(SelectArgs a) {
    __shared__ unsigned long long l_cand[kCandCap];
    __shared__ uint32_t h1[kBins1];
    __shared__ uint32_t h2[kBins2];
    __shared__ uint32_t cnt[kSelUnroll * (kSelThreads / 64)];
    __shared__ int sb1, sb2;
    __shared__ uint32_t sabove1, sabove2, n_cand_l, g_cand, tile_total;
    const int r = blockIdx.y, x = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int b = clamp_bound(a.row_bound[r], a.max_bound);
    const int k = a.topk;
    const int S = a.L.sel_wgs;
    int32_t *out_row = a.out_idx + (int64_t)r * k;
    if (b <= k) {   // every key selected: indices 0..b-1, then -1
        if (x == 0)
            for (int i = t; i < k; i += kSelThreads) out_row[i] = i < b ? i : -1;
        return;
    }
    const uint32_t *hist1 = (const uint32_t *)(a.ws + a.L.hist1) + (int64_t)r * kBins1;
    const uint32_t *hist2 = (const uint32_t *)(a.ws + a.L.hist2) + (int64_t)r * kBins2;
    uint32_t *cand_slot = (uint32_t *)(a.ws + a.L.cand_slot) + r;
    unsigned long long *cand = (unsigned long long *)(a.ws + a.L.cand) + (int64_t)r * kCandCap;
    int32_t *slice = (int32_t *)(a.ws + a.L.sure_list) + ((int64_t)r * S + x) * kMaxTopk;
    const float *row = a.scores + (int64_t)r * a.sstride;
    const int64_t s0 = (int64_t)x * a.L.sel_chunk;
    const int64_t s1 = min(s0 + a.L.sel_chunk, (int64_t)b);

    uint32_t u[kSelUnroll];
    if (s0 < s1) load_tile(row, s0, s1, u);   // overlaps the split below
    // ---- the split: (b1, above1) from the first digit, (b2, above2) from the second
    if (t < kBins1) h1[t] = hist1[t];
    h2[t] = hist2[t];
    if (t == 0) { sb1 = 0; sabove1 = 0; sb2 = 0; sabove2 = 0; n_cand_l = 0; }
    __syncthreads();
    if (t < 64) wave_find_bin(h1, 1, (uint32_t)k, lane, &sb1, &sabove1);
    __syncthreads();
    if (t < 64) wave_find_bin(h2, kBins2 / 64, (uint32_t)k - sabove1, lane, &sb2, &sabove2);
    __syncthreads();
    const uint32_t b1 = (uint32_t)sb1, b2 = (uint32_t)sb2;
    const uint32_t T14 = (b1 << kDigit2Bits) | b2;
    if (x == 0 && t == 0) {
        RowState st;
        st.b1 = b1;
        st.b2 = b2;
        st.sure = sabove1 + sabove2;
        st.need = (uint32_t)k - st.sure;
        st.cand = h2[b2];
        st.pad[0] = st.pad[1] = st.pad[2] = 0;
        ((RowState *)(a.ws + a.L.state))[r] = st;
    }

    uint32_t written = 0;   // sure keys of this workgroup so far (uniform)
    for (int64_t base = s0; base < s1; base += kSelTile) {
        if (base != s0) load_tile(row, base, s1, u);
        // pass 1: sure keys per (step j, wave); candidates to the LDS list
#pragma unroll
        for (int j = 0; j < kSelUnroll; ++j) {
            const bool valid = base + j * kSelThreads + t < s1;
            const uint32_t top = u[j] >> kDigit2Shift;
            const uint64_t ms = __ballot(valid && top > T14);
            if (lane == 0) cnt[j * 4 + wave] = (uint32_t)__popcll(ms);
            const bool cnd = valid && top == T14;
            const uint64_t mc = __ballot(cnd);
            if (mc) {
                uint32_t pos0 = 0;
                if (lane == 0) pos0 = atomicAdd(&n_cand_l, (uint32_t)__popcll(mc));
                pos0 = __shfl(pos0, 0);
                const uint32_t pos = pos0 + lane_prefix(mc);
                const int64_t s = base + j * kSelThreads + t;
                if (cnd && pos < (uint32_t)kCandCap)
                    l_cand[pos] = ((unsigned long long)u[j] << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)s);
            }
        }
        __syncthreads();
        // exclusive prefix of the 128 counts, in key order (step-major, then wave)
        if (t < 64) {
            const uint32_t c0 = cnt[2 * lane], c1 = cnt[2 * lane + 1];
            uint32_t incl = c0 + c1;
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t v = __shfl_up(incl, off);
                if (lane >= off) incl += v;
            }
            const uint32_t excl = incl - c0 - c1;
            cnt[2 * lane] = excl;
            cnt[2 * lane + 1] = excl + c0;
            if (lane == 63) tile_total = incl;
        }
        __syncthreads();
        // pass 2: each sure key to its place
#pragma unroll
        for (int j = 0; j < kSelUnroll; ++j) {
            const bool valid = base + j * kSelThreads + t < s1;
            const bool sure = valid && (u[j] >> kDigit2Shift) > T14;
            const uint64_t ms = __ballot(sure);
            if (sure) {
                const uint32_t pos = written + cnt[j * 4 + wave] + lane_prefix(ms);
                if (pos < (uint32_t)kMaxTopk) slice[pos] = (int32_t)(base + j * kSelThreads + t);
            }
        }
        written += tile_total;
        __syncthreads();
    }
    if (t == 0) {
        ((uint32_t *)(a.ws + a.L.sure_cnt))[(int64_t)r * S + x] = written < (uint32_t)kMaxTopk ? written : (uint32_t)kMaxTopk;
        g_cand = n_cand_l ? atomicAdd(cand_slot, n_cand_l) : 0u;
    }
    __syncthreads();
    const uint32_t nc = min(n_cand_l, (uint32_t)kCandCap);
    for (uint32_t i = t; i < nc; i += kSelThreads)
        if (g_cand + i < (uint32_t)kCandCap) cand[g_cand + i] = l_cand[i];
}

// -------------------------------------------------------------- finalize
// One workgroup per row: choose the `need` candidates, merge them with the
// sure keys into the row's output in ascending index order, and leave the
// row's histograms and candidate counter zeroed.
__global__ __launch_bounds__(kSelThreads) void finalize_kernel(SelectArgs a) {
    __shared__ unsigned long long sortbuf[kCandCap];
    __shared__ int32_t su[kMaxTopk];
    __shared__ int32_t ch[kMaxTopk];
    __shared__ uint32_t off[kSelMaxWgs + 1];
    __shared__ uint32_t h[kBins2];
    __shared__ uint32_t wtot[kSelThreads / 64];
    __shared__ int sB;
    __shared__ uint32_t sAbove, spos;
    const int r = blockIdx.x, t = threadIdx.x, lane = t & 63;
    const int b = clamp_bound(a.row_bound[r], a.max_bound);
    const int k = a.topk;
    const int S = a.L.sel_wgs;
    int32_t *out_row = a.out_idx + (int64_t)r * k;
    if (b > k) {
        const RowState st = ((const RowState *)(a.ws + a.L.state))[r];
        const unsigned long long *cand = (const unsigned long long *)(a.ws + a.L.cand) + (int64_t)r * kCandCap;
        const uint32_t *cnts = (const uint32_t *)(a.ws + a.L.sure_cnt) + (int64_t)r * S;
        const int32_t *slices = (const int32_t *)(a.ws + a.L.sure_list) + (int64_t)r * S * kMaxTopk;
        const float *row = a.scores + (int64_t)r * a.sstride;
        // slice offsets: exclusive prefix of the per-workgroup sure counts
        if (t < 64) {
            const uint32_t c = lane < S ? cnts[lane] : 0u;
            uint32_t incl = c;
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t v = __shfl_up(incl, o);
                if (lane >= o) incl += v;
            }
            off[lane] = incl - c;
            if (lane == 63) off[kSelMaxWgs] = incl;
        }
        // the candidates to take
        const uint32_t need = st.need < (uint32_t)kMaxTopk ? st.need : (uint32_t)kMaxTopk;
        const uint32_t n_cand = st.cand;
        if (n_cand <= (uint32_t)kCandCap) {
            if (n_cand <= 256) take_candidates<1>(cand, n_cand, need, ch, sortbuf);
            else if (n_cand <= 512) take_candidates<2>(cand, n_cand, need, ch, sortbuf);
            else if (n_cand <= 1024) take_candidates<4>(cand, n_cand, need, ch, sortbuf);
            else if (n_cand <= 2048) take_candidates<8>(cand, n_cand, need, ch, sortbuf);
            else take_candidates<16>(cand, n_cand, need, ch, sortbuf);
        } else {
            fallback_select(row, b, (st.b1 << kDigit2Bits) | st.b2, need, ch, h, &sB, &sAbove, wtot, &spos);
        }
        __syncthreads();
        int32_t *scratch = (int32_t *)sortbuf;
        if (need <= 256) sort_small<1>(ch, need, scratch);
        else if (need <= 512) sort_small<2>(ch, need, scratch);
        else if (need <= 1024) sort_small<4>(ch, need, scratch);
        else sort_small<8>(ch, need, scratch);
        // the sure keys: slices concatenated in workgroup order are ascending
        const int ns = (int)min(off[kSelMaxWgs], (uint32_t)k - need);
        for (int p = t; p < ns; p += kSelThreads) {
            int lo = 0, hi = S - 1;   // last slice whose offset is <= p
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (off[mid] <= (uint32_t)p) lo = mid; else hi = mid - 1;
            }
            su[p] = slices[(int64_t)lo * kMaxTopk + (p - (int)off[lo])];
        }
        __syncthreads();
        // merge: each value's place is its rank in its own list plus its rank in the other
        for (int p = t; p < ns; p += kSelThreads) {
            const int32_t v = su[p];
            out_row[p + lower_bound(ch, (int)need, v)] = v;
        }
        for (int j = t; j < (int)need; j += kSelThreads) {
            const int32_t c = ch[j];
            out_row[j + lower_bound(su, ns, c)] = c;
        }
    }
    uint32_t *hist1 = (uint32_t *)(a.ws + a.L.hist1) + (int64_t)r * kBins1;
    uint32_t *hist2 = (uint32_t *)(a.ws + a.L.hist2) + (int64_t)r * kBins2;
    if (t < kBins1) hist1[t] = 0;
    hist2[t] = 0;
    if (t == 0) ((uint32_t *)(a.ws + a.L.cand_slot))[r] = 0;
}

__global__ void fill_zero_kernel(uint32_t *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

hipError_t launch_hist1(const SelectArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(hist1_kernel, dim3(a.L.sel_wgs, a.rows), dim3(kSelThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_refine(const SelectArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(refine_kernel, dim3(a.L.sel_wgs, a.rows), dim3(kSelThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_gather(const SelectArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(gather_kernel, dim3(a.L.sel_wgs, a.rows), dim3(kSelThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_finalize(const SelectArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(finalize_kernel, dim3(a.rows), dim3(kSelThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t st) {
    const size_t n = bytes / 4;
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (uint32_t *)p, n);
    return hipGetLastError();
}

}  // namespace fp8idx
