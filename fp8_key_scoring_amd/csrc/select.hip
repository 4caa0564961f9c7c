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
// gather_kernel writes the sure keys' indices and collects the candidates;
// the last of a row's workgroups sorts the candidates by (key desc, index
// asc), takes `need`, and sorts the row's output by index so the bytes are
// deterministic.  If a row has more than kCandCap candidates (heavy ties)
// that workgroup resolves the remaining 18 bits itself with three more digit
// passes over the row and takes exact ties in index order.
//
// Cross-workgroup hand-off uses only completion counters (atomicAdd, device
// scope) and fences; no workgroup ever waits for another, and the last
// workgroup of a row to finish does the row's serial tail and re-zeroes the
// row's counters and histograms for the next launch.
#include "common.h"

namespace fp8idx {

static_assert(kSelThreads == kBins2, "one thread per second-digit bin");

__device__ __forceinline__ uint32_t lane_prefix(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Executed by one full wave.  h: `nb` bins in LDS (nb = 64 * per).  Finds the
// largest bin B with sum_{b >= B} h[b] >= need (need >= 1) and the count
// strictly above B.  Results land in *outB / *outAbove (LDS), written by one lane.
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

template <typename T, bool kDesc>
__device__ void bitonic_sort(T *v, int n, int t) {
    for (int kk = 2; kk <= n; kk <<= 1) {
        for (int j = kk >> 1; j > 0; j >>= 1) {
            for (int i = t; i < n; i += kSelThreads) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const bool up = (i & kk) == 0;
                    const T x = v[i], y = v[ixj];
                    const bool sw = kDesc ? (up ? x < y : x > y) : (up ? x > y : x < y);
                    if (sw) { v[i] = y; v[ixj] = x; }
                }
            }
            __syncthreads();
        }
    }
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
    for (int64_t s = s0 + t; s < s1; s += kSelThreads)
        atomicAdd(&h[radix_key(row[s]) >> kDigit1Shift], 1u);
    __syncthreads();
    uint32_t *hist1 = (uint32_t *)(a.ws + a.L.hist1);
    if (t < kBins1 && h[t]) atomicAdd(hist1 + (int64_t)r * kBins1 + t, h[t]);
}

// ---------------------------------------------------------------- refine
// Second digit inside the first-digit bin of the k-th largest key; the last
// workgroup of the row fixes (b1, b2) and the sure / need / candidate counts.
__global__ __launch_bounds__(kSelThreads) void refine_kernel(SelectArgs a) {
    __shared__ uint32_t h1[kBins1];
    __shared__ uint32_t h2[kBins2];
    __shared__ int sb1, sb2;
    __shared__ uint32_t sabove1, sabove2, slast;
    const int r = blockIdx.y, x = blockIdx.x, t = threadIdx.x, lane = t & 63;
    const int b = clamp_bound(a.row_bound[r], a.max_bound);
    const uint32_t k = (uint32_t)a.topk;
    if ((uint32_t)b <= k) return;   // every key of the row is selected
    const int S = a.L.sel_wgs;
    uint32_t *hist1 = (uint32_t *)(a.ws + a.L.hist1) + (int64_t)r * kBins1;
    uint32_t *hist2p = (uint32_t *)(a.ws + a.L.hist2p) + (int64_t)r * S * kBins2;
    uint32_t *cnt2 = (uint32_t *)(a.ws + a.L.cnt2) + r;

    if (t < kBins1) h1[t] = hist1[t];
    h2[t] = 0;
    if (t == 0) { sb1 = 0; sabove1 = 0; }
    __syncthreads();
    if (t < 64) wave_find_bin(h1, 1, k, lane, &sb1, &sabove1);
    __syncthreads();
    const uint32_t b1 = (uint32_t)sb1;

    const int64_t s0 = (int64_t)x * a.L.sel_chunk;
    const int64_t s1 = min(s0 + a.L.sel_chunk, (int64_t)b);
    const float *row = a.scores + (int64_t)r * a.sstride;
    for (int64_t s = s0 + t; s < s1; s += kSelThreads) {
        const uint32_t u = radix_key(row[s]);
        if ((u >> kDigit1Shift) == b1) atomicAdd(&h2[(u >> kDigit2Shift) & (kBins2 - 1)], 1u);
    }
    __syncthreads();
    hist2p[(int64_t)x * kBins2 + t] = h2[t];
    __threadfence();
    __syncthreads();
    if (t == 0) slast = (atomicAdd(cnt2, 1u) == (uint32_t)(S - 1));
    __syncthreads();
    if (!slast) return;
    __threadfence();

    uint32_t tot = 0;
    for (int xx = 0; xx < S; ++xx) tot += __builtin_nontemporal_load(hist2p + (int64_t)xx * kBins2 + t);
    h2[t] = tot;
    if (t == 0) { sb2 = 0; sabove2 = 0; }
    __syncthreads();
    const uint32_t need1 = k - sabove1;
    if (t < 64) wave_find_bin(h2, kBins2 / 64, need1, lane, &sb2, &sabove2);
    __syncthreads();
    if (t == 0) {
        RowState st;
        st.b1 = b1;
        st.b2 = (uint32_t)sb2;
        st.sure = sabove1 + sabove2;
        st.need = k - st.sure;
        st.cand = h2[sb2];
        st.pad[0] = st.pad[1] = st.pad[2] = 0;
        ((RowState *)(a.ws + a.L.state))[r] = st;
        *cnt2 = 0;
    }
}

// ------------------------------------------------------------- fallback
// Exact resolution inside the 14-bit prefix bin by one workgroup, used when
// the bin holds more than kCandCap keys: three more digit passes fix the
// threshold key T, then keys above T and the first ties at T in index order
// are written after the sure keys.
__device__ void fallback_select(const float *row, int b, uint32_t T14, uint32_t need,
                                int32_t *out_row, uint32_t sure, uint32_t *h,
                                int *sB, uint32_t *sAbove, uint32_t *wtot, uint32_t *spos) {
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
        for (int s = t; s < b; s += kSelThreads) {
            const uint32_t u = radix_key(row[s]);
            if ((u >> pshift) == prefix) atomicAdd(&h[(u >> shifts[d]) & mask], 1u);
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
            if (sure + p < (uint32_t)kMaxTopk && sure + p < sure + need) out_row[sure + p] = s;
        }
        tie_run += all;
        __syncthreads();
    }
}

// ---------------------------------------------------------------- gather
__global__ __launch_bounds__(kSelThreads) void gather_kernel(SelectArgs a) {
    __shared__ unsigned long long sortbuf[kCandCap];
    __shared__ uint32_t h[kBins2];
    __shared__ uint32_t wtot[kSelThreads / 64];
    __shared__ int sB;
    __shared__ uint32_t sAbove, spos, slast;
    const int r = blockIdx.y, x = blockIdx.x, t = threadIdx.x, lane = t & 63;
    const int b = clamp_bound(a.row_bound[r], a.max_bound);
    const int k = a.topk;
    const int S = a.L.sel_wgs;
    int32_t *out_row = a.out_idx + (int64_t)r * k;
    uint32_t *cnt3 = (uint32_t *)(a.ws + a.L.cnt3) + r;
    uint32_t *sure_slot = (uint32_t *)(a.ws + a.L.sure_slot) + r;
    uint32_t *cand_slot = (uint32_t *)(a.ws + a.L.cand_slot) + r;
    unsigned long long *cand = (unsigned long long *)(a.ws + a.L.cand) + (int64_t)r * kCandCap;
    const float *row = a.scores + (int64_t)r * a.sstride;
    const bool all = b <= k;
    RowState st{};
    if (all) {
        if (x == 0)
            for (int i = t; i < k; i += kSelThreads) out_row[i] = i < b ? i : -1;
    } else {
        st = ((const RowState *)(a.ws + a.L.state))[r];
        const uint32_t T14 = (st.b1 << kDigit2Bits) | st.b2;
        const int64_t s0 = (int64_t)x * a.L.sel_chunk;
        const int64_t s1 = min(s0 + a.L.sel_chunk, (int64_t)b);
        const int64_t nfull = s0 < s1 ? (s1 - s0 + kSelThreads - 1) / kSelThreads * kSelThreads : 0;
        for (int64_t o = t; o < nfull; o += kSelThreads) {
            const int64_t s = s0 + o;
            const uint32_t u = s < s1 ? radix_key(row[s]) : 0u;
            const uint32_t top = u >> kDigit2Shift;
            const bool sure = s < s1 && top > T14;
            const bool cnd = s < s1 && top == T14;
            const uint64_t ms = __ballot(sure);
            if (ms) {
                uint32_t base = 0;
                if (lane == 0) base = atomicAdd(sure_slot, (uint32_t)__popcll(ms));
                base = __shfl(base, 0);
                const uint32_t pos = base + lane_prefix(ms);
                if (sure && pos < (uint32_t)k) out_row[pos] = (int32_t)s;
            }
            const uint64_t mc = __ballot(cnd);
            if (mc) {
                uint32_t base = 0;
                if (lane == 0) base = atomicAdd(cand_slot, (uint32_t)__popcll(mc));
                base = __shfl(base, 0);
                const uint32_t pos = base + lane_prefix(mc);
                if (cnd && pos < (uint32_t)kCandCap)
                    cand[pos] = ((unsigned long long)u << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)s);
            }
        }
    }
    __threadfence();
    __syncthreads();
    if (t == 0) slast = (atomicAdd(cnt3, 1u) == (uint32_t)(S - 1));
    __syncthreads();
    if (!slast) return;
    __threadfence();

    if (!all) {
        const uint32_t n_cand = st.cand;
        if (n_cand <= (uint32_t)kCandCap) {
            int n2 = 1;
            while (n2 < (int)n_cand) n2 <<= 1;
            for (int i = t; i < n2; i += kSelThreads)
                sortbuf[i] = i < (int)n_cand ? __builtin_nontemporal_load(cand + i) : 0ull;
            __syncthreads();
            bitonic_sort<unsigned long long, true>(sortbuf, n2, t);
            for (uint32_t i = t; i < st.need; i += kSelThreads)
                out_row[st.sure + i] = (int32_t)(0xFFFFFFFFu - (uint32_t)(sortbuf[i] & 0xFFFFFFFFull));
        } else {
            fallback_select(row, b, (st.b1 << kDigit2Bits) | st.b2, st.need, out_row, st.sure,
                            h, &sB, &sAbove, wtot, &spos);
        }
        __threadfence();
        __syncthreads();
        // deterministic bytes: the row's k indices in ascending order
        int32_t *ib = (int32_t *)sortbuf;
        for (int i = t; i < kMaxTopk; i += kSelThreads)
            ib[i] = i < k ? __builtin_nontemporal_load(out_row + i) : 0x7FFFFFFF;
        __syncthreads();
        int n2 = 1;
        while (n2 < k) n2 <<= 1;
        bitonic_sort<int32_t, false>(ib, n2, t);
        for (int i = t; i < k; i += kSelThreads) out_row[i] = ib[i];
    }
    // leave the row's counters and first-digit histogram zeroed
    uint32_t *hist1 = (uint32_t *)(a.ws + a.L.hist1) + (int64_t)r * kBins1;
    if (t < kBins1) hist1[t] = 0;
    if (t == 0) { *cnt3 = 0; *sure_slot = 0; *cand_slot = 0; }
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

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t st) {
    const size_t n = bytes / 4;
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (uint32_t *)p, n);
    return hipGetLastError();
}

}  // namespace fp8idx
