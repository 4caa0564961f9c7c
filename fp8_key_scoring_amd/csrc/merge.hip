// Key-sharded (DCP-style) selection on gfx950: the exact top-k of a row whose
// keys are split over G shards, from each shard's own top-k.
//
// Shard g of G holds pages g, g+G, g+2G, ... of every request (the release
// test-suite page for GLM-5.2 serves its context this way, 64-key pages
// interleaved over ranks, and merges each rank's top-k by owner).  A shard runs
// the ordinary launch over its own page table; its key s is global key
// 64 * (g + G * (s / 64)) + s % 64.  Every key's score depends only on the row
// and the key, so a shard computes bit for bit the score the unsharded launch
// would, and the top-k of the union of the shards' top-k sets (same order:
// larger score first, equal scores to the lower global index) is the row's
// global top-k: a key outside its own shard's top-k has k keys of that shard
// ranked above it.
//
//   shard_cand_kernel  one shard's (local index, score) selection becomes
//                      (global index, score) candidates in slot block g;
//   merge_kernel       one workgroup per row: an exact radix select over the
//                      row's G*k candidates on a 64-bit key (radix key of the
//                      score, then the inverted index, so every key is
//                      distinct); the selected global indices go out grouped
//                      by shard, each group ascending, then -1.
#include "common.h"

namespace fp8idx {

constexpr int kMergeThreads = 1024;
constexpr int kMergeMax = kMergeMaxCand;                 // candidates per row (G * k)
constexpr int kMergePer = kMergeMax / kMergeThreads;     // per thread
constexpr int kMergeBits = 11;                           // digit width
constexpr int kMergeBins = 1 << kMergeBits;

__global__ __launch_bounds__(256) void shard_cand_kernel(const float *scores, int64_t sstride,
                                                         const int32_t *out_idx, int k, int g, int G,
                                                         float *cand_score, int32_t *cand_idx) {
    const int r = blockIdx.y;
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= k) return;
    const int s = out_idx[(int64_t)r * k + i];
    const int64_t o = ((int64_t)r * G + g) * k + i;
    if (s >= 0) {
        cand_score[o] = scores[(int64_t)r * sstride + s];
        cand_idx[o] = kPage * (g + G * (s / kPage)) + s % kPage;
    } else {
        cand_score[o] = 0.0f;
        cand_idx[o] = -1;
    }
}

// Exclusive prefix over the workgroup, in thread order, of a v <= 16 per
// thread: within a wave five ballots (one per bit of v) and their lane
// prefixes, across waves one barrier and the wave totals; `total` receives
// the sum in every thread.  wsum (one word per wave) must not be written
// again until every thread has returned.
__device__ uint32_t merge_scan(uint32_t v, uint32_t *wsum, uint32_t &total) {
    const int t = threadIdx.x, wave = t >> 6;
    uint32_t pre = 0, tot = 0;
#pragma unroll
    for (int bit = 0; bit < 5; ++bit) {
        const uint64_t m = __ballot((v >> bit) & 1u);
        pre += __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << bit;
        tot += (uint32_t)__popcll(m) << bit;
    }
    if ((t & 63) == 0) wsum[wave] = tot;
    __syncthreads();
    uint32_t off = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kMergeThreads / 64; ++w) {
        const uint32_t x = wsum[w];
        off += w < wave ? x : 0u;
        all += x;
    }
    total = all;
    return off + pre;
}

// Wave-wide reductions of a 32-bit value (every lane gets the result):
// DPP rotations within each 16-lane row (1, 2, 4, 8), then the rows through
// permlane swaps.
template <typename F>
__device__ __forceinline__ uint32_t merge_wave_reduce(uint32_t v, F op) {
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xf, 0xf, false));   // row_ror:1
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xf, 0xf, false));   // row_ror:2
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false));   // row_ror:4
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false));   // row_ror:8
    const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    v = op(a[0], a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return op(b[0], b[1]);
}

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(int n, int k, const float *cand_score,
                                                              const int32_t *cand_idx, int32_t *out_idx) {
    constexpr int kW = kMergeThreads / 64;
    __shared__ uint32_t hist[2][kMergeBins];   // pass p counts into hist[p & 1]
    __shared__ uint32_t wred[3][kW];           // per wave: valid keys, lowest and highest score key
    __shared__ uint32_t wsum[kW], wsum2[kW];   // per-wave scan totals
    __shared__ uint32_t s_bin, s_above, s_cnt;
    static_assert(kMergePer <= 16, "merge: a thread's counts fit the five-bit scan");
    static_assert(kMergeBins == 2 * kMergeThreads, "two bins per thread in the bin search");
    const int r = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const float *sc = cand_score + (int64_t)r * n;
    const int32_t *ix = cand_idx + (int64_t)r * n;

    // Thread t holds candidate slots 16t .. 16t+15.  64-bit keys: larger is
    // better (radix key of the score, then the inverted index); an empty
    // slot is 0, below every candidate (a NaN score's key is ~index > 0).
    // (n is a multiple of 16 and the arrays 16-byte aligned: four 16-byte
    // loads per array, all issued before any is used)
    uint64_t key[kMergePer];
    uint32_t valid = 0, lo_hi = 0xFFFFFFFFu, hi_hi = 0u;
    {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        u32x4 vi[kMergePer / 4], vs[kMergePer / 4];
        const bool here = t * kMergePer < n;
        const int base = here ? t * kMergePer : 0;
#pragma unroll
        for (int q = 0; q < kMergePer / 4; ++q) vi[q] = *(const u32x4 *)(ix + base + 4 * q);
#pragma unroll
        for (int q = 0; q < kMergePer / 4; ++q) vs[q] = *(const u32x4 *)(sc + base + 4 * q);
        // both histograms start at zero (hist[1] is cleared again during
        // every pass that uses hist[0], and the other way round)
        for (int i = t; i < 2 * kMergeBins; i += kMergeThreads) (&hist[0][0])[i] = 0u;
#pragma unroll
        for (int m = 0; m < kMergePer; ++m) {
            const int32_t id = here ? (int32_t)vi[m >> 2][m & 3] : -1;
            const uint32_t rk = radix_key(__uint_as_float(vs[m >> 2][m & 3]));
            key[m] = id >= 0 ? ((uint64_t)rk << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)id) : 0ull;
            valid += id >= 0;
            lo_hi = id >= 0 && rk < lo_hi ? rk : lo_hi;
            hi_hi = id >= 0 && rk > hi_hi ? rk : hi_hi;
        }
    }
    // one exchange for the three row-wide values
    valid = merge_wave_reduce(valid, [](uint32_t x, uint32_t y) { return x + y; });
    lo_hi = merge_wave_reduce(lo_hi, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
    hi_hi = merge_wave_reduce(hi_hi, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
    if (lane == 0) { wred[0][wave] = valid; wred[1][wave] = lo_hi; wred[2][wave] = hi_hi; }
    __syncthreads();
    uint32_t total_valid = 0;
    lo_hi = 0xFFFFFFFFu;
    hi_hi = 0u;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
        total_valid += wred[0][w];
        lo_hi = wred[1][w] < lo_hi ? wred[1][w] : lo_hi;
        hi_hi = wred[2][w] > hi_hi ? wred[2][w] : hi_hi;
    }
    const uint32_t want = total_valid < (uint32_t)k ? total_valid : (uint32_t)k;

    // The candidates are the shards' top-k: their scores crowd into a narrow
    // band, so the top bits of the keys are nearly all equal and a first digit
    // taken there would send every atomic to a handful of bins.  The select
    // runs on the offset key (key - (lowest score key << 32) + 1), whose first
    // digit starts at the top bit of the range; the order is the same.
    const uint64_t kmin = (uint64_t)lo_hi << 32;
#pragma unroll
    for (int m = 0; m < kMergePer; ++m) key[m] = key[m] != 0ull ? key[m] - kmin + 1 : 0ull;   // valid keys stay > 0
    const uint64_t range = ((uint64_t)(hi_hi - lo_hi) << 32) + 0x100000000ull;   // above every offset key
    const int top = total_valid ? 64 - __clzll((long long)range) : 1;

    // Radix select of the want-th largest offset key, 11 bits at a time from
    // the top of the range, over the keys that share the prefix found so far.
    // Thread t sums bins 2047-2t and 2046-2t; a workgroup scan of those sums
    // from the top bin down gives the keys in higher bins, and the thread
    // whose pair holds the want-th key names the bin.  The select stops as
    // soon as the remaining need equals the count of the chosen bin (keys are
    // distinct, so the last digit always ends it).  Three barriers per pass.
    uint64_t prefix = 0, pmask = 0;
    uint32_t need = want;
    if (want > 0 && want < total_valid) {
        for (int shift = top - kMergeBits, pass = 0; ; shift -= kMergeBits, ++pass) {
            const int sh = shift < 0 ? 0 : shift;
            const int bits = shift < 0 ? kMergeBits + shift : kMergeBits;
            const uint64_t dmask = ((uint64_t)1 << bits) - 1;
            uint32_t *h = hist[pass & 1];
#pragma unroll
            for (int m = 0; m < kMergePer; ++m)
                if (key[m] != 0ull && (key[m] & pmask) == prefix)
                    atomicAdd(&h[(key[m] >> sh) & dmask], 1u);
            __syncthreads();
            const int b_hi = kMergeBins - 1 - 2 * t;
            const uint32_t c_hi = h[b_hi], c_lo = h[b_hi - 1];
            uint32_t *hn = hist[(pass + 1) & 1];   // the next pass's counters
            hn[b_hi] = 0u;
            hn[b_hi - 1] = 0u;
            const uint32_t c = c_hi + c_lo;
            const uint32_t incl = wave_incl_scan(c, lane);
            if (lane == 63) wsum[wave] = incl;
            __syncthreads();
            uint32_t before = incl - c;
#pragma unroll
            for (int w = 0; w < kW; ++w) before += w < wave ? wsum[w] : 0u;
            if (before < need && need <= before + c) {   // exactly one thread
                const bool upper = before + c_hi >= need;
                s_bin = upper ? b_hi : b_hi - 1;
                s_above = upper ? before : before + c_hi;
                s_cnt = upper ? c_hi : c_lo;
            }
            __syncthreads();
            need -= s_above;
            prefix |= (uint64_t)s_bin << sh;
            pmask |= dmask << sh;
            if (s_cnt == need || sh == 0) break;
            // (s_bin, s_above, s_cnt and wsum are written again only after
            // the next pass's second barrier, which every thread reaches
            // after reading them here)
        }
    }
    // The selected keys (masked top bits at or above the prefix; all valid
    // keys when fewer than k are valid) go out in slot order: block g of the
    // candidates first, within a block in slot order (ascending global index
    // for the candidates indexer_shard_candidates writes), then -1.
    uint32_t take = 0;
#pragma unroll
    for (int m = 0; m < kMergePer; ++m)
        take |= (key[m] != 0ull && (want >= total_valid || (key[m] & pmask) >= prefix)) ? (1u << m) : 0u;
    uint32_t taken;
    uint32_t pos = merge_scan((uint32_t)__builtin_popcount(take), wsum2, taken);
    int32_t *out = out_idx + (int64_t)r * k;
#pragma unroll
    for (int m = 0; m < kMergePer; ++m)
        if (take & (1u << m)) {
            if (pos < (uint32_t)k) out[pos] = (int32_t)(0xFFFFFFFFu - (uint32_t)(key[m] + kmin - 1));
            ++pos;
        }
    for (int i = want + t; i < k; i += kMergeThreads) out[i] = -1;
}

hipError_t launch_shard_cand(const float *scores, int64_t sstride, const int32_t *out_idx, int rows, int k,
                             int g, int G, float *cand_score, int32_t *cand_idx, hipStream_t st) {
    hipLaunchKernelGGL(shard_cand_kernel, dim3((k + 255) / 256, rows), dim3(256), 0, st, scores, sstride,
                       out_idx, k, g, G, cand_score, cand_idx);
    return hipGetLastError();
}

hipError_t launch_merge(int rows, int n, int k, const float *cand_score, const int32_t *cand_idx,
                        int32_t *out_idx, hipStream_t st) {
    hipLaunchKernelGGL(merge_kernel, dim3(rows), dim3(kMergeThreads), 0, st, n, k, cand_score, cand_idx,
                       out_idx);
    return hipGetLastError();
}

}  // namespace fp8idx
