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

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(int n, int k, const float *cand_score,
                                                              const int32_t *cand_idx, int32_t *out_idx) {
    __shared__ uint32_t hist[kMergeBins];
    __shared__ uint32_t wsum[kMergeThreads / 64], wsum2[kMergeThreads / 64];   // one per scan
    __shared__ uint64_t wmin[kMergeThreads / 64], wmax[kMergeThreads / 64];
    __shared__ uint32_t s_bin, s_above, s_cnt;
    static_assert(kMergePer <= 16, "merge: a thread's counts fit the five-bit scan");
    const int r = blockIdx.x, t = threadIdx.x, lane = t & 63;
    const float *sc = cand_score + (int64_t)r * n;
    const int32_t *ix = cand_idx + (int64_t)r * n;

    // Thread t holds candidate slots 16t .. 16t+15.  64-bit keys: larger is
    // better (radix key of the score, then the inverted index); an empty
    // slot is 0, below every candidate (a NaN score's key is ~index > 0).
    // (n is a multiple of 16 and the arrays 16-byte aligned: four 16-byte
    // loads per array, all issued before any is used)
    uint64_t key[kMergePer];
    uint32_t valid = 0;
    {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        u32x4 vi[kMergePer / 4], vs[kMergePer / 4];
        const bool here = t * kMergePer < n;
        const int base = here ? t * kMergePer : 0;
#pragma unroll
        for (int q = 0; q < kMergePer / 4; ++q) vi[q] = *(const u32x4 *)(ix + base + 4 * q);
#pragma unroll
        for (int q = 0; q < kMergePer / 4; ++q) vs[q] = *(const u32x4 *)(sc + base + 4 * q);
#pragma unroll
        for (int m = 0; m < kMergePer; ++m) {
            const int32_t id = here ? (int32_t)vi[m >> 2][m & 3] : -1;
            const float f = __uint_as_float(vs[m >> 2][m & 3]);
            key[m] = id >= 0 ? ((uint64_t)radix_key(f) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)id) : 0ull;
            valid += id >= 0;
        }
    }
    uint32_t total_valid;   // the row's valid candidates
    (void)merge_scan(valid, wsum, total_valid);
    const uint32_t want = total_valid < (uint32_t)k ? total_valid : (uint32_t)k;

    // The candidates are the shards' top-k: their scores crowd into a narrow
    // band, so the top bits of the keys are nearly all equal and a first digit
    // taken there would send every atomic to a handful of bins.  The select
    // runs on the offset key (key - min over the row's valid keys, + 1), whose
    // first digit starts at the top bit of the range; the order is the same.
    uint64_t kmin = ~0ull, kmax = 0ull;
#pragma unroll
    for (int m = 0; m < kMergePer; ++m)
        if (key[m] != 0ull) { kmin = key[m] < kmin ? key[m] : kmin; kmax = key[m] > kmax ? key[m] : kmax; }
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t a = __shfl_xor(kmin, off), b = __shfl_xor(kmax, off);
        kmin = a < kmin ? a : kmin;
        kmax = b > kmax ? b : kmax;
    }
    if (lane == 0) { wmin[t >> 6] = kmin; wmax[t >> 6] = kmax; }
    __syncthreads();
    kmin = ~0ull; kmax = 0ull;
    for (int w = 0; w < kMergeThreads / 64; ++w) {
        kmin = wmin[w] < kmin ? wmin[w] : kmin;
        kmax = wmax[w] > kmax ? wmax[w] : kmax;
    }
#pragma unroll
    for (int m = 0; m < kMergePer; ++m) key[m] = key[m] != 0ull ? key[m] - kmin + 1 : 0ull;   // valid keys stay > 0
    const int top = kmax >= kmin ? 64 - __clzll((long long)(kmax - kmin + 1)) : 1;   // bits of the offset keys

    // Radix select of the want-th largest offset key, 11 bits at a time from
    // the top of the range, over the keys that share the prefix found so far.
    // Wave 0 finds the bin: lane l sums bins 2047-32l down to 2016-32l, a wave
    // scan gives the keys in higher bins, the lane holding the want-th key
    // walks its 32 bins.  The select stops as soon as the remaining need
    // equals the count of the chosen bin (keys are distinct, so the last
    // digit always ends it).
    uint64_t prefix = 0, pmask = 0;
    uint32_t need = want;
    if (want > 0 && want < total_valid) {
        for (int shift = top - kMergeBits; ; shift -= kMergeBits) {
            const int sh = shift < 0 ? 0 : shift;
            const int bits = shift < 0 ? kMergeBits + shift : kMergeBits;
            const uint64_t dmask = ((uint64_t)1 << bits) - 1;
            for (int i = t; i < kMergeBins; i += kMergeThreads) hist[i] = 0;
            __syncthreads();
#pragma unroll
            for (int m = 0; m < kMergePer; ++m)
                if (key[m] != 0ull && (key[m] & pmask) == prefix)
                    atomicAdd(&hist[(key[m] >> sh) & dmask], 1u);
            __syncthreads();
            if (t < 64) {
                const int hi = kMergeBins - 1 - 32 * lane;   // this lane's bins: hi, hi-1, ..., hi-31
                uint32_t hv[32];
                uint32_t mine = 0;
#pragma unroll
                for (int j = 0; j < 32; ++j) { hv[j] = hist[hi - j]; mine += hv[j]; }
                uint32_t incl = mine;
                for (int off = 1; off < 64; off <<= 1) {
                    const uint32_t y = __shfl_up(incl, off);
                    if (lane >= off) incl += y;
                }
                const uint32_t before = incl - mine;
                if (before < need && need <= incl) {   // walk the counts in registers
                    uint32_t cum = before;
                    int jb = 31;
                    uint32_t ab = 0, cb = 0;
                    bool found = false;
#pragma unroll
                    for (int j = 0; j < 32; ++j) {
                        const bool here = !found && cum + hv[j] >= need;
                        jb = here ? j : jb;
                        ab = here ? cum : ab;
                        cb = here ? hv[j] : cb;
                        found = found || here;
                        cum += hv[j];
                    }
                    s_bin = hi - jb; s_above = ab; s_cnt = cb;
                }
            }
            __syncthreads();
            need -= s_above;
            prefix |= (uint64_t)s_bin << sh;
            pmask |= dmask << sh;
            const bool done = s_cnt == need || sh == 0;
            __syncthreads();
            if (done) break;
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
