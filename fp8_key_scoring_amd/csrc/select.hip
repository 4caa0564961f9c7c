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
//   d3 = bits 17..10 (256 bins)  counted by gather_kernel over the candidates
// The 14-bit prefix (d1, d2) of the k-th largest key splits a row into
//   "sure" keys (prefix above it: all selected) and
//   candidates (prefix equal: the remaining `need` are chosen among them).
// Kernels, one after the other on the stream (a kernel boundary is the only
// hand-off between workgroups: an agent-scope release inside a kernel writes
// back the whole L2 of an XCD, which costs far more than a dependent launch):
//   hist1    (only for indexer_topk) first-digit counts of stored scores;
//   refine   second-digit counts inside the first-digit bin, added to the
//            row's histogram (copy x % kHist2Slots for workgroup x) with one atomic per non-empty bin
//            (the first workgroup also records the first-digit bin);
//   gather   every workgroup derives the same split from that bin and the
//            second-digit histogram, writes its sure keys and candidates as
//            one list in index order to its own slice of the workspace
//            (ballot prefix sums, no atomics; a flag marks the sure keys),
//            and adds its candidates' third digits to the row's third
//            histogram;
//   finalize one workgroup per row: the slices, concatenated, are the row's
//            entries in index order; the third digit's bin of the k-th key
//            splits the candidates once more; all above it are taken, the few
//            inside it are ranked by (key desc, index asc); a stable
//            compaction of the kept entries is the row's output in ascending
//            index order (deterministic bytes), with no sort and no merge.
// Workgroups are 1024 threads (four waves per SIMD hide LDS latency) and each
// thread keeps 8 score loads in flight, so a workgroup's scan of its 8192
// keys is one memory round trip.  Rows whose candidates overflow the slices
// (heavy ties) are resolved exactly by finalize rescanning the row with three
// more digit passes and taking ties in index order.
#include "common.h"

namespace fp8idx {

constexpr int kWaves = kSelThreads / 64;
static_assert(kSelThreads == 1024, "selection workgroups are 16 waves");
static_assert(kSelUnroll * kWaves == 128, "gather prefix: two entries per lane");
static_assert(kHist1Slots * kBins1 <= kSelThreads, "finalize clears the first-digit copies in one pass");

__device__ __forceinline__ uint32_t lane_prefix(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Executed by one full wave.  h: 64 * PER bins in LDS.  Finds the largest
// bin B with sum_{b >= B} h[b] >= need (need >= 1) and the count strictly
// above B.  Results land in *outB / *outAbove (LDS), written by one lane.
// A lane's PER counts stay in registers for the final walk.
template <int PER>
__device__ __forceinline__ void wave_find_bin(const uint32_t *h, uint32_t need, int lane, int *outB,
                                              uint32_t *outAbove) {
    uint32_t c[PER], mine = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        c[j] = h[lane * PER + j];
        mine += c[j];
    }
    const uint32_t incl = wave_incl_scan(mine, lane);
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    const uint32_t above_lane = total - incl;   // lanes after this one (higher bins)
    const uint64_t m = __ballot((above_lane < need) & (need <= above_lane + mine));
    if (m && lane == __ffsll((unsigned long long)m) - 1) {
        uint32_t cum = above_lane;
#pragma unroll
        for (int j = PER - 1; j >= 0; --j) {
            if (cum + c[j] >= need) {
                *outB = lane * PER + j;
                *outAbove = cum;
                break;
            }
            cum += c[j];
        }
    }
}

// Executed by one full wave: c[0..128) becomes its exclusive prefix sum (in
// index order); *total gets the sum.
__device__ void wave_scan128(uint32_t *c, uint32_t *total, int lane) {
    const uint32_t c0 = c[2 * lane], c1 = c[2 * lane + 1];
    const uint32_t incl = wave_incl_scan(c0 + c1, lane);
    const uint32_t excl = incl - c0 - c1;
    c[2 * lane] = excl;
    c[2 * lane + 1] = excl + c0;
    if (lane == 63) *total = incl;
}

// Exclusive prefix over the workgroup, in thread order, of a v < 8 per
// thread: within a wave three ballots (one per bit of v) and their lane
// prefixes, across waves one barrier and the wave totals.  wsum must not be
// written again by the workgroup after this call.
__device__ uint32_t block_scan_small(uint32_t v, uint32_t *wsum) {
    const int t = threadIdx.x, wave = t >> 6;
    uint32_t pre = 0, tot = 0;
#pragma unroll
    for (int bit = 0; bit < 3; ++bit) {
        const uint64_t m = __ballot((v >> bit) & 1u);
        pre += lane_prefix(m) << bit;
        tot += (uint32_t)__popcll(m) << bit;
    }
    if ((t & 63) == 0) wsum[wave] = tot;
    __syncthreads();
    uint32_t off = 0;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    return off + pre;
}

// Radix keys of keys base + j*kSelThreads + t (j < kSelUnroll) into
// registers; every load is issued before any is used.  Positions at or past
// s1 (> base) re-read key s1 - 1, so no load sits behind a branch; callers
// test the position.
__device__ __forceinline__ void load_raw(const float *row, int64_t base, int64_t s1, float (&v)[kSelUnroll]) {
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < kSelUnroll; ++j) {
        const int64_t s = base + j * kSelThreads + t;
        v[j] = row[s < s1 ? s : s1 - 1];
    }
}
__device__ __forceinline__ void to_keys(const float (&v)[kSelUnroll], uint32_t (&u)[kSelUnroll]) {
#pragma unroll
    for (int j = 0; j < kSelUnroll; ++j) u[j] = radix_key(v[j]);
}
__device__ __forceinline__ void load_keys(const float *row, int64_t base, int64_t s1,
                                          uint32_t (&u)[kSelUnroll]) {
    float v[kSelUnroll];
    load_raw(row, base, s1, v);
    to_keys(v, u);
}

__device__ __forceinline__ int clamp_bound(int b, int max_bound) {
    return b < 0 ? 0 : (b > max_bound ? max_bound : b);
}

// Row r's count in first-digit bin `bin` is the sum of its kHist1Slots
// copies: loaded by hist1_load, summed by hist1_sum (split so that other
// loads can be issued in between).
__device__ __forceinline__ void hist1_load(const SelectArgs &a, int r, int bin, uint32_t (&c)[kHist1Slots]) {
    const uint32_t *h = (const uint32_t *)(a.ws + a.L.hist1) + (int64_t)r * kHist1Slots * kBins1 + bin;
#pragma unroll
    for (int s = 0; s < kHist1Slots; ++s) c[s] = h[s * kBins1];
}
__device__ __forceinline__ uint32_t hist1_sum(const uint32_t (&c)[kHist1Slots]) {
    uint32_t v = 0;
#pragma unroll
    for (int s = 0; s < kHist1Slots; ++s) v += c[s];
    return v;
}

// ---------------------------------------------------------------- hist1
// First-digit histogram of stored scores (used when the scores were not
// produced by this launch's scoring pass).  One LDS copy per wave.
__device__ __forceinline__ void hist1_body(const SelectArgs &a, int x, int r) {
    __shared__ uint32_t h[kWaves][kBins1];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int b = clamp_bound(a.row_bound[r], a.max_bound);
    const int64_t s0 = (int64_t)x * a.L.sel_chunk;
    if (s0 >= b) return;
    const int64_t s1 = min(s0 + a.L.sel_chunk, (int64_t)b);
    const float *row = a.scores + (int64_t)r * a.sstride;
    uint32_t u[kSelUnroll];
    load_keys(row, s0, s1, u);
    h[wave][lane] = 0;
    __syncthreads();
    for (int64_t base = s0; base < s1; base += kSelTile) {
        if (base != s0) load_keys(row, base, s1, u);
#pragma unroll
        for (int j = 0; j < kSelUnroll; ++j)
            if (base + j * kSelThreads + t < s1) atomicAdd(&h[wave][u[j] >> kDigit1Shift], 1u);
    }
    __syncthreads();
    if (t < kBins1) {
        uint32_t c = 0;
        for (int w = 0; w < kWaves; ++w) c += h[w][t];
        if (c) atomicAdd((uint32_t *)(a.ws + a.L.hist1) + ((int64_t)r * kHist1Slots + x % kHist1Slots) * kBins1 + t, c);
    }
}

// ---------------------------------------------------------------- refine
// Second-digit counts inside the first-digit bin of the k-th largest key.
// Four LDS copies (wave % 4) keep the waves' atomics apart; with one copy per
// wave the zeroing and the final sum over 16 copies cost more than the
// collisions they avoid (256 rows of 8K-262K keys: the launch 3 us longer).
__device__ __forceinline__ void refine_body(const SelectArgs &a, int x, int r) {
    __shared__ uint32_t h1[kBins1];
    __shared__ uint32_t h2[4][kBins2];
    __shared__ int sb1;
    __shared__ uint32_t sabove1;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int b = clamp_bound(a.row_bound[r], a.max_bound);
    const uint32_t k = (uint32_t)a.topk;
    const int64_t s0 = (int64_t)x * a.L.sel_chunk;
    if ((uint32_t)b <= k || s0 >= b) return;   // all selected, or nothing here
    const int64_t s1 = min(s0 + a.L.sel_chunk, (int64_t)b);
    const float *row = a.scores + (int64_t)r * a.sstride;

    // the first-digit counts are loaded before the first step's keys: loads
    // complete in order, so the digit search then waits on the counts alone
    // while the keys are in flight
    uint32_t c1[kHist1Slots] = {};
    if (wave == 0) hist1_load(a, r, lane, c1);
    __builtin_amdgcn_sched_barrier(0);
    float v0[kSelUnroll];
    load_raw(row, s0, s1, v0);
    __builtin_amdgcn_sched_barrier(0);
    if (t < kBins1) h1[t] = hist1_sum(c1);
    for (int i = t; i < 4 * kBins2; i += kSelThreads) (&h2[0][0])[i] = 0;
    if (t == 0) { sb1 = 0; sabove1 = 0; }
    __syncthreads();
    if (t < 64) wave_find_bin<1>(h1, k, lane, &sb1, &sabove1);
    __syncthreads();
    const uint32_t b1 = (uint32_t)sb1;
    if (x == 0 && t == 0) {   // the split's first half, for gather
        RowState *st = (RowState *)(a.ws + a.L.state) + r;
        st->b1 = b1;
        st->above1 = sabove1;
    }
    uint32_t u[kSelUnroll];
    to_keys(v0, u);
    for (int64_t base = s0; base < s1; base += kSelTile) {
        if (base != s0) load_keys(row, base, s1, u);
#pragma unroll
        for (int j = 0; j < kSelUnroll; ++j)
            if (base + j * kSelThreads + t < s1 && (u[j] >> kDigit1Shift) == b1)
                atomicAdd(&h2[wave & 3][(u[j] >> kDigit2Shift) & (kBins2 - 1)], 1u);
    }
    __syncthreads();
    if (t < kBins2) {
        uint32_t c = 0;
        for (int w = 0; w < 4; ++w) c += h2[w][t];
        if (c) atomicAdd((uint32_t *)(a.ws + a.L.hist2) + ((int64_t)r * kHist2Slots + x % kHist2Slots) * kBins2 + t, c);
    }
}

// ---------------------------------------------------------------- gather
// Every workgroup of a row derives the same split from the two histograms,
// writes its sure keys and candidates (each ascending) to its own slices and
// counts the candidates' third digits.
__device__ __forceinline__ void gather_body(const SelectArgs &a, int x, int r) {
    __shared__ uint32_t h2[kBins2];
    __shared__ uint32_t h3[kBins3];
    __shared__ uint32_t cs[kSelUnroll * kWaves], cc[kSelUnroll * kWaves];
    __shared__ int sb2;
    __shared__ uint32_t sabove2, tot_s, tot_c;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int b = clamp_bound(a.row_bound[r], a.max_bound);
    const int k = a.topk;
    const int S = a.L.sel_wgs;
    int32_t *out_row = a.out_idx + (int64_t)r * k;
    if (b <= k) {   // every key selected: indices 0..b-1, then -1
        if (x == 0)
            for (int i = t; i < k; i += kSelThreads) out_row[i] = i < b ? i : -1;
        return;
    }
    const int64_t s0 = (int64_t)x * a.L.sel_chunk;
    if (s0 >= b) return;   // past the row's bound: finalize counts this slice as empty
    unsigned long long *slice_e = (unsigned long long *)(a.ws + a.L.ent_list) + ((int64_t)r * S + x) * kSliceCap;
    const float *row = a.scores + (int64_t)r * a.sstride;
    const int64_t s1 = min(s0 + a.L.sel_chunk, (int64_t)b);

    // ---- the split: (b1, above1) as refine found them, (b2, above2) from
    // the second digit.  The state and counts are loaded before the first
    // step's keys (loads complete in order), so the split waits on them
    // alone and the key loads overlap it.  The count copies are loaded by
    // the four waves that sum them (a wave-uniform condition).
    const RowState *st_in = (const RowState *)(a.ws + a.L.state) + r;
    const uint32_t b1 = st_in->b1, above1 = st_in->above1;
    uint32_t c2s[kHist2Slots] = {};   // the row's second-digit counts: the sum of its copies
    if (t < kBins2) {                  // (waves 0-3: a wave-uniform branch)
#pragma unroll
        for (int sl = 0; sl < kHist2Slots; ++sl)
            c2s[sl] = ((const uint32_t *)(a.ws + a.L.hist2))[((int64_t)r * kHist2Slots + sl) * kBins2 + t];
    }
    __builtin_amdgcn_sched_barrier(0);
    float v0[kSelUnroll];
    load_raw(row, s0, s1, v0);   // (b > k >= 1, so key s1 - 1 exists also when s0 >= s1)
    __builtin_amdgcn_sched_barrier(0);
    if (t < kBins2) {
        uint32_t c2 = 0;
#pragma unroll
        for (int sl = 0; sl < kHist2Slots; ++sl) c2 += c2s[sl];
        h2[t] = c2;
        h3[t] = 0;
    }
    if (t == 0) { sb2 = 0; sabove2 = 0; }
    __syncthreads();
    if (t < 64) wave_find_bin<kBins2 / 64>(h2, (uint32_t)k - above1, lane, &sb2, &sabove2);
    __syncthreads();
    const uint32_t b2 = (uint32_t)sb2;
    const uint32_t T14 = (b1 << kDigit2Bits) | b2;
    if (x == 0 && t == 0) {
        RowState st;
        st.b1 = b1;
        st.b2 = b2;
        st.sure = above1 + sabove2;
        st.need = (uint32_t)k - st.sure;
        st.cand = h2[b2];
        st.above1 = above1;
        st.pad[0] = st.pad[1] = 0;
        ((RowState *)(a.ws + a.L.state))[r] = st;
    }

    uint32_t we_ = 0, wc_ = 0;   // entries / candidates of this workgroup so far
    uint32_t u[kSelUnroll];
    if (s0 < s1) to_keys(v0, u);
    for (int64_t base = s0; base < s1; base += kSelTile) {
        if (base != s0) load_keys(row, base, s1, u);
        // pass 1: entry and candidate counts per (step j, wave), in key
        // order; third digits of candidates
#pragma unroll
        for (int j = 0; j < kSelUnroll; ++j) {
            const bool valid = base + j * kSelThreads + t < s1;
            const uint32_t top = u[j] >> kDigit2Shift;
            const bool cnd = valid && top == T14;
            const uint64_t me = __ballot(valid && top >= T14);
            const uint64_t mc = __ballot(cnd);
            if (lane == 0) {
                cs[j * kWaves + wave] = (uint32_t)__popcll(me);
                cc[j * kWaves + wave] = (uint32_t)__popcll(mc);
            }
            if (cnd) atomicAdd(&h3[(u[j] >> kDigit3Shift) & (kBins3 - 1)], 1u);
        }
        __syncthreads();
        if (wave == 0) wave_scan128(cs, &tot_s, lane);
        if (wave == 1) wave_scan128(cc, &tot_c, lane);
        __syncthreads();
        // pass 2: each entry to its place (sure keys carry a flag, candidates
        // their key)
#pragma unroll
        for (int j = 0; j < kSelUnroll; ++j) {
            const int64_t s = base + j * kSelThreads + t;
            const uint32_t top = u[j] >> kDigit2Shift;
            const bool ent = s < s1 && top >= T14;
            const uint64_t me = __ballot(ent);
            if (ent) {
                const uint32_t pos = we_ + cs[j * kWaves + wave] + lane_prefix(me);
                const uint32_t lo = (uint32_t)s | (top > T14 ? 0x80000000u : 0u);
                if (pos < (uint32_t)kSliceCap) slice_e[pos] = ((unsigned long long)u[j] << 32) | lo;
            }
        }
        we_ += tot_s;
        wc_ += tot_c;
        __syncthreads();
    }
    if (t == 0) {
        ((uint32_t *)(a.ws + a.L.ent_cnt))[(int64_t)r * S + x] = we_;
        ((uint32_t *)(a.ws + a.L.cand_cnt))[(int64_t)r * S + x] = wc_;
    }
    if (t < kBins3 && h3[t]) atomicAdd((uint32_t *)(a.ws + a.L.hist3) + (int64_t)r * kBins3 + t, h3[t]);
}

// ------------------------------------------------------------- fallback
// Exact resolution inside the 14-bit prefix bin T14 by one workgroup, used
// when the row's entries overflow the slices or finalize's LDS (heavy ties,
// or a very crowded bin).  h3 (LDS) holds gather's third-digit counts of every
// key in the bin (counted in full, whatever overflowed), so the third digit
// needs no pass: it gives the 22-bit prefix of the k-th largest key T and the
// keys still to take inside it.  One pass over the row counts the last 10
// bits of the keys with that prefix (each thread adds a run of equal digits
// at once: equal keys are the case here, and adds to one LDS word
// serialize), which fixes T.  A last pass in index order writes the keys above T and the first
// ties at T (ascending index), each thread taking 32 consecutive keys, and
// stops once the row's output is complete.  Both passes keep eight 16-byte
// loads per thread in flight (32K keys per workgroup step).
// Heavy-tie fallback, part 1: adds to h10 (LDS, kFbBins counters) the last
// 10 bits of every key in [s0, s1) whose top 22 bits are T22.  Each step
// loads 8 x 16 bytes per thread (32K keys), all issued before any is used.
constexpr int kFbVec = 8;
constexpr int64_t kFbStep = (int64_t)kFbVec * 4 * kSelThreads;
// A step's keys into registers, every load issued before any is used:
// 16-byte loads when the whole step lies below `end` and the row is 16-byte
// aligned (a caller's score rows need only be 4-byte aligned), else 4-byte
// loads at clamped positions (callers test the position).  idx(j) is the
// first of the four keys of load j.
template <typename Idx>
__device__ __forceinline__ void fb_step_keys(const float *row, int64_t base, int64_t end, Idx idx,
                                             uint32_t (&u)[kFbVec][4]) {
    const bool al16 = ((uintptr_t)row & 15) == 0;
    if (al16 && base + kFbStep <= end) {   // (uniform)
#pragma unroll
        for (int j = 0; j < kFbVec; ++j) {
            const u32x4_t v = *(const u32x4_t *)(row + idx(j));
            u[j][0] = v[0]; u[j][1] = v[1]; u[j][2] = v[2]; u[j][3] = v[3];
        }
    } else {
#pragma unroll
        for (int j = 0; j < kFbVec; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t sj = idx(j) + e;
                u[j][e] = __float_as_uint(row[sj < end ? sj : end - 1]);
            }
    }
#pragma unroll
    for (int j = 0; j < kFbVec; ++j)   // raw bits -> radix keys, in place
#pragma unroll
        for (int e = 0; e < 4; ++e) u[j][e] = radix_key(__uint_as_float(u[j][e]));
}

__device__ __forceinline__ void fallback_count(const float *row, int64_t s0, int64_t s1, uint32_t T22, uint32_t *h10) {
    const int t = threadIdx.x;
    constexpr uint32_t kNone = 0xFFFFFFFFu;
    uint32_t u[kFbVec][4];
    for (int64_t base = s0; base < s1; base += kFbStep) {
        fb_step_keys(row, base, s1, [&](int j) { return base + ((int64_t)j * kSelThreads + t) * 4; }, u);
        // runs of equal digits within a thread's keys are added at once (ties
        // are the case here, and adds to one LDS word serialize)
        uint32_t run_d = kNone, run_n = 0;
#pragma unroll
        for (int j = 0; j < kFbVec; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t s = base + ((int64_t)j * kSelThreads + t) * 4 + e;
                const uint32_t uk = u[j][e];
                if (s < s1 && (uk >> kFbBits) == T22) {
                    const uint32_t d = uk & (kFbBins - 1);
                    if (d != run_d) {
                        if (run_n) atomicAdd(&h10[run_d], run_n);
                        run_d = d;
                        run_n = 0;
                    }
                    ++run_n;
                }
            }
        if (run_n) atomicAdd(&h10[run_d], run_n);
    }
}

// Part 2 (one workgroup): with T the k-th largest key and need3 the keys
// equal to T to take, writes the row's selection in ascending index order:
// thread t takes the 32 consecutive keys base + 32t .. base + 32t + 31 of
// each step, exclusive prefixes over the workgroup of the tie and the
// greater-than counts place them; stops once k keys are out.
__device__ __forceinline__ void fallback_output(const float *row, int b, uint32_t T, uint32_t need3, int32_t *out_row, int k,
                                uint32_t *wsum) {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    uint32_t u[kFbVec][4];
    uint32_t sel_run = 0, tie_run = 0;
    for (int64_t base = 0; base < b && sel_run < (uint32_t)k; base += kFbStep) {
        const int64_t s0 = base + (int64_t)kFbVec * 4 * t;
        fb_step_keys(row, base, (int64_t)b, [&](int j) { return s0 + 4 * j; }, u);
        uint32_t ngt = 0, ntie = 0;
#pragma unroll
        for (int j = 0; j < kFbVec; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool ok = s0 + 4 * j + e < b;
                ngt += ok && u[j][e] > T;
                ntie += ok && u[j][e] == T;
            }
        // exclusive prefixes over the workgroup of the tie and the
        // greater-than counts (both <= 32 per thread: ballots on 6 bits)
        uint32_t tpre = 0, gpre = 0, ttot = 0, gtot = 0;
#pragma unroll
        for (int bit = 0; bit < 6; ++bit) {
            const uint64_t mt = __ballot((ntie >> bit) & 1u), mg = __ballot((ngt >> bit) & 1u);
            tpre += lane_prefix(mt) << bit;
            gpre += lane_prefix(mg) << bit;
            ttot += (uint32_t)__popcll(mt) << bit;
            gtot += (uint32_t)__popcll(mg) << bit;
        }
        if (lane == 0) { wsum[wave] = ttot; wsum[kWaves + wave] = gtot; }
        __syncthreads();
        uint32_t toff = 0, goff = 0, tall = 0, gall = 0;
        for (int w = 0; w < kWaves; ++w) {
            if (w < wave) { toff += wsum[w]; goff += wsum[kWaves + w]; }
            tall += wsum[w];
            gall += wsum[kWaves + w];
        }
        __syncthreads();   // wsum is written again in the next step
        uint32_t tr = tie_run + toff + tpre;   // ties before this thread's keys
        uint32_t pos_g = goff + gpre;           // greater keys before them in this step
        for (int j = 0; j < kFbVec; ++j)
            for (int e = 0; e < 4; ++e) {
                const int64_t s = s0 + 4 * j + e;
                if (s >= b) break;
                const uint32_t uk = u[j][e];
                bool sel = uk > T;
                if (uk == T) { sel = tr < need3; ++tr; }
                if (sel) {
                    // selected keys before this one: earlier steps' (sel_run),
                    // this step's greater keys and taken ties before it
                    const uint32_t taken_ties_before = min(tr - (uk == T ? 1u : 0u), need3) - min(tie_run, need3);
                    const uint32_t pos = sel_run + pos_g + taken_ties_before;
                    if (pos < (uint32_t)k) out_row[pos] = (int32_t)s;
                }
                if (uk > T) ++pos_g;
            }
        sel_run += gall + min(tie_run + tall, need3) - min(tie_run, need3);
        tie_run += tall;
    }
}

// -------------------------------------------------------------- finalize
// Workgroup 0 of a row: the slices' entries (sure keys and candidates, each
// slice in ascending index, slices in index order) are gathered into LDS in
// one ascending list; the third digit's bin of the k-th key splits the
// candidates once more (all above it are taken, the few inside it ranked by
// key desc, index asc); a stable compaction of the kept entries is the row's
// output in ascending index order.
// Heavy ties (candidates past the slices' capacity, or more keys in the
// third-digit bin than it ranks): every workgroup of the row (L.fb_wgs, each
// deciding so from the same counts) counts the last 10 bits of the bin's keys
// over its share of the row into the row's global counters; the last one to
// arrive finds the k-th key and writes the selection.  Every workgroup of the
// row arrives at a counter; the last one leaves the row's histograms and
// counters zeroed, after every read of them.
__device__ __forceinline__ void finalize_body(const SelectArgs &a, int xw, int r) {
    __shared__ unsigned long long ent[kEntCap];   // the row's entries, ascending index
    __shared__ unsigned long long tie[kTieCap];   // candidates inside the third-digit bin
    __shared__ uint32_t offe[kSelMaxWgs + 1];
    __shared__ uint32_t roff[kSelMaxWgs + 1];    // exclusive prefix of the entries past 16*kPre per slice
    __shared__ uint32_t h3[kBins3];
    __shared__ uint32_t wsum[kWaves], wsum2[2 * kWaves];
    __shared__ int sB, sB10;
    __shared__ uint32_t sAbove, sAbove10, ntie, ovf, s_ticket, s_late;
    constexpr int kPer = kEntCap / kSelThreads;   // entries per thread
    constexpr int kPre = 4;                       // entries per thread loaded ahead of the counts
    static_assert(kPer < 8, "finalize: a thread's kept count fits the three-bit scan");
    static_assert(kEntCap % kSelThreads == 0, "finalize: whole entries per thread");
    static_assert(kSelMaxWgs * 16 == kSelThreads, "finalize: at least 16 threads per slice");
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int nfb = a.L.fb_wgs;
    const int k = a.topk;
    const int S = a.L.sel_wgs;
    int32_t *out_row = a.out_idx + (int64_t)r * k;
    uint32_t *hist3 = (uint32_t *)(a.ws + a.L.hist3) + (int64_t)r * kBins3;
    // Every load goes out before any is waited on, the row's bound included
    // (one workgroup per row, so none of them is wasted but for rows whose
    // keys are all selected, where the state and lists are stale and unused):
    // the bound, the state, the third digits, the per-slice counts and,
    // without waiting for those, the first kPre * tps entries of every slice
    // (tps = 1024 / S rounded down to a power of two threads per slice: 64
    // entries at 64 slices, 256 at 16), which is all of a slice in the usual
    // case (a slice's share of the row's ~2,048 entries grows as S shrinks).
    const int b_raw = a.row_bound[r];
    const uint32_t *ecnt = (const uint32_t *)(a.ws + a.L.ent_cnt) + (int64_t)r * S;
    const uint32_t *ccnt = (const uint32_t *)(a.ws + a.L.cand_cnt) + (int64_t)r * S;
    const unsigned long long *sl = (const unsigned long long *)(a.ws + a.L.ent_list) + (int64_t)r * S * kSliceCap;
    const int tsh = 10 - (S > 1 ? 32 - __builtin_clz((uint32_t)(S - 1)) : 0);   // log2(tps)
    const int tps = 1 << tsh;
    const int x = t >> tsh, j0 = t & (tps - 1);
    const int xs = x < S ? x : 0;
    const RowState st = ((const RowState *)(a.ws + a.L.state))[r];
    const uint32_t h3v = hist3[t & (kBins3 - 1)];
    const uint32_t ne = ecnt[lane < S ? lane : 0], ncx = ccnt[lane < S ? lane : 0];
    unsigned long long pre[kPre];
#pragma unroll
    for (int m = 0; m < kPre; ++m) pre[m] = sl[(int64_t)xs * kSliceCap + min(j0 + tps * m, kSliceCap - 1)];
    __builtin_amdgcn_sched_barrier(0);
    const int b = clamp_bound(b_raw, a.max_bound);
    bool overflow = false;        // heavy ties: the row takes the fallback
    uint32_t T22 = 0, need2 = 0;  // the k-th key's top 22 bits, keys to take inside that bin
    if (b > k) {
        // slices that start at or past the bound were not written: empty
        const bool live = lane < S && (int64_t)lane * a.L.sel_chunk < b;
        const int need = (int)(st.need < (uint32_t)kMaxTopk ? st.need : (uint32_t)kMaxTopk);
        const uint32_t T14 = (st.b1 << kDigit2Bits) | st.b2;
        // slice offsets (exclusive prefix of the entry counts); candidates
        // past a slice's capacity or the row's send the row to the fallback
        if (wave == 0) {
            const uint32_t c = live ? ne : 0u, cc = live ? ncx : 0u;
            const uint32_t rm = c > (uint32_t)(tps * kPre) ? c - (uint32_t)(tps * kPre) : 0u;
            // a slice holding more entries than its capacity (possible only
            // with counters left dirty by a misused workspace) is never read
            // past its end: the row takes the fallback instead
            const uint64_t big = __ballot(cc > (uint32_t)kCandSlice || c > (uint32_t)kSliceCap);
            const uint32_t incl = wave_incl_scan(c, lane), cincl = wave_incl_scan(cc, lane),
                           rincl = wave_incl_scan(rm, lane);
            offe[lane] = incl - c;
            roff[lane] = rincl - rm;
            if (lane == 63) {
                offe[kSelMaxWgs] = incl;
                roff[kSelMaxWgs] = rincl;
                ovf = (big != 0ull) || cincl > (uint32_t)kCandCap || incl > (uint32_t)kEntCap;
            }
        }
        if (t < kBins3) h3[t] = h3v;
        if (t == 0) { sB = 0; sAbove = 0; ntie = 0; s_late = 0; }
        __syncthreads();
        // the third-digit bin of the k-th key and the keys in it: the same
        // decision in every workgroup of the row
        if (t < 64) wave_find_bin<kBins3 / 64>(h3, (uint32_t)need, lane, &sB, &sAbove);
        __syncthreads();
        const int N = (int)offe[kSelMaxWgs];
        overflow = ovf != 0u || h3[sB] > (uint32_t)kTieCap;
        T22 = (T14 << kDigit3Bits) | (uint32_t)sB;
        need2 = (uint32_t)need - sAbove;
        unsigned long long e[kPer];
        if (!overflow && xw == 0) {
            if (x < S) {
                const int o = (int)offe[x], n = (int)(offe[x + 1] - offe[x]);
#pragma unroll
                for (int m = 0; m < kPre; ++m)
                    if (j0 + tps * m < n) ent[o + j0 + tps * m] = pre[m];
            }
            // entries past the first tps*kPre of their slice (a short row puts
            // all its entries in one or two slices): spread over every thread,
            // each finding its slice by a binary search of roff; all loads go
            // out before any is stored
            const int NR = (int)roff[kSelMaxWgs];
            if (NR > 0) {
                int dst[kPer];
                unsigned long long v[kPer];
#pragma unroll
                for (int m = 0; m < kPer; ++m) {
                    const int i = m * kSelThreads + t;
                    dst[m] = -1;
                    if (i < NR) {
                        int lo = 0, hi = S - 1;   // the last slice with roff <= i
                        while (lo < hi) {
                            const int mid = (lo + hi + 1) >> 1;
                            if ((int)roff[mid] <= i) lo = mid; else hi = mid - 1;
                        }
                        const int jj = tps * kPre + (i - (int)roff[lo]);
                        dst[m] = (int)offe[lo] + jj;
                        v[m] = sl[(int64_t)lo * kSliceCap + jj];
                    }
                }
#pragma unroll
                for (int m = 0; m < kPer; ++m)
                    if (dst[m] >= 0) ent[dst[m]] = v[m];
            }
            __syncthreads();
            // this thread's entries t*kPer .. t*kPer+kPer-1; candidates in the
            // third-digit bin are collected for ranking
#pragma unroll
            for (int q = 0; q < kPer; ++q) {
                const int i = t * kPer + q;
                e[q] = i < N ? ent[i] : 0ull;
                const bool cand_in_bin = i < N && !((uint32_t)e[q] & 0x80000000u) &&
                                         (uint32_t)(e[q] >> (32 + kDigit3Shift)) == T22;
                if (cand_in_bin) {
                    const uint32_t p = atomicAdd(&ntie, 1u);
                    if (p < (uint32_t)kTieCap) tie[p] = e[q];
                }
            }
            __syncthreads();
            // (more ties than the bin's count only with counters left dirty
            // by a misused workspace: this workgroup then counts the whole
            // row alone, below)
            if (t == 0 && ntie > (uint32_t)kTieCap) s_late = 1;
            __syncthreads();
        }
        if (!overflow && xw == 0 && !s_late) {
            const uint32_t need3 = need2;
            const int nt = (int)ntie;
            bool kept[kPer];
            uint32_t cnt = 0;
#pragma unroll
            for (int q = 0; q < kPer; ++q) {
                kept[q] = false;
                if (t * kPer + q < N) {
                    const uint32_t lo = (uint32_t)e[q];
                    const uint32_t key = (uint32_t)(e[q] >> 32);
                    const uint32_t d = key >> kDigit3Shift;
                    if (lo & 0x80000000u) {   // sure key
                        kept[q] = true;
                    } else if (d > T22) {
                        kept[q] = true;
                    } else if (d == T22) {   // rank inside the bin: larger key first, then lower index
                        const uint32_t idx = lo;
                        uint32_t rank = 0;
                        for (int f = 0; f < nt; ++f) {
                            const uint32_t ek = (uint32_t)(tie[f] >> 32), ei = (uint32_t)tie[f];
                            rank += (ek > key) || (ek == key && ei < idx);
                        }
                        kept[q] = rank < need3;
                    }
                }
                cnt += kept[q];
            }
            uint32_t pos = block_scan_small(cnt, wsum);
#pragma unroll
            for (int q = 0; q < kPer; ++q)
                if (kept[q]) {
                    if (pos < (uint32_t)k) out_row[pos] = (int32_t)((uint32_t)e[q] & 0x7FFFFFFFu);
                    ++pos;
                }
        } else if (overflow || (xw == 0 && s_late)) {
            // the last 10 bits of the bin's keys over this workgroup's share
            // (the whole row when it counts alone), into LDS
            const bool alone = !overflow;   // (the late case: workgroup 0 only)
            int64_t share = ((int64_t)b + nfb - 1) / nfb;
            share = (share + kFbStep - 1) / kFbStep * kFbStep;
            const int64_t s0 = alone ? 0 : min((int64_t)xw * share, (int64_t)b);
            const int64_t s1 = alone ? (int64_t)b : min(s0 + share, (int64_t)b);
            uint32_t *h10 = (uint32_t *)ent;
            for (int i = t; i < kFbBins; i += kSelThreads) h10[i] = 0;
            __syncthreads();
            fallback_count(a.scores + (int64_t)r * a.sstride, s0, s1, T22, h10);
            __syncthreads();
            if (!alone && nfb > 1) {   // into the row's counters (device-scope atomics)
                uint32_t *g10 = (uint32_t *)(a.ws + a.L.fb_hist) + (int64_t)r * kFbBins;
                for (int i = t; i < kFbBins; i += kSelThreads)
                    if (h10[i]) __hip_atomic_fetch_add(&g10[i], h10[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (alone) {
                if (t < 64) wave_find_bin<kFbBins / 64>(h10, need2, lane, &sB10, &sAbove10);
                __syncthreads();
                fallback_output(a.scores + (int64_t)r * a.sstride, b, (T22 << kFbBits) | (uint32_t)sB10,
                                need2 - sAbove10, out_row, k, wsum2);
            }
        }
    }
    // ---- every workgroup of the row arrives; the last one finishes the
    // heavy-tie case and clears the row's counters.  No fence: the counts go
    // in with device-scope atomics, each thread waits until its own are
    // performed, and the ticket is a device-scope atomic taken after that;
    // the last workgroup reads the counts with device-scope atomic loads.  (A
    // device-scope fence here would write back this XCD's L2.)
    if (nfb > 1) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (t == 0)
            s_ticket = __hip_atomic_fetch_add((uint32_t *)(a.ws + a.L.fb_cnt) + r, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (s_ticket != (uint32_t)nfb - 1) return;
    }
    if (b > k && overflow) {
        uint32_t *h10 = (uint32_t *)ent;
        if (nfb > 1) {
            uint32_t *g10 = (uint32_t *)(a.ws + a.L.fb_hist) + (int64_t)r * kFbBins;
            for (int i = t; i < kFbBins; i += kSelThreads) {
                h10[i] = __hip_atomic_load(&g10[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                g10[i] = 0;
            }
        }
        __syncthreads();
        if (t < 64) wave_find_bin<kFbBins / 64>(h10, need2, lane, &sB10, &sAbove10);
        __syncthreads();
        fallback_output(a.scores + (int64_t)r * a.sstride, b, (T22 << kFbBits) | (uint32_t)sB10,
                        need2 - sAbove10, out_row, k, wsum2);
    }
    if (t < kHist1Slots * kBins1) ((uint32_t *)(a.ws + a.L.hist1))[(int64_t)r * kHist1Slots * kBins1 + t] = 0;
    for (int i = t; i < kHist2Slots * kBins2; i += kSelThreads)
        ((uint32_t *)(a.ws + a.L.hist2))[(int64_t)r * kHist2Slots * kBins2 + i] = 0;
    if (t < kBins3) hist3[t] = 0;
    if (t == 0 && nfb > 1) ((uint32_t *)(a.ws + a.L.fb_cnt))[r] = 0;
}

__global__ __launch_bounds__(kSelThreads) void hist1_kernel(SelectArgs a) { hist1_body(a, blockIdx.x, blockIdx.y); }
__global__ __launch_bounds__(kSelThreads) void refine_kernel(SelectArgs a) { refine_body(a, blockIdx.x, blockIdx.y); }
__global__ __launch_bounds__(kSelThreads) void gather_kernel(SelectArgs a) { gather_body(a, blockIdx.x, blockIdx.y); }
__global__ __launch_bounds__(kSelThreads) void finalize_kernel(SelectArgs a) {
    finalize_body(a, blockIdx.x, blockIdx.y);
}

// ---------------------------------------------------------------------------
// Rows of at most kSmallMax keys (select_small_kernel): one workgroup per row
// reads the row's scores once into registers as radix keys (thread t holds
// keys t + 1024 j, at most 16), finds the k-th largest key T digit by digit
// in LDS histograms, and writes, in ascending index order, every key above T
// and the first `need` keys equal to T (exact for any ties; no fallback).
// Digits: the first (bits 31..26) as everywhere else, from the scoring pass's
// counts in the workspace (the kernel clears them) or counted here; then bits
// 25..17, 16..8 and 7..0 (512, 512 and 256 bins) in eight LDS histogram
// copies (wave % 8), double-buffered so that one is cleared while the other
// counts.  Once at most 64 keys share the 15-bit prefix (after the first of
// those passes, for all but heavily tied rows) they are ranked directly and
// the last two passes are skipped.  LDS adds are one per counted key and
// lane; a wave whose keys share one digit (heavy ties) folds them into one
// add.  Wave scans use DPP row
// shifts (a shuffle goes through the LDS crossbar at LDS latency per step).
// Output: per 1024-key slice, each wave's counts of keys above and equal to T
// (ballots), one scan of those counts in index order, then every lane writes
// its selected key at (keys above before it) + min(keys equal before it, need).
constexpr int kSmallWaves = kSelThreads / 64;
constexpr int kSmallSlots = kSmallMax / kSelThreads;   // keys per thread
constexpr int kSmallBins = 512;
constexpr int kSmallCopies = 8;   // histogram copies (wave % 8)
constexpr int kSmallRank = 64;    // a bin of at most this many keys is ranked directly
static_assert(kSmallRank % kSmallWaves == 0 && kSmallRank <= 64, "direct rank: whole comparisons per thread, one candidate per lane");
static_assert(kSmallSlots * kSmallWaves <= 64 * 8, "the output scan covers 8 counts per lane");

// Digit counts of up to four distinct digits folded per wave (the first
// digit: a row's keys share few of them, and same-address LDS atomics of one
// instruction serialize); the remaining lanes add one by one.
__device__ __forceinline__ void small_count_folded(uint32_t *h, uint32_t d, bool valid, int lane) {
    uint64_t todo = __ballot(valid);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        if (!todo) break;
        const int leader = __ffsll((unsigned long long)todo) - 1;
        const uint32_t dl = __builtin_amdgcn_readlane(d, leader);
        const uint64_t m = __ballot(valid & (d == dl)) & todo;
        if (lane == leader) atomicAdd(h + dl, (uint32_t)__popcll(m));
        todo &= ~m;
    }
    if ((todo >> lane) & 1) atomicAdd(h + d, 1u);
}

// Digit counts: one add when every counted lane of the wave has the same
// digit, else one per lane.
__device__ __forceinline__ void small_count(uint32_t *h, uint32_t d, bool valid, int lane) {
    const uint64_t act = __ballot(valid);
    if (!act) return;
    const int first = __ffsll((unsigned long long)act) - 1;
    const uint32_t d0 = __builtin_amdgcn_readlane(d, first);
    if (__ballot(valid & (d == d0)) == act) {
        if (lane == first) atomicAdd(h + d0, (uint32_t)__popcll(act));
    } else if (valid) {
        atomicAdd(h + d, 1u);
    }
}

template <bool kHist1>
__global__ __launch_bounds__(kSelThreads) void select_small_kernel(SelectArgs a) {
    __shared__ uint32_t shist2[2][kSmallCopies][kSmallBins];   // double-buffered: one is cleared while the other counts
    __shared__ uint32_t stot[kSmallBins];
    __shared__ uint32_t scnt[kSmallSlots * kSmallWaves];   // [slice][wave]: above << 16 | equal, then their prefix
    __shared__ int s_bin;
    __shared__ uint32_t s_above;
    __shared__ uint32_t s_rk[kSmallRank];   // the keys of a small bin and their indices
    __shared__ int s_ri[kSmallRank];
    __shared__ uint32_t s_rank[kSmallRank];
    __shared__ uint32_t s_nr, s_T, s_need;
    const int r = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int k = a.topk;
    int32_t *out = a.out_idx + (int64_t)r * k;
    uint32_t *h1 = (uint32_t *)(a.ws + a.L.hist1) + (int64_t)r * kHist1Slots * kBins1;
    const int b = clamp_bound(a.row_bound[r], a.max_bound);
    if (b <= k) {   // every key of the row is selected (uniform exit)
        for (int j = t; j < k; j += kSelThreads) out[j] = j < b ? j : -1;
        if (!kHist1 && t < kHist1Slots * kBins1) h1[t] = 0;
        return;
    }
    // ---- the scoring pass's first-digit counts, then the row's keys into
    // registers (every load issued before any use)
    uint32_t c1[kHist1Slots] = {};
    if (!kHist1 && wave == 0) hist1_load(a, r, lane, c1);
    const int J = (b + kSelThreads - 1) / kSelThreads;   // slices, 2 .. kSmallSlots
    const float *sc = a.scores + (int64_t)r * a.sstride;
    // (lanes past the bound re-read the last key: no per-lane branch, and
    // validity below comes from the one partial slice)
    float v[kSmallSlots];
#pragma unroll
    for (int j = 0; j < kSmallSlots; ++j) {
        v[j] = 0.0f;
        if (j < J) v[j] = sc[min(j * kSelThreads + t, b - 1)];
    }
    uint32_t key[kSmallSlots];
#pragma unroll
    for (int j = 0; j < kSmallSlots; ++j) key[j] = radix_key(v[j]);
    const int tail = b - (J - 1) * kSelThreads;   // keys in the last slice, 1 .. 1024
    auto valid = [&](int j) { return (j < J - 1) | (t < tail); };

    // ---- first digit: the k-th largest key's bin and the keys above it
    uint32_t need = (uint32_t)k;
    if (t == 0) s_nr = 0;
    if (t < kSmallRank) s_rank[t] = 0;
    for (int j = t; j < kSmallCopies * kSmallBins; j += kSelThreads) (&shist2[0][0][0])[j] = 0;
    if (kHist1) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kSmallSlots; ++j)
            if (j < J) small_count_folded(shist2[0][wave & (kSmallCopies - 1)], key[j] >> kDigit1Shift, valid(j), lane);
        __syncthreads();
        if (t < kBins1) {
            uint32_t c = 0;
#pragma unroll
            for (int w = 0; w < kSmallCopies; ++w) c += shist2[0][w][t];
            stot[t] = c;
        }
        for (int j = t; j < kSmallCopies * kSmallBins; j += kSelThreads) (&shist2[0][0][0])[j] = 0;
    } else if (t < kBins1) {
        stot[t] = hist1_sum(c1);
    }
    __syncthreads();
    if (!kHist1 && t < kHist1Slots * kBins1) h1[t] = 0;   // (read above; the workspace is left clean)
    if (wave == 0) wave_find_bin<1>(stot, need, lane, &s_bin, &s_above);
    __syncthreads();
    uint32_t prefix = (uint32_t)s_bin << kDigit1Shift;
    uint32_t pmask = (uint32_t)(kBins1 - 1) << kDigit1Shift;
    need -= s_above;

    // ---- the other 26 bits: 9 + 9 + 8 (buffer 0 was cleared above; each
    // pass clears the other buffer for the next while it sums its own)
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
        const int sh = pass == 0 ? 17 : (pass == 1 ? 8 : 0);
        const uint32_t nb = pass == 2 ? 256u : 512u;
        uint32_t(*shist)[kSmallBins] = shist2[pass & 1];
        // A wave whose first slot counts a single digit (heavy ties: then
        // likely every slot does) folds its adds; other waves add per lane.
        uint32_t *hw = shist[wave & (kSmallCopies - 1)];
        const uint32_t d0 = (key[0] >> sh) & (nb - 1);
        const bool m0 = valid(0) & ((key[0] & pmask) == prefix);
        const uint64_t act0 = __ballot(m0);
        bool fold = false;
        if (act0) {
            const uint32_t dl = __builtin_amdgcn_readlane(d0, __ffsll((unsigned long long)act0) - 1);
            fold = __ballot(m0 & (d0 != dl)) == 0;
        }
        if (fold) {
#pragma unroll
            for (int j = 0; j < kSmallSlots; ++j)
                if (j < J) small_count(hw, (key[j] >> sh) & (nb - 1), valid(j) & ((key[j] & pmask) == prefix), lane);
        } else {
#pragma unroll
            for (int j = 0; j < kSmallSlots; ++j)
                if (j < J && (valid(j) & ((key[j] & pmask) == prefix))) atomicAdd(hw + ((key[j] >> sh) & (nb - 1)), 1u);
        }
        __syncthreads();
        if (t < (int)nb) {
            uint32_t c = 0;
#pragma unroll
            for (int w = 0; w < kSmallCopies; ++w) c += shist[w][t];
            stot[t] = c;
        }
        if (pass < 2)
            for (int j = t; j < kSmallCopies * kSmallBins; j += kSelThreads) (&shist2[(pass + 1) & 1][0][0])[j] = 0;
        __syncthreads();
        if (wave == 0) {
            if (pass < 2) wave_find_bin<kSmallBins / 64>(stot, need, lane, &s_bin, &s_above);
            else wave_find_bin<4>(stot, need, lane, &s_bin, &s_above);
        }
        __syncthreads();
        prefix |= (uint32_t)s_bin << sh;
        pmask |= (nb - 1) << sh;
        need -= s_above;
        if (pass == 0 && stot[s_bin] <= (uint32_t)kSmallRank) {
            // few keys share the prefix (the usual case after 15 bits): they
            // are ranked directly, (key desc, index asc), and the need-th is
            // T; the digit passes that remain are skipped.  Thread t compares
            // candidate t % 64 with candidates 4 (t / 64) .. 4 (t / 64) + 3.
            const uint32_t nbin = stot[s_bin];
#pragma unroll
            for (int j = 0; j < kSmallSlots; ++j)
                if (j < J && (valid(j) & ((key[j] & pmask) == prefix))) {
                    const uint32_t slot = atomicAdd(&s_nr, 1u);
                    if (slot < (uint32_t)kSmallRank) {
                        s_rk[slot] = key[j];
                        s_ri[slot] = j * kSelThreads + t;
                    }
                }
            __syncthreads();
            const uint32_t ci = (uint32_t)lane;
            if (ci < nbin) {
                const uint32_t kl = s_rk[ci];
                const int il = s_ri[ci];
                uint32_t c = 0;
#pragma unroll
                for (int q = 0; q < kSmallRank / kSmallWaves; ++q) {
                    const uint32_t f = (uint32_t)(wave * (kSmallRank / kSmallWaves) + q);
                    if (f < nbin) {
                        const uint32_t kf = s_rk[f];
                        const int jf = s_ri[f];
                        c += (kf > kl) || (kf == kl && jf < il);
                    }
                }
                if (c) atomicAdd(&s_rank[ci], c);
            }
            __syncthreads();
            if (wave == 0) {
                const bool mine = (uint32_t)lane < nbin;
                const uint32_t kl = mine ? s_rk[lane] : 0u;
                const uint64_t at = __ballot(mine && s_rank[lane] == need - 1);   // exactly one lane
                const uint32_t T = (uint32_t)__builtin_amdgcn_readlane((int)kl, __ffsll((unsigned long long)at) - 1);
                const uint32_t above = (uint32_t)__popcll(__ballot(mine && kl > T));
                if (lane == 0) { s_T = T; s_need = need - above; }
            }
            __syncthreads();
            prefix = s_T;
            need = s_need;
            break;
        }
    }

    // ---- output in index order (key index = slice * 1024 + wave * 64 + lane)
    const uint32_t T = prefix;
#pragma unroll
    for (int j = 0; j < kSmallSlots; ++j)
        if (j < J) {
            const bool ok = valid(j);
            const uint32_t na = (uint32_t)__popcll(__ballot(ok & (key[j] > T)));
            const uint32_t ne = (uint32_t)__popcll(__ballot(ok & (key[j] == T)));
            if (lane == 0) scnt[j * kSmallWaves + wave] = na << 16 | ne;
        }
    __syncthreads();
    if (wave == 0) {   // exclusive prefix of the J * 16 counts (8 per lane); each total is < 2^16
        const int n = J * kSmallWaves;
        uint32_t c[8], sum = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            c[e] = 8 * lane + e < n ? scnt[8 * lane + e] : 0u;
            sum += c[e];
        }
        uint32_t run = wave_incl_scan(sum, lane) - sum;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (8 * lane + e < n) scnt[8 * lane + e] = run;
            run += c[e];
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kSmallSlots; ++j)
        if (j < J) {
            const bool ok = valid(j);
            const bool above = ok & (key[j] > T), equal = ok & (key[j] == T);
            const uint64_t ma = __ballot(above), me = __ballot(equal);
            const uint32_t base = scnt[j * kSmallWaves + wave];
            const uint32_t pa = (base >> 16) + lane_prefix(ma), pe = (base & 0xffffu) + lane_prefix(me);
            const int i = j * kSelThreads + t;
            if (above) out[pa + min(pe, need)] = i;
            if (equal & (pe < need)) out[pa + pe] = i;
        }
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
    hipLaunchKernelGGL(finalize_kernel, dim3(a.L.fb_wgs, a.rows), dim3(kSelThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_select_small(const SelectArgs &a, bool with_hist1, hipStream_t st) {
    if (a.max_bound > kSmallMax) return hipErrorInvalidValue;
    if (with_hist1)
        hipLaunchKernelGGL(select_small_kernel<true>, dim3(a.rows), dim3(kSelThreads), 0, st, a);
    else
        hipLaunchKernelGGL(select_small_kernel<false>, dim3(a.rows), dim3(kSelThreads), 0, st, a);
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
