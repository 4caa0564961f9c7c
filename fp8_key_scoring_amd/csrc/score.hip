// Scoring pass of the paged FP8-E4M3 decode indexer (gfx950).
//
// score(r, s) = k_scale(s) * sum_{h<64} w[r][h] * max(q[r][h] . k(s), 0),
// for s below row r's exclusive bound (sglang pull request page
// "sgl-project/sglang#48224", sgl-amd-mono #86 commit body: Motivation for the
// launch; Modifications rows 1-2 for the per-16-key-group addressing from the
// page and first key, the head-half reduction across lane rows, the scale
// loaded with the key group and the mask at the store; row 4 for counting the
// first radix digit of every stored score in the scoring pass).
//
// Design on gfx950 (not the page's: its kernels are prior art here):
//  * A workgroup is 4 waves and takes one group of up to 4 rows that share a
//    page-table row (one request's verify rows) and one chunk of its keys.
//    With 4 rows each wave owns one row and walks every 16-key group of the
//    chunk; the four waves read the same key bytes, so HBM sees each key once
//    and the repeats hit the CU's L1.  With 1 or 2 rows the waves split the
//    chunk's 16-key groups so no key is read twice per row.
//  * Per 16-key group a lane loads 32 contiguous code bytes of key lane%16
//    (two 16-byte loads; the page id comes from a scalar load of the page
//    table, the rest is a fixed per-lane offset) plus that key's scale.  The
//    codes go straight to registers, are widened E4M3 -> bf16 (exact) with the
//    gfx950 packed conversion, and feed the B operand of
//    v_mfma_f32_16x16x32_bf16 (K = the 128 head dims in 4 steps, N = 16
//    keys).  The A operand is q, 16 heads per MFMA, held in registers for the
//    whole chunk (64 VGPRs: 4 head blocks x 4 K steps).  The order in which
//    head dims feed the K index is a free permutation applied to q and k alike.
//    (The fp8 x fp8 MFMA is not used: its internal accumulation is far below
//    fp32 precision, while the bf16 one accumulates in fp32.)
//  * Epilogue: lane l holds heads 16b + 4(l/16) + j of key l%16 for b, j < 4;
//    it sums w * max(d, 0) over its 16 heads, two permlane swaps (32 and 16
//    lanes) finish the sum over the 64 heads, and the key's scale multiplies
//    the total.  Scores of four consecutive groups are gathered in one
//    register (lane row i holds group i) and stored by all 64 lanes at once,
//    masked at the row's bound; the same lanes add the first radix digit of
//    each stored score to a 64-bin LDS histogram per row, which is added to
//    the row's global histogram at the end of the workgroup.
#include "common.h"

namespace fp8idx {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRing = 8;   // 16-key groups loaded ahead per wave (a multiple of 4)

__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
    bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// max(x, 0) in one integer max on the bit pattern: every negative float
// (sign bit set, -0 included) is a negative int32 and becomes +0; values
// >= +0 are unchanged.  (A float max would first be canonicalised by the
// compiler, two instructions per element.)
__device__ __forceinline__ float relu(float x) {
    return __int_as_float(max(__float_as_int(x), 0));
}

__device__ __forceinline__ float lane_sum_64(float v) {
    // after the 32-swap every lane holds v[l%32] + v[l%32 + 32]; after the
    // 16-swap every lane holds the sum of its column over all four lane rows
    int x = __float_as_int(v);
    auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    float s = __int_as_float(p[0]) + __int_as_float(p[1]);
    int y = __float_as_int(s);
    auto q = __builtin_amdgcn_permlane16_swap(y, y, false, false);
    return __int_as_float(q[0]) + __int_as_float(q[1]);
}

// Adds one to bin d of an LDS histogram for every lane with valid set.  Scores
// of one row mostly share a first digit, so per-lane atomics would pile onto
// one LDS address; the two most common bins of the wave are added once each
// (ballot + popcount) and only the remaining lanes add one by one.
__device__ __forceinline__ void count_digit1(uint32_t *hist, uint32_t d, bool valid, int lane) {
    bool pending = valid;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const uint64_t act = __ballot(pending);
        if (act == 0) return;
        const int leader = __ffsll((unsigned long long)act) - 1;
        const uint32_t d0 = __builtin_amdgcn_readlane(d, leader);
        const bool mine = pending && d == d0;
        const uint64_t m = __ballot(mine);
        if (lane == leader) atomicAdd(&hist[d0], (uint32_t)__popcll(m));
        pending = pending && !mine;
    }
    if (pending) atomicAdd(&hist[d], 1u);
}

struct KeyGroup {
    u32x4_t lo, hi;   // 32 code bytes of key lane%16
    float scale;
    int ok;           // wave-uniform: the page id was in range
};

template <bool kHist>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreArgs a) {
    __shared__ uint32_t lds_hist[kGroupRows][kBins1];
    extern __shared__ float lds_sc[];   // [kGroupRows][chunk] this chunk's scores
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r0 = blockIdx.y;

    // ---- row grouping: rows sharing a page-table row, in runs of up to 4.
    // One round of loads: every lane reads one of the 64 rows before r0 (to
    // find where r0's run of equal page-table rows starts), and lanes 0..3
    // read the page-table rows and bounds of r0..r0+3.
    const int back = r0 - 1 - lane;
    const int fwd = r0 + (lane & 3);
    const int v_back = back >= 0 ? a.row_pt[back] : 0;
    const int v_fwd = fwd < a.rows ? a.row_pt[fwd] : 0;
    int v_bnd = fwd < a.rows ? a.row_bound[fwd] : 0;
    v_bnd = v_bnd < 0 ? 0 : (v_bnd > a.max_bound ? a.max_bound : v_bnd);
    const int pr0 = __builtin_amdgcn_readlane(v_fwd, 0);
    int rs;
    {
        const uint64_t m = __ballot(back < 0 || v_back != pr0);
        if (m) {
            rs = r0 - (__ffsll((unsigned long long)m) - 1);
        } else {   // the run is longer than 64 rows: keep walking back
            rs = 0;
            for (int base = r0 - 64; base > 0; base -= 64) {
                const int idx = base - 1 - lane;
                const uint64_t m2 = __ballot(idx < 0 || a.row_pt[idx < 0 ? 0 : idx] != pr0);
                if (m2) { rs = base - (__ffsll((unsigned long long)m2) - 1); break; }
            }
        }
    }
    if ((r0 - rs) % kGroupRows != 0) return;
    const int rg = __ffsll((unsigned long long)~__ballot(lane < kGroupRows && fwd < a.rows && v_fwd == pr0)) - 1;
    int gmax = 0;
    for (int j = 0; j < rg; ++j) gmax = max(gmax, __builtin_amdgcn_readlane(v_bnd, j));
    const int c0 = blockIdx.x * a.chunk;
    if (c0 >= gmax) return;
    const int c1 = min(c0 + a.chunk, gmax);

    // ---- this wave's row and 16-key groups
    const int wpr = kGroupRows / rg;                 // waves per row
    const bool active = wave < rg * wpr;
    const int slot = wave % rg;
    const int myrow = r0 + slot;
    const int wsub = wave / rg;
    const int b = __builtin_amdgcn_readlane(v_bnd, slot);
    const int myend = min(c1, b);
    const int g_first = c0 / kKeysPerMfma + wsub;
    const int g_end = (myend + kKeysPerMfma - 1) / kKeysPerMfma;
    const int n_my = (active && g_first < g_end) ? (g_end - g_first + wpr - 1) / wpr : 0;
    const bool pt_ok = pr0 >= 0 && pr0 < a.pt_rows;
    // the chunk's page ids, one per lane (a chunk spans at most 64 pages);
    // a group picks its page with a lane read, so the loop never waits on a
    // scalar load.  Out-of-range ids become -1 (their keys score NaN).
    int vpage;
    {
        const int npg = (c1 - c0 + kPage - 1) / kPage;
        const int32_t *pt = a.page_table + (int64_t)(pt_ok ? pr0 : 0) * a.pt_stride + c0 / kPage;
        vpage = (pt_ok && lane < npg) ? pt[lane] : -1;
        vpage = (vpage >= 0 && vpage < a.num_pages) ? vpage : -1;
    }

    if (kHist) {
        lds_hist[threadIdx.x >> 6][lane] = 0;
        __syncthreads();
    }

    const int key_in_group = lane & 15;
    const int lane_row = lane >> 4;
    // fixed per-lane byte offsets inside one 16-key group (32 code bytes of
    // key lane%16) and of its scale; the page and group parts are uniform
    const uint32_t lane_koff = (uint32_t)(key_in_group * kDim + lane_row * 32);
    const uint32_t lane_soff = (uint32_t)key_in_group;

    // Loads are unconditional: past the wave's last group they re-read that
    // group (always in range), so no branch separates a load from its use.
    // The group's base addresses are wave-uniform (scalar registers); each
    // lane adds only its fixed 32-bit offset.
    auto load_group = [&](int i, KeyGroup &kg) {
        const int ic = i < n_my ? i : n_my - 1;
        const int g = g_first + ic * wpr;
        const int page = __builtin_amdgcn_readlane(vpage, (g - c0 / kKeysPerMfma) >> 2);
        kg.ok = page >= 0;
        const int64_t key0 = (int64_t)(kg.ok ? page : 0) * kPage + (g & 3) * kKeysPerMfma;
        const uint8_t *kbase = a.k8 + key0 * kDim;         // uniform
        const float *sbase = a.kscale + key0;               // uniform
        kg.lo = *(const u32x4_t *)(kbase + lane_koff);
        kg.hi = *(const u32x4_t *)(kbase + lane_koff + 16);
        kg.scale = sbase[lane_soff];
    };

    if (n_my > 0) {
    // q as the MFMA A operand: head 16*hb + lane%16, dims 32*(lane/16) + 8*ks + [0, 8),
    // and the weights of the output rows this lane holds: heads 16*hb + 4*(lane/16) + j.
    // Issued before the key loads: these do not depend on the page ids.
    bf16x8_t qa[4][4];
    f32x4_t wv[4];
    {
        const uint16_t *qrow = a.q + (int64_t)myrow * kHeads * kDim;
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                qa[hb][ks] = *(const bf16x8_t *)(qrow + (16 * hb + key_in_group) * kDim + 32 * lane_row + 8 * ks);
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
            wv[hb] = *(const f32x4_t *)(a.w + (int64_t)myrow * kHeads + 16 * hb + 4 * lane_row);
    }
    KeyGroup kb[kRing];   // group j lives in slot j % kRing
#pragma unroll
    for (int p = 0; p < kRing; ++p) load_group(p, kb[p]);
    // keep every load above ahead of the first use
    __builtin_amdgcn_sched_barrier(0);

    float out = 0.0f;

    auto convert = [&](const KeyGroup &kg, bf16x8_t (&kv)[4]) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const u32x4_t &src = ks < 2 ? kg.lo : kg.hi;
            kv[ks] = e4m3x8_to_bf16(src[(ks & 1) * 2], src[(ks & 1) * 2 + 1]);
        }
    };
    auto scale_of = [&](const KeyGroup &kg) { return kg.ok ? kg.scale : __builtin_nanf(""); };
    auto mfma_group = [&](const bf16x8_t (&kv)[4], f32x4_t (&acc)[4]) {
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) acc[hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int hb = 0; hb < 4; ++hb)
                acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[hb][ks], kv[ks], acc[hb], 0, 0, 0);
    };

    // Three-stage software pipeline per wave: in the step for group i the
    // MFMAs of group i+1, the epilogue of group i and the conversion of group
    // i+2 are independent, and the scheduler interleaves them (one MFMA, then
    // up to four VALU ops), so the conversion and epilogue run in the MFMA
    // shadow instead of after it.
    bf16x8_t kv[2][4];    // group j's converted keys in kv[j & 1]
    f32x4_t acc[2][4];    // group j's MFMA results in acc[j & 1]
    float sc0, sc1, sc2;  // scales of groups i, i+1, i+2
    convert(kb[0], kv[0]);
    sc0 = scale_of(kb[0]);
    load_group(kRing, kb[0]);
    mfma_group(kv[0], acc[0]);
    convert(kb[1], kv[1]);
    sc1 = scale_of(kb[1]);
    load_group(kRing + 1, kb[1]);

    const int n_iter = (n_my + kRing - 1) / kRing * kRing;
    for (int i0 = 0; i0 < n_iter; i0 += kRing) {
#pragma unroll
        for (int p = 0; p < kRing; ++p) {
            const int i = i0 + p;   // p and i have the same parity (kRing is even)
            mfma_group(kv[(p + 1) & 1], acc[(p + 1) & 1]);
            float part = 0.0f;
#pragma unroll
            for (int hb = 0; hb < 4; ++hb)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    part = fmaf(wv[hb][j], relu(acc[p & 1][hb][j]), part);
            const float score = lane_sum_64(part) * sc0;
            if (lane_row == (p & 3)) out = score;
            KeyGroup &nx = kb[(p + 2) % kRing];
            convert(nx, kv[p & 1]);
            sc2 = scale_of(nx);
            load_group(i + 2 + kRing, nx);
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // then four VALU
            }
            if ((p & 3) == 3) {
                // lane row q holds group i - 3 + q; stage the four groups in
                // LDS (a global store here would make every later load wait
                // drain the whole prefetch ring: loads and stores share one
                // counter and may complete out of order)
                const int iq = i - 3 + lane_row;
                const int s = (g_first + iq * wpr) * kKeysPerMfma + key_in_group;
                if (iq < n_my && s < b) lds_sc[slot * a.chunk + (s - c0)] = out;
            }
            sc0 = sc1;
            sc1 = sc2;
        }
    }
    }  // n_my > 0

    // ---- write the chunk's scores (coalesced) and count their first digit
    __syncthreads();
    for (int r = 0; r < rg; ++r) {
        const int n = min(c1, __builtin_amdgcn_readlane(v_bnd, r)) - c0;
        float *dst = a.scores + (int64_t)(r0 + r) * a.sstride + c0;
        const float *src = lds_sc + r * a.chunk;
        for (int j0 = 0; j0 < n; j0 += kScoreThreads) {
            const int j = j0 + (int)threadIdx.x;
            const bool v = j < n;
            const float x = v ? src[j] : 0.0f;
            if (v) dst[j] = x;
            if (kHist) count_digit1(lds_hist[r], radix_key(x) >> kDigit1Shift, v, lane);
        }
    }
    if (kHist) {
        __syncthreads();
        const int hr = threadIdx.x >> 6;
        if (hr < rg) {
            const uint32_t c = lds_hist[hr][lane];
            if (c) atomicAdd(a.hist1 + (int64_t)(r0 + hr) * kBins1 + lane, c);
        }
    }
}

hipError_t launch_score(const ScoreArgs &a, hipStream_t st) {
    if (a.max_bound <= 0) return hipSuccess;
    const int nchunks = (a.max_bound + a.chunk - 1) / a.chunk;
    dim3 grid(nchunks, a.rows);
    const size_t lds = (size_t)kGroupRows * a.chunk * sizeof(float);
    if (a.hist1)
        hipLaunchKernelGGL(score_kernel<true>, grid, dim3(kScoreThreads), lds, st, a);
    else
        hipLaunchKernelGGL(score_kernel<false>, grid, dim3(kScoreThreads), lds, st, a);
    return hipGetLastError();
}

}  // namespace fp8idx
