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

constexpr int kPrefetch = 8;   // 16-key groups in flight per wave (a multiple of 4)

__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
    bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
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

struct KeyGroup {
    u32x4_t lo, hi;   // 32 code bytes of key lane%16
    float scale;
    int ok;           // wave-uniform: the page id was in range
};

template <bool kHist>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreArgs a) {
    __shared__ uint32_t lds_hist[kGroupRows][kBins1];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r0 = blockIdx.y;

    // ---- row grouping: rows sharing a page-table row, in runs of up to 4
    const int pr0 = a.row_pt[r0];
    int rs = 0;
    for (int base = r0; base > 0; base -= 64) {
        int idx = base - 1 - lane;
        bool diff = idx < 0 || a.row_pt[idx < 0 ? 0 : idx] != pr0;
        uint64_t m = __ballot(diff);
        if (m) { rs = base - (__ffsll((unsigned long long)m) - 1); break; }
    }
    if ((r0 - rs) % kGroupRows != 0) return;
    int rg;
    {
        bool same = lane < kGroupRows && r0 + lane < a.rows && a.row_pt[r0 + (lane < kGroupRows ? lane : 0)] == pr0;
        uint64_t m = __ballot(same);
        rg = __ffsll((unsigned long long)~m) - 1;
    }
    int gmax = 0;
    for (int j = 0; j < rg; ++j) {
        int bj = a.row_bound[r0 + j];
        bj = bj < 0 ? 0 : (bj > a.max_bound ? a.max_bound : bj);
        gmax = bj > gmax ? bj : gmax;
    }
    gmax = __builtin_amdgcn_readfirstlane(gmax);
    const int c0 = blockIdx.x * a.chunk;
    if (c0 >= gmax) return;
    const int c1 = min(c0 + a.chunk, gmax);

    if (kHist) {
        lds_hist[threadIdx.x >> 6][lane] = 0;
        __syncthreads();
    }

    // ---- this wave's row and 16-key groups
    const int wpr = kGroupRows / rg;                 // waves per row
    const bool active = wave < rg * wpr;
    const int slot = wave % rg;
    const int myrow = r0 + slot;
    const int wsub = wave / rg;
    int b = __builtin_amdgcn_readfirstlane(a.row_bound[myrow]);
    b = b < 0 ? 0 : (b > a.max_bound ? a.max_bound : b);
    const int myend = min(c1, b);
    const int g_first = c0 / kKeysPerMfma + wsub;
    const int g_end = (myend + kKeysPerMfma - 1) / kKeysPerMfma;
    const int n_my = (active && g_first < g_end) ? (g_end - g_first + wpr - 1) / wpr : 0;
    const int prow = a.row_pt[myrow];
    const bool pt_ok = prow >= 0 && prow < a.pt_rows;
    const int32_t *pt = a.page_table + (int64_t)(pt_ok ? prow : 0) * a.pt_stride;

    const int key_in_group = lane & 15;
    const int lane_row = lane >> 4;
    const int64_t lane_byte = (int64_t)key_in_group * kDim + lane_row * 32;

    // Loads are unconditional: past the wave's last group they re-read that
    // group (always in range), so no branch separates a load from its use.
    auto load_group = [&](int i, KeyGroup &kg) {
        const int ic = i < n_my ? i : n_my - 1;
        const int g = g_first + ic * wpr;
        int page = pt_ok ? pt[g >> 2] : -1;
        page = __builtin_amdgcn_readfirstlane(page);
        kg.ok = page >= 0 && page < a.num_pages;
        const int64_t key0 = (int64_t)(kg.ok ? page : 0) * kPage + (g & 3) * kKeysPerMfma;
        const uint8_t *kp = a.k8 + key0 * kDim + lane_byte;
        kg.lo = *(const u32x4_t *)(kp);
        kg.hi = *(const u32x4_t *)(kp + 16);
        kg.scale = a.kscale[key0 + key_in_group];
    };

    if (n_my > 0) {
    KeyGroup kb[kPrefetch];
#pragma unroll
    for (int p = 0; p < kPrefetch; ++p) load_group(p, kb[p]);

    // q as the MFMA A operand: head 16*hb + lane%16, dims 32*(lane/16) + 8*ks + [0, 8)
    bf16x8_t qa[4][4];
    f32x4_t wv[4];
    {
        const uint16_t *qrow = a.q + (int64_t)myrow * kHeads * kDim;
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                qa[hb][ks] = *(const bf16x8_t *)(qrow + (16 * hb + key_in_group) * kDim + 32 * lane_row + 8 * ks);
        // weights of the output rows this lane holds: heads 16*hb + 4*(lane/16) + j
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
            wv[hb] = *(const f32x4_t *)(a.w + (int64_t)myrow * kHeads + 16 * hb + 4 * lane_row);
    }

    float *srow = a.scores + (int64_t)myrow * a.sstride;
    float out = 0.0f;
    const int n_iter = (n_my + kPrefetch - 1) / kPrefetch * kPrefetch;
    for (int i0 = 0; i0 < n_iter; i0 += kPrefetch) {
#pragma unroll
        for (int p = 0; p < kPrefetch; ++p) {
            const int i = i0 + p;
            bf16x8_t kv[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const u32x4_t &src = ks < 2 ? kb[p].lo : kb[p].hi;
                kv[ks] = e4m3x8_to_bf16(src[(ks & 1) * 2], src[(ks & 1) * 2 + 1]);
            }
            const float scale = kb[p].ok ? kb[p].scale : __builtin_nanf("");
            load_group(i + kPrefetch, kb[p]);
            f32x4_t acc[4];
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) acc[hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int hb = 0; hb < 4; ++hb)
                    acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[hb][ks], kv[ks], acc[hb], 0, 0, 0);
            float part = 0.0f;
#pragma unroll
            for (int hb = 0; hb < 4; ++hb)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    part = fmaf(wv[hb][j], fmaxf(acc[hb][j], 0.0f), part);
            const float score = lane_sum_64(part) * scale;
            if (lane_row == (p & 3)) out = score;
            if ((p & 3) == 3) {
                // lane row q holds group i - 3 + q; store the four groups at once
                const int iq = i - 3 + lane_row;
                const int s = (g_first + iq * wpr) * kKeysPerMfma + key_in_group;
                if (iq < n_my && s < b) {
                    srow[s] = out;
                    if (kHist) atomicAdd(&lds_hist[slot][radix_key(out) >> kDigit1Shift], 1u);
                }
            }
        }
    }
    }  // n_my > 0

    if (kHist) {
        __syncthreads();
        const int srow_slot = threadIdx.x >> 6;
        if (srow_slot < rg) {
            const uint32_t c = lds_hist[srow_slot][lane];
            if (c) atomicAdd(a.hist1 + (int64_t)(r0 + srow_slot) * kBins1 + lane, c);
        }
    }
}

hipError_t launch_score(const ScoreArgs &a, hipStream_t st) {
    if (a.max_bound <= 0) return hipSuccess;
    const int nchunks = (a.max_bound + a.chunk - 1) / a.chunk;
    dim3 grid(nchunks, a.rows);
    if (a.hist1)
        hipLaunchKernelGGL(score_kernel<true>, grid, dim3(kScoreThreads), 0, st, a);
    else
        hipLaunchKernelGGL(score_kernel<false>, grid, dim3(kScoreThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace fp8idx
