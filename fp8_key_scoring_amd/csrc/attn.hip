// Sparse attention over each row's selected keys (gfx950): the step the
// indexer feeds (sglang pull request page "sgl-project/sglang#48224", the
// sgl-amd-mono #86 commit body, Motivation: each row's exact top-2048 keys
// are picked for the attention that follows; the GLM-5.2 release test-suite
// page runs that step with an MLA sparse-attention backend over a
// DeepSeek-style latent cache).  The pages give neither formula nor shapes;
// the reading (absorbed multi-head latent attention, decode) is:
//
//   every key position s holds a latent vector c_s of 576 bf16 values (512
//   latent + 64 rotary) in a paged cache with the index keys' page table;
//   row r has 16 query heads q_h of 576 bf16 values;
//   over the row's selected positions J (its index list; -1 entries, and
//   positions outside [0, max_bound) or on a page id out of range, skipped):
//     l_j   = sm_scale * q_h . c_j
//     out_h = sum_j exp(l_j) c_j[0..512) / sum_j exp(l_j),  lse_h = log sum_j exp(l_j)
//   (no selected position: out_h = 0, lse_h = -inf).
//
// Design on gfx950 (split over the selected keys, "flash decoding"):
//  * attn_kernel: workgroup (split x, row r) of 4 waves takes the row's index
//    list entries [x*span, (x+1)*span).  It first resolves those entries to
//    cache rows (page table lookups, -1 for a skipped entry) into an LDS
//    table, then streams them in chunks of 64 keys.  A chunk's 64 cache rows
//    (1,152 B each) go straight from HBM to LDS with global_load_lds_dwordx4
//    (16 bytes per lane, no registers): one instruction moves 8 keys x 128 B,
//    eight lanes per key reading one whole 128-byte line, into a 1 KiB block;
//    block (key group G, piece group P) holds pieces 8P..8P+7 (piece p = dims
//    8p..8p+7) of keys 8G..8G+7, key kk's piece p in slot (p - kk) mod 8 so
//    that the operand reads below spread over the banks.  Chunks are
//    double-buffered: chunk c+1 is in flight while chunk c is computed.
//  * S = Q K^T on v_mfma_f32_16x16x32_bf16: M = the 16 heads, N = 16 keys
//    (wave w takes keys 16w..16w+15 of the chunk), K = 576 dims in 18 steps;
//    q sits in registers as the A operand for the whole split.
//  * Online softmax over the chunks: the chunk's per-head maximum and sum
//    across the four waves through LDS; the running output is rescaled by
//    exp(m_old - m_new).
//  * O += P V on the same MFMA: M = heads, N = 16 dims (wave w takes dims
//    128w..128w+127), K = 32 keys.  The B operand (8 consecutive keys of one
//    dim) comes from the key-major tile through ds_read_b64_tr_b16, which
//    hands lane i of a 16-lane group dim i of the 4 keys the group points at;
//    two such reads give the 8 keys.  P (fp32) is split into bf16 hi + lo and
//    both are accumulated, so the weights keep ~16 significant bits.
//  * With one split per row the kernel normalises and writes out and lse
//    itself.  Otherwise each split's unnormalised output, maximum and sum go
//    to the workspace and combine_kernel merges them (a workgroup per 256
//    outputs of a row): M = max_x m_x, w_x = exp(m_x - M),
//    out = sum w_x o_x / sum w_x l_x, lse = M + log sum w_x l_x.
#include "common.h"

namespace fp8idx {

namespace {

typedef __bf16 abf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 abf16x4_t __attribute__((ext_vector_type(4)));
typedef float af32x4_t __attribute__((ext_vector_type(4)));
#define AS_GLOBAL(p) ((const void __attribute__((address_space(1))) *)(p))
#define AS_LDS(p) ((void __attribute__((address_space(3))) *)(p))

constexpr int kAH = kAttnHeads;      // 16 query heads
constexpr int kAD = kAttnDim;        // 576 latent + rotary dims
constexpr int kAV = kAttnVDim;       // 512 value dims
constexpr int kChunk = 64;           // keys per chunk
constexpr int kKs = kAD / 32;        // 18 K steps of Q K^T
constexpr int kPieces = kAD / 8;     // 72 16-byte pieces per cache row
constexpr int kPGroups = kPieces / 8;     // 9 groups of 8 pieces (128 B of a row)
constexpr int kKGroups = kChunk / 8;      // 8 groups of 8 keys
// block (G, P) sits at (P * 8 + G) * kBlk: 1 KiB + 16 B, so the blocks of
// neighbouring key groups start on different banks
constexpr int kBlk = 1024 + 16;
constexpr int kBuf = kPGroups * kKGroups * kBlk;      // 74,880 B per chunk buffer
constexpr int kMaxSpan = 2048;                        // entries one split takes at most
constexpr int kLdsTab = kMaxSpan * 4;                 // 8,192 B
constexpr int kPStride = kChunk + 8;                  // P row stride, elements
constexpr int kLdsP = 2 * kAH * kPStride * 2;         // hi and lo, 4,608 B
constexpr int kLdsRed = 2 * 4 * kAH * 4;              // per-wave head maxima and sums
constexpr int kLdsAttn = 2 * kBuf + kLdsTab + kLdsP + kLdsRed;
static_assert(kLdsAttn <= 160 * 1024, "attention tile fits the LDS");
static_assert(kBlk % 16 == 0 && (kPStride * 2) % 16 == 0 && kBuf % 16 == 0, "16-byte operand reads");
static_assert(kMaxSpan % 256 == 0, "table fill: whole rounds of 256 entries");

__device__ __forceinline__ float shfl_xor16_max(float v) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float shfl_xor16_sum(float v) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
    return v;
}

// Workgroup barriers inside the chunk loop.  __syncthreads() is a release
// fence as well, which waits for every outstanding memory operation of the
// wave, the next chunk's global_load_lds included; these wait only for what
// the barrier guards.
//  lds_barrier:   this wave's LDS reads and writes are done (lgkmcnt)
//  chunk_barrier: as lds_barrier, and this wave's share of the current chunk
//                 has landed in LDS (vmcnt: the only loads in flight then)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void chunk_barrier() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    unsigned char *kbuf = lds;                                      // 2 x [72 blocks][kBlk B]
    int32_t *tab = (int32_t *)(lds + 2 * kBuf);                     // [span] cache row, -1: none
    __bf16 *ph = (__bf16 *)(lds + 2 * kBuf + kLdsTab);              // [16 heads][kPStride]  P hi
    __bf16 *pl = ph + kAH * kPStride;                               // P lo
    float *red_max = (float *)(lds + 2 * kBuf + kLdsTab + kLdsP);   // [4 waves][16 heads]
    float *red_sum = red_max + 4 * kAH;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int x = blockIdx.x, r = blockIdx.y;
    const int l16 = lane & 15, lg = lane >> 4;
    const int64_t j0 = (int64_t)x * a.span;
    const int n = (int)max((int64_t)0, min((int64_t)a.span, (int64_t)a.topk - j0));   // entries of the split
    const int nch = (n + kChunk - 1) / kChunk;

    // ---- resolve the split's entries to cache rows (independent loads, then lookups)
    {
        const int prow = a.row_pt[r];
        const bool prow_ok = prow >= 0 && prow < a.pt_rows;
        const int32_t *pt = a.page_table + (int64_t)(prow_ok ? prow : 0) * a.pt_stride;
        const int32_t *sl = a.sel + (int64_t)r * a.topk + j0;
        int sv[kMaxSpan / 256];
#pragma unroll
        for (int u = 0; u < kMaxSpan / 256; ++u) {
            const int i = t + 256 * u;
            sv[u] = (i < n && prow_ok) ? sl[i] : -1;
        }
#pragma unroll
        for (int u = 0; u < kMaxSpan / 256; ++u) {
            const int i = t + 256 * u;
            const int s = sv[u];
            int row = -1;
            if (s >= 0 && s < a.max_bound && s / kPage < a.pt_stride) {
                const int page = pt[s / kPage];
                if (page >= 0 && page < a.num_pages) row = page * kPage + s % kPage;
            }
            if (i < nch * kChunk) tab[i] = row;
        }
    }
    // q of the row in A-operand order: head l16, dims 32ks + 8lg .. +8
    abf16x8_t qa[kKs];
    {
        const uint16_t *q = a.q + ((int64_t)r * kAH + l16) * kAD + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) qa[ks] = *(const abf16x8_t *)(q + 32 * ks);
    }
    __syncthreads();   // the table is complete

    // chunk c into buffer b: wave w loads key groups 2w and 2w+1, all nine
    // piece groups; lane (kk = lane/8, j = lane%8) loads piece (j + kk) mod 8
    // of each group of key 8G + kk into slot j
    auto issue = [&](int c, int b) {
        const int kk = lane >> 3, pj = ((lane & 7) + kk) & 7;
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
            const int G = 2 * wave + gi;
            const int row = tab[c * kChunk + 8 * G + kk];
            const uint16_t *src = a.kv + (int64_t)(row < 0 ? 0 : row) * kAD + 8 * pj;
            unsigned char *dst = kbuf + b * kBuf + G * kBlk;
#pragma unroll
            for (int P = 0; P < kPGroups; ++P)
                __builtin_amdgcn_global_load_lds(AS_GLOBAL(src + 64 * P), AS_LDS(dst + P * kKGroups * kBlk), 16, 0, 0);
        }
    };

    float m_run[4], l_run[4];   // this lane's heads 4lg + jj
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) { m_run[jj] = -INFINITY; l_run[jj] = 0.0f; }
    af32x4_t o[8];              // dims 128w + 16nt + l16, heads 4lg + jj
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[nt] = af32x4_t{0.f, 0.f, 0.f, 0.f};

    if (nch > 0) issue(0, 0);
    for (int c = 0; c < nch; ++c) {
        const int b = c & 1;
        const unsigned char *cb = kbuf + b * kBuf;
        chunk_barrier();   // chunk c complete; every wave is done with chunk c-1's buffer
        if (c + 1 < nch) issue(c + 1, b ^ 1);
        // ---- S = Q K^T for keys 16w .. 16w+15
        af32x4_t sacc = af32x4_t{0.f, 0.f, 0.f, 0.f};
        // lane (lg, l16): key 16w + l16 (group 2w + l16/8, kk = l16 % 8),
        // piece 4ks + lg (group ks/2, 4 (ks % 2) + lg within it)
        const int skk = l16 & 7;
        const unsigned char *kb = cb + (2 * wave + (l16 >> 3)) * kBlk + skk * 128;
        const int so0 = ((lg - skk) & 7) * 16, so1 = ((4 + lg - skk) & 7) * 16;
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks)
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                qa[ks], *(const abf16x8_t *)(kb + (ks >> 1) * kKGroups * kBlk + ((ks & 1) ? so1 : so0)), sacc, 0, 0, 0);
        const bool kok = tab[c * kChunk + 16 * wave + l16] >= 0;   // this lane's key (column l16)
        float sv[4], cmax[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            sv[jj] = kok ? sacc[jj] * a.sm_scale : -INFINITY;
            cmax[jj] = shfl_xor16_max(sv[jj]);
        }
        if (l16 == 0)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) red_max[wave * kAH + 4 * lg + jj] = cmax[jj];
        lds_barrier();
        float alpha[4], p[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int h = 4 * lg + jj;
            const float cm = fmaxf(fmaxf(red_max[h], red_max[kAH + h]), fmaxf(red_max[2 * kAH + h], red_max[3 * kAH + h]));
            const float m_new = fmaxf(m_run[jj], cm);
            // (a head with nothing selected so far keeps -inf and weight 0)
            alpha[jj] = m_new == -INFINITY ? 1.0f : expf(m_run[jj] - m_new);
            p[jj] = sv[jj] == -INFINITY ? 0.0f : expf(sv[jj] - m_new);
            m_run[jj] = m_new;
            const float csum = shfl_xor16_sum(p[jj]);
            if (l16 == 0) red_sum[wave * kAH + h] = csum;
        }
        // P to LDS as bf16 hi + lo: head 4lg + jj, key 16w + l16
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const __bf16 hi = (__bf16)p[jj];
            const __bf16 lo = (__bf16)(p[jj] - (float)hi);
            ph[(4 * lg + jj) * kPStride + 16 * wave + l16] = hi;
            pl[(4 * lg + jj) * kPStride + 16 * wave + l16] = lo;
        }
        lds_barrier();
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int h = 4 * lg + jj;
            l_run[jj] = l_run[jj] * alpha[jj] + (red_sum[h] + red_sum[kAH + h] + red_sum[2 * kAH + h] + red_sum[3 * kAH + h]);
        }
        // ---- O = O * alpha + P V for dims 128w .. 128w+127
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) o[nt][jj] *= alpha[jj];
        // transposed read: lane (lg, l16) points at key 32kq + 8lg + l16/4 (+4
        // for the second read; key group 4kq + lg), dims d0 + 4 (l16 % 4) .. +4
        // with d0 = 128w + 16nt: piece 16w + 2nt + (l16 % 4)/2 (group 2w + nt/4,
        // 2 (nt % 4) + (l16 % 4)/2 within it), bytes 8 (l16 % 2) of the piece
        const int vkk = l16 >> 2, vh = (l16 & 3) >> 1;
        const unsigned char *vb0 = cb + lg * kBlk + vkk * 128 + (l16 & 1) * 8;
#pragma unroll
        for (int kq = 0; kq < kChunk / 32; ++kq) {
            const abf16x8_t pah = *(const abf16x8_t *)(ph + l16 * kPStride + 32 * kq + 8 * lg);
            const abf16x8_t pal = *(const abf16x8_t *)(pl + l16 * kPStride + 32 * kq + 8 * lg);
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                const unsigned char *vp = vb0 + 4 * kq * kBlk + (2 * wave + (nt >> 2)) * kKGroups * kBlk;
                const int pg = 2 * (nt & 3) + vh;
                const abf16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (abf16x4_t __attribute__((address_space(3))) *)(vp + ((pg - vkk) & 7) * 16));
                const abf16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (abf16x4_t __attribute__((address_space(3))) *)(vp + 4 * 128 + ((pg - vkk - 4) & 7) * 16));
                const abf16x8_t vb = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
                o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pah, vb, o[nt], 0, 0, 0);
                o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pal, vb, o[nt], 0, 0, 0);
            }
        }
    }
    if (a.nsplit == 1) {
        // ---- the row's result: out = o / l, lse = m + log l
        float *op = a.out + (int64_t)r * kAH * kAV;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float inv = l_run[jj] > 0.0f ? 1.0f / l_run[jj] : 0.0f;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) op[(4 * lg + jj) * kAV + 128 * wave + 16 * nt + l16] = o[nt][jj] * inv;
        }
        if (wave == 0 && l16 == 0)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                a.lse[(int64_t)r * kAH + 4 * lg + jj] = l_run[jj] > 0.0f ? m_run[jj] + logf(l_run[jj]) : -INFINITY;
        return;
    }
    // ---- the split's partial result: o (unnormalised), m, l per head
    float *op = a.part_o + ((int64_t)r * a.nsplit + x) * kAH * kAV;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) op[(4 * lg + jj) * kAV + 128 * wave + 16 * nt + l16] = o[nt][jj];
    if (wave == 0 && l16 == 0) {
        float *mp = a.part_ml + ((int64_t)r * a.nsplit + x) * 2 * kAH;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            mp[4 * lg + jj] = m_run[jj];
            mp[kAH + 4 * lg + jj] = l_run[jj];
        }
    }
}

// Workgroup (blk, r) merges the splits of outputs blk*256 .. +256 of row r
// (half of one head's 512 values).
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a) {
    __shared__ float wsc[kAttnMaxSplit];   // exp(m_x - M) of the head, per split
    __shared__ float inv_l;
    const int blk = blockIdx.x, r = blockIdx.y, t = threadIdx.x;
    const int h = blk / (kAV / 256);
    const float *ml = a.part_ml + (int64_t)r * a.nsplit * 2 * kAH;
    if (t < 64) {   // wave 0: lane x holds split x (nsplit <= 32)
        const float m = t < a.nsplit ? ml[t * 2 * kAH + h] : -INFINITY;
        const float l = t < a.nsplit ? ml[t * 2 * kAH + kAH + h] : 0.0f;
        float M = m;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
        const float w = (m == -INFINITY) ? 0.0f : expf(m - M);
        float L = w * l;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) L += __shfl_xor(L, o);
        if (t < kAttnMaxSplit) wsc[t] = w;
        if (t == 0) {
            inv_l = L > 0.0f ? 1.0f / L : 0.0f;
            if (blk % (kAV / 256) == 0) a.lse[(int64_t)r * kAH + h] = L > 0.0f ? M + logf(L) : -INFINITY;
        }
    }
    __syncthreads();
    const int i = blk * 256 + t;   // output element of the row: head h, dim i % 512
    const float *po = a.part_o + (int64_t)r * a.nsplit * kAH * kAV + i;
    float acc = 0.0f;
#pragma unroll 8
    for (int x = 0; x < a.nsplit; ++x) acc += wsc[x] * po[(int64_t)x * kAH * kAV];
    a.out[(int64_t)r * kAH * kAV + i] = acc * inv_l;
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, hipStream_t st) {
    const size_t lds = (size_t)kLdsAttn;
    // above 64 KiB of dynamic LDS the kernel declares how much it takes
    static const hipError_t attr = hipFuncSetAttribute((const void *)attn_kernel,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
    if (a.span > kMaxSpan || a.nsplit > kAttnMaxSplit) return hipErrorInvalidValue;
    hipLaunchKernelGGL(attn_kernel, dim3(a.nsplit, a.rows), dim3(256), lds, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    hipLaunchKernelGGL(combine_kernel, dim3(kAH * kAV / 256, a.rows), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace fp8idx
