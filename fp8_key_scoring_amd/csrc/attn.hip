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
//  * Grid (split x, row r), 4 waves per workgroup.  The split's span of the
//    index list is cut into chunks of 16 entries; wave w takes chunks w,
//    w+4, ... and runs the whole online softmax over them on its own: no
//    workgroup barrier and no exchange between waves until the end, where
//    the four waves' (max, sum, output) are merged through LDS.
//  * A chunk's 16 cache rows (1,152 B each, found through the page table)
//    go straight from HBM to LDS with global_load_lds_dwordx4 (16 bytes per
//    lane, no registers): one instruction moves 8 keys x 128 B, eight lanes
//    per key reading one whole 128-byte line, into a 1 KiB block.  Block
//    (key group G, piece group P) holds pieces 8P..8P+7 (piece p = dims
//    8p..8p+7) of keys 8G..8G+7, key kk of group G keeping piece p in slot
//    (p - kk + G) mod 8, which leaves both operand reads below free of bank
//    conflicts.  Each wave has two buffers: chunk i+1 streams in while chunk
//    i is computed.  (The chunk step takes the two buffers as restrict
//    pointers: with that the compiler knows the reads of one do not wait for
//    the DMA into the other.)
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (M = the chunk's 16 keys, N =
//    the 16 heads, K = 576 dims in 18 steps, two accumulation chains; q in
//    registers for the whole split).  Its result leaves each lane one head
//    and 4 keys, which is exactly the B operand of O^T = V^T P^T on
//    v_mfma_f32_16x16x16_bf16 (K = the 16 keys), so the weights never leave
//    registers.
//  * Softmax in base 2 (logits times sm_scale * log2 e, v_exp_f32); the
//    per-head maximum and sum over the chunk combine the lane's 4 keys and
//    the four 16-lane rows (permlane32/16 swaps).  The output is rescaled
//    only when some head's maximum grows by more than 2^8 over the one in use
//    (otherwise the weights stay below 2^8, exact enough in fp32), so most
//    chunks skip the 128-register rescale.
//  * O^T += V^T P^T: A = 16 dims x 16 keys of V, read transposed from the
//    key-major tile with ds_read_b64_tr_b16 (lane i of a 16-lane group gets
//    dim i of the 4 keys the group points at), B = P split into bf16 hi + lo
//    (~16 significant bits), 32 tiles for the 512 value dims.
//  * With one split per row the workgroup normalises and writes out and lse
//    itself.  Otherwise each split's unnormalised output, base-2 maximum and
//    sum go to the workspace and combine_kernel merges them (a workgroup per
//    256 outputs of a row): M = max_x m_x, w_x = 2^(m_x - M),
//    out = sum w_x o_x / sum w_x l_x, lse = ln 2 * (M + log2 sum w_x l_x).
#include "common.h"

namespace fp8idx {

namespace {

typedef __bf16 abf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 abf16x4_t __attribute__((ext_vector_type(4)));
typedef short ai16x4_t __attribute__((ext_vector_type(4)));
typedef float af32x4_t __attribute__((ext_vector_type(4)));
#define AS_GLOBAL(p) ((const void __attribute__((address_space(1))) *)(p))
#define AS_LDS(p) ((void __attribute__((address_space(3))) *)(p))

constexpr int kAH = kAttnHeads;      // 16 query heads
constexpr int kAD = kAttnDim;        // 576 latent + rotary dims
constexpr int kAV = kAttnVDim;       // 512 value dims
constexpr int kWChunk = kAttnWaveChunk;   // 16 keys per wave chunk
constexpr int kWaves = 4;            // waves per workgroup, two buffers each
constexpr int kKs = kAD / 32;        // 18 K steps of Q K^T
constexpr int kPGroups = kAD / 64;   // 9 groups of 8 pieces (128 B of a row)
constexpr int kKGroups = kWChunk / 8;     // 2 groups of 8 keys
constexpr int kVTiles = kAV / 16;    // 32 tiles of 16 value dims
constexpr int kBlk = 1024;           // block (G, P) at (P * kKGroups + G) * kBlk
constexpr int kWBuf = kPGroups * kKGroups * kBlk;     // 18,432 B per chunk buffer
constexpr int kOStride = kAV + 4;    // merge area row stride (floats): rows start on different banks
constexpr int kLdsAttn = 2 * kWaves * kWBuf;          // 147,456 B
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.0f;     // log2 of the weight growth allowed before rescaling
static_assert(kLdsAttn <= 160 * 1024, "attention tile fits the LDS");
static_assert(kAH * kOStride * 4 + 2 * kAH * 4 <= 2 * kWBuf, "a wave's result fits its two buffers");
static_assert(kWChunk == 16, "one S^T tile per chunk");

// Sums / maxima over the four 16-lane rows (lane l with l +- 16, +- 32): every
// lane ends with the value of its column.
__device__ __forceinline__ float rows4_max(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
    v = fmaxf(__int_as_float(a[0]), __int_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
    return fmaxf(__int_as_float(b[0]), __int_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
    v = __int_as_float(a[0]) + __int_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
    return __int_as_float(b[0]) + __int_as_float(b[1]);
}

__device__ __forceinline__ ai16x4_t tr_read(const unsigned char *p) {
    return __builtin_bit_cast(ai16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                            (abf16x4_t __attribute__((address_space(3))) *)(p)));
}

__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(1, 1))) void attn_kernel(AttnArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int x = blockIdx.x, r = blockIdx.y;
    const int l16 = lane & 15, lg = lane >> 4;
    unsigned char *wb0 = lds + 2 * wave * kWBuf;             // this wave's two chunk buffers
    unsigned char *wb1 = wb0 + kWBuf;
    const int64_t j0 = (int64_t)x * a.span;
    const int n = (int)max((int64_t)0, min((int64_t)a.span, (int64_t)a.topk - j0));   // entries of the split
    const int nwc = n > kWChunk * wave ? (n - kWChunk * wave + kWaves * kWChunk - 1) / (kWaves * kWChunk) : 0;

    const int prow = a.row_pt[r];
    const bool prow_ok = prow >= 0 && prow < a.pt_rows;
    const int32_t *pt = a.page_table + (int64_t)(prow_ok ? prow : 0) * a.pt_stride;
    const int32_t *sl = a.sel + (int64_t)r * a.topk + j0;
    // DMA lane roles: key kk = lane / 8 of each key group G; slot j = lane % 8
    // of each piece group receives piece (j + kk - G) mod 8
    const int kk = lane >> 3;
    // (loads are unconditional, from clamped in-range addresses, and their
    // values are selected afterwards: a load under a branch would be waited
    // for inside the branch, one round trip per key group)
    auto load_sel = [&](int i, int (&sv)[kKGroups]) {
#pragma unroll
        for (int G = 0; G < kKGroups; ++G) {
            const int e = kWChunk * (wave + kWaves * i) + 8 * G + kk;
            const bool in = (i < nwc) & (e < n) & prow_ok;
            const int v = sl[max(min(e, n - 1), 0)];   // (j0 < topk: entry 0 of the split exists)
            sv[G] = in ? v : -1;
        }
    };
    // the page ids of the entries (loads only: they are combined into cache
    // rows when the chunk is issued)
    auto load_pages = [&](const int (&sv)[kKGroups], int (&pg)[kKGroups]) {
#pragma unroll
        for (int G = 0; G < kKGroups; ++G) {
            const int s = sv[G];
            const bool sok = (s >= 0) & (s < a.max_bound);   // (max_bound <= pt_stride * 64)
            pg[G] = pt[sok ? s / kPage : 0];
        }
    };
    auto rows_of = [&](const int (&sv)[kKGroups], const int (&pg)[kKGroups], int (&row)[kKGroups]) {
#pragma unroll
        for (int G = 0; G < kKGroups; ++G) {
            const int s = sv[G];
            const bool ok = (s >= 0) & (s < a.max_bound) & (pg[G] >= 0) & (pg[G] < a.num_pages);   // (no branches)
            row[G] = ok ? pg[G] * kPage + s % kPage : -1;
        }
    };
    auto issue = [&](const int (&row)[kKGroups], unsigned char *buf) {
#pragma unroll
        for (int G = 0; G < kKGroups; ++G) {
            const int pj = ((lane & 7) + kk - G) & 7;
            const uint16_t *src = a.kv + (int64_t)(row[G] < 0 ? 0 : row[G]) * kAD + 8 * pj;
            unsigned char *dst = buf + G * kBlk;
#pragma unroll
            for (int P = 0; P < kPGroups; ++P)
                __builtin_amdgcn_global_load_lds(AS_GLOBAL(src + 64 * P), AS_LDS(dst + P * kKGroups * kBlk), 16, 0, 0);
        }
    };

    // ---- prologue: entries of chunks 0-2 and page ids of chunks 0-1 out,
    // then chunk 0's DMA.  In the loop every lookup value is used only after
    // the next loop-head wait, so no wait inside an iteration stalls on them
    // (or on the DMA issued behind them).
    int sv0[kKGroups], pg0[kKGroups], row[kKGroups];
    int sv1[kKGroups], sv2[kKGroups], pg1[kKGroups];
    load_sel(0, sv0);
    load_sel(1, sv1);
    load_sel(2, sv2);
    // q of the row, the B operand of S^T: head l16, dims 32ks + 8lg .. +8
    abf16x8_t qb[kKs];
    {
        const uint16_t *q = a.q + ((int64_t)r * kAH + l16) * kAD + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) qb[ks] = *(const abf16x8_t *)(q + 32 * ks);
    }
    // q lives in AGPRs (the MFMA reads its B operand there)
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) asm volatile("" : "+a"(qb[ks]));
    load_pages(sv0, pg0);
    load_pages(sv1, pg1);
    rows_of(sv0, pg0, row);
    if (nwc > 0) issue(row, wb0);

    const float c2 = a.sm_scale * kLog2e;
    float m_use = -INFINITY, l_run = 0.0f;   // head l16 (base-2 maximum)
    af32x4_t o[kVTiles];        // O^T: dims 16nt + 4lg + jj, head l16
#pragma unroll
    for (int nt = 0; nt < kVTiles; ++nt) o[nt] = af32x4_t{0.f, 0.f, 0.f, 0.f};
    bool o_zero = true;         // nothing accumulated yet (wave-uniform)

    // S^T lane roles (A operand): key l16 (group l16/8, kk = l16 % 8), piece
    // 4ks + lg (group ks/2, 4 (ks % 2) + lg within it)
    const int skk = l16 & 7, sg = l16 >> 3;
    const int ka_off = sg * kBlk + skk * 128;
    const int so0 = ((lg - skk + sg) & 7) * 16, so1 = ((4 + lg - skk + sg) & 7) * 16;
    // V^T lane roles (A operand): the 16 lanes of row lg point at key
    // 4lg + l16/4 (group lg/2), dims 16nt + 4 (l16 % 4) .. +4 (piece
    // 2nt + (l16 % 4)/2)
    const int vkk = 4 * (lg & 1) + (l16 >> 2), vg = lg >> 1, vh = (l16 & 3) >> 1;
    const int va_off = vg * kBlk + vkk * 128 + (l16 & 1) * 8;

    // One chunk: issue the next chunk's DMA into `nxt`, then compute the
    // current one from `cur`.  The two never overlap; as restrict pointers
    // they tell the compiler that the reads of `cur` need not wait for the
    // DMA into `nxt` (the wait for `cur`'s own rows is the explicit one).
    auto step = [&](int i, const unsigned char *__restrict__ cur, unsigned char *__restrict__ nxt) {
        // validity of the lane's 4 keys 4lg + jj (key 8G + kk is valid iff
        // lane 8kk resolved a row for group G)
        // (both ballots by the whole wave, then the lane's pick)
        const uint64_t bal0 = __ballot(row[0] >= 0), bal1 = __ballot(row[1] >= 0);
        const uint64_t bal = (lg >> 1) ? bal1 : bal0;
        int rown[kKGroups], pg2[kKGroups];
        rows_of(sv1, pg1, rown);   // chunk i+1
        load_pages(sv2, pg2);      // chunk i+2 (issued ahead of the DMA)
        if (i + 1 < nwc) issue(rown, nxt);
        // ---- S^T = K Q^T (two chains: even and odd K steps)
        const unsigned char *ka = cur + ka_off;
        af32x4_t s0 = af32x4_t{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
        for (int ks = 0; ks < kKs; ks += 2) {
            const int off = (ks >> 1) * kKGroups * kBlk;
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const abf16x8_t *)(ka + off + so0), qb[ks], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const abf16x8_t *)(ka + off + so1), qb[ks + 1], s1, 0, 0, 0);
        }
        // ---- online softmax (base 2) over the lane's keys of head l16
        float v[4];
        float cm = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const bool ok = ((bal >> (8 * (4 * (lg & 1) + jj))) & 1) != 0;
            v[jj] = ok ? (s0[jj] + s1[jj]) * c2 : -INFINITY;
            cm = fmaxf(cm, v[jj]);
        }
        cm = rows4_max(cm);
        if (__ballot(cm > m_use + kRescale)) {   // (also the first finite maximum)
            const float mn = fmaxf(m_use, cm);
            const float alpha = m_use == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_use - mn);
            l_run *= alpha;
            m_use = mn;
            if (!o_zero)
#pragma unroll
                for (int nt = 0; nt < kVTiles; ++nt) o[nt] *= alpha;
        }
        ai16x4_t ph, pl;
        float csum = 0.0f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float p = v[jj] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(v[jj] - m_use);
            csum += p;
            const __bf16 hi = (__bf16)p;
            ph[jj] = __builtin_bit_cast(short, hi);
            pl[jj] = __builtin_bit_cast(short, (__bf16)(p - (float)hi));
        }
        l_run += rows4_sum(csum);
        // ---- O^T += V^T P^T (A: V tiles read transposed from `cur`)
        const unsigned char *va = cur + va_off;
#pragma unroll
        for (int nt = 0; nt < kVTiles; ++nt) {
            const int pp = 2 * (nt & 3) + vh;   // piece within its group
            const ai16x4_t vt = tr_read(va + (nt >> 2) * kKGroups * kBlk + ((pp - vkk + vg) & 7) * 16);
            o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, ph, o[nt], 0, 0, 0);
            o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, pl, o[nt], 0, 0, 0);
        }
        o_zero = false;
        int sv3[kKGroups];
        load_sel(i + 3, sv3);
#pragma unroll
        for (int G = 0; G < kKGroups; ++G) {
            row[G] = rown[G];
            sv1[G] = sv2[G];
            pg1[G] = pg2[G];
            sv2[G] = sv3[G];
        }
    };
    for (int i = 0; i < nwc; ++i) {
        // chunk i (and chunk i+1's entries and page ids) have landed; this
        // wave's reads of the other buffer (chunk i-1) have returned, so it
        // may be refilled.  (The intrinsic, unlike an asm wait, tells the
        // compiler that every earlier load is complete; the empty asm keeps
        // memory accesses from moving across it.)
        __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
        asm volatile("" ::: "memory");
        const int odd = i & 1;
        step(i, odd ? wb1 : wb0, odd ? wb0 : wb1);
    }

    // ---- merge the waves: each writes (o, m, l) into its two buffers
    float *so = (float *)wb0;                           // [16 heads][kOStride]
    float *sml = (float *)(wb0 + kAH * kOStride * 4);   // [2][16]: base-2 maxima, sums
    __builtin_amdgcn_s_waitcnt(0x0070);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int nt = 0; nt < kVTiles; ++nt) *(af32x4_t *)(so + l16 * kOStride + 16 * nt + 4 * lg) = o[nt];
    if (lg == 0) {
        sml[l16] = m_use;
        sml[kAH + l16] = l_run;
    }
    __syncthreads();
    __shared__ float wgt[kWaves][kAH];   // 2^(m_w - M) per wave and head
    __shared__ float hM[kAH], hL[kAH];
    if (t < kAH) {
        float mw[kWaves], M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            mw[w] = ((const float *)(lds + 2 * w * kWBuf + kAH * kOStride * 4))[t];
            M = fmaxf(M, mw[w]);
        }
        float L = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float g = mw[w] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw[w] - M);
            wgt[w][t] = g;
            L += g * ((const float *)(lds + 2 * w * kWBuf + kAH * kOStride * 4))[kAH + t];
        }
        hM[t] = M;
        hL[t] = L;
    }
    __syncthreads();
    const bool direct = a.nsplit == 1;
    float *dst = direct ? a.out + (int64_t)r * kAH * kAV : a.part_o + ((int64_t)r * a.nsplit + x) * kAH * kAV;
    // four consecutive outputs per thread and step (16-byte loads and stores)
#pragma unroll 4
    for (int e = 4 * t; e < kAH * kAV; e += 4 * 64 * kWaves) {
        const int h = e / kAV, d = e % kAV;
        af32x4_t v = af32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            v += wgt[w][h] * *(const af32x4_t *)((const float *)(lds + 2 * w * kWBuf) + h * kOStride + d);
        if (direct) v *= hL[h] > 0.0f ? 1.0f / hL[h] : 0.0f;
        *(af32x4_t *)(dst + e) = v;
    }
    if (t < kAH) {
        if (direct) {
            a.lse[(int64_t)r * kAH + t] = hL[t] > 0.0f ? kLn2 * (hM[t] + __log2f(hL[t])) : -INFINITY;
        } else {
            float *mp = a.part_ml + ((int64_t)r * a.nsplit + x) * 2 * kAH;
            mp[t] = hM[t];
            mp[kAH + t] = hL[t];
        }
    }
}

// Workgroup (blk, r) merges the splits of outputs blk*256 .. +256 of row r
// (half of one head's 512 values).  The partial outputs are loaded before
// the weights are known (they do not depend on them).
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a) {
    __shared__ float wsc[kAttnMaxSplit];   // 2^(m_x - M) of the head, per split
    __shared__ float inv_l;
    const int blk = blockIdx.x, r = blockIdx.y, t = threadIdx.x;
    const int h = blk / (kAV / 256);
    const int i = blk * 256 + t;   // output element of the row: head h, dim i % 512
    const float *po = a.part_o + (int64_t)r * a.nsplit * kAH * kAV + i;
    float pv[kAttnMaxSplit];
#pragma unroll
    for (int x = 0; x < kAttnMaxSplit; ++x) pv[x] = x < a.nsplit ? po[(int64_t)x * kAH * kAV] : 0.0f;
    const float *ml = a.part_ml + (int64_t)r * a.nsplit * 2 * kAH;
    if (t < 64) {   // wave 0: lane x holds split x (nsplit <= 32)
        const float m = t < a.nsplit ? ml[t * 2 * kAH + h] : -INFINITY;
        const float l = t < a.nsplit ? ml[t * 2 * kAH + kAH + h] : 0.0f;
        const float M = wave_max_f32(m);
        const float w = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
        const float L = wave_sum_f32(w * l);
        if (t < kAttnMaxSplit) wsc[t] = w;
        if (t == 0) {
            inv_l = L > 0.0f ? 1.0f / L : 0.0f;
            if (blk % (kAV / 256) == 0) a.lse[(int64_t)r * kAH + h] = L > 0.0f ? kLn2 * (M + __log2f(L)) : -INFINITY;
        }
    }
    __syncthreads();
    float acc = 0.0f;
#pragma unroll
    for (int x = 0; x < kAttnMaxSplit; ++x) acc += wsc[x] * pv[x];   // (wsc is 0 past nsplit)
    a.out[(int64_t)r * kAH * kAV + i] = acc * inv_l;
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, hipStream_t st) {
    const size_t lds = (size_t)kLdsAttn;
    // above 64 KiB of dynamic LDS the kernel declares how much it takes
    static const hipError_t attr = hipFuncSetAttribute((const void *)attn_kernel,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
    if (a.nsplit > kAttnMaxSplit || a.span % kWChunk != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(attn_kernel, dim3(a.nsplit, a.rows), dim3(64 * kWaves), lds, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    hipLaunchKernelGGL(combine_kernel, dim3(kAH * kAV / 256, a.rows), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace fp8idx
