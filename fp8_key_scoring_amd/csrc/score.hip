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
//  * A workgroup is 4 waves, one per SIMD, each with the whole 512-entry
//    register file.  It takes the row groups (up to 4 consecutive rows that
//    share a page-table row: one request's verify rows) that start in its
//    block of 4 rows, and one chunk of their keys.  Each wave scores all of a
//    group's rows, so a key is read from HBM once and converted once; wave w
//    takes page w of every block of four pages of the chunk.
//  * Per 16-key group a lane loads 32 contiguous code bytes of key lane%16
//    (two 16-byte loads from a wave-uniform base: the page id is read from a
//    register holding the chunk's page ids, the rest is a fixed per-lane
//    offset) plus that key's scale, four groups ahead.  The codes go straight
//    to registers, are widened E4M3 -> bf16 (exact) with the gfx950 packed
//    conversion, and feed the B operand of v_mfma_f32_16x16x32_bf16 (K = the
//    128 head dims in 4 steps, N = 16 keys).  The A operand is q, 16 heads
//    per MFMA, held in AGPRs for the whole chunk (64 per row).  The order in
//    which head dims feed the K index is a free permutation applied to q and
//    k alike.  (The fp8 x fp8 MFMA is not used: it would need q in fp8.)
//  * Epilogue: lane l holds heads 16b + 4(l/16) + j of key l%16 for b, j < 4.
//    max(d, 0) = (d + |d|) / 2: the linear half, (1/2) sum_h w_h d_h, is one
//    more MFMA block against (1/2) sum_h w_h q_h; the other half is one fma
//    per head with |d| as a free source modifier.  Two permlane swap rounds
//    (32 and 16 lanes) finish the sum over the 64 heads for four groups at
//    once, and the keys' scales multiply the totals.
//  * Scores leave from registers: after every page of a wave, lane l holds
//    the score of the page's key l, so each row's 64 scores are one 256-byte
//    buffer store, masked at the row's bound by the buffer's extent.  When
//    counting, the same lanes add each score's first radix digit to per-row
//    LDS counters, which are added to the row's global histogram at the end.
#include "common.h"

namespace fp8idx {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 16-key groups loaded ahead per wave (a multiple of 4).  A group feeds 16
// MFMAs per row; eight groups ahead pay only for one row over a long context
// (1 row x 524,288 keys: 19.5 against 20.2 us with four); with two rows four
// are faster (2 rows x 524,288 keys: 21.6 against 23.1 us with eight: the
// start-up burst of every wave's ring is half as long).  The loop runs whole
// rings, so a wave with fewer groups than its ring computes (and discards)
// the difference: one row's waves with fewer than 16 groups take four.
constexpr int kDeepRingGroups = 16;
template <int R>
constexpr int ring_depth() { return R >= 2 ? 4 : 8; }

__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
    bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// First-digit counters in LDS: [wave][row slot][digit][4], each wave with its
// own, lane l adding into copy l % 4 of its digit.  A wave's scores share only
// a handful of first digits, so its lanes' adds collide on a few words; the
// adds need no result, so the collisions cost LDS cycles the wave does not
// wait for.  What the wave does wait for is the sum at the end of a row group
// (lane = digit: four 16-byte reads, one per wave); with one counter per lane
// and digit that sum read 64 words per lane and cost about 1.2 us more.
constexpr int kCntCopies = 4;
constexpr int kHistLds = (kScoreThreads / 64) * kGroupRows * kBins1 * kCntCopies;   // u32 counters
constexpr int kBlockPieces = kGroupRows * kHeads * kDim / 8 / kScoreThreads;   // q pieces per thread, 4 rows
// Word 3 of a raw buffer resource for 32-bit accesses (32-bit data format).
constexpr int kBufferFlags = 0x00020000;
// Cache policy of the score stores: sc1, written through to the device-coherent
// level, so the kernel's end has no dirty score lines to write back from the
// XCD's L2 before the selection kernels (on other XCDs) read them (4 rows x
// 524,288 keys: the launch 48.5 -> 47.4 us, interleaved).
constexpr int kScoreStorePolicy = 16;

// Dynamic LDS: q of four rows, then the linear term's A operand.  q is read
// only while a row group is set up; when counting, the same 64 KB then hold
// the first-digit counters.  (A launch asking for twice the LDS, q and the
// counters side by side, costs about 3 us more to start even when its
// workgroups return at once.)
constexpr int kLdsQ = kGroupRows * kHeads * kDim * 2;     // 64 KB
constexpr int kLdsT1 = 4 * 64 * 8 * 2;                   // [ks][lane][8] bf16, 4 KB
static_assert(kHistLds * 4 <= kLdsQ, "the counters reuse the q region");

// The same pointer, held in scalar registers and opaque to the optimiser:
// a load from it plus a 32-bit lane offset then uses the scalar-base
// addressing form instead of a 64-bit vector add per load.
template <typename T>
using gptr = const __attribute__((address_space(1))) T *;   // global memory

template <typename T>
__device__ __forceinline__ gptr<T> scalar_ptr(const T *p) {
    uint64_t v = (uint64_t)p;
    asm volatile("" : "+s"(v));
    return (gptr<T>)v;
}

// A workgroup barrier for LDS traffic: it waits for this wave's LDS
// operations only.  __syncthreads() also waits for every global load the wave
// has in flight, which in the set-up would hold every wave until its whole
// key ring had arrived.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Sums each of four per-lane partials over the four 16-lane rows and leaves
// the total of partial q in lane row q (each lane keeps its column): one
// 32-lane swap round and one 16-lane swap round.
__device__ __forceinline__ float reduce4(float p0, float p1, float p2, float p3) {
    const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_int(p0), __float_as_int(p2), false, false);
    const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_int(p1), __float_as_int(p3), false, false);
    // lanes 0-31: partial 0 (or 1) summed over lane rows {0,2} / {1,3};
    // lanes 32-63: the same for partial 2 (or 3)
    const float a02 = __int_as_float(s02[0]) + __int_as_float(s02[1]);
    const float a13 = __int_as_float(s13[0]) + __int_as_float(s13[1]);
    const auto t = __builtin_amdgcn_permlane16_swap(__float_as_int(a02), __float_as_int(a13), false, false);
    return __int_as_float(t[0]) + __int_as_float(t[1]);
}

// q in LDS: [row slot][head][16 pieces of 16 bytes], piece p of head h at
// position p ^ (h % 16), so the sixteen heads that one A-operand read
// instruction touches hit distinct banks.
__device__ __forceinline__ int q_lds_off(int r, int h, int piece) {
    return ((r * kHeads + h) * 16 + (piece ^ (h & 15))) * 16;
}

// Loads q of rows row0 .. row0+R-1 (every thread of the workgroup a share)
// and writes it to LDS row slots 0..R-1.
template <int R>
__device__ __forceinline__ void stage_q(const ScoreArgs &a, int row0, int tid, unsigned char *lds_q) {
    constexpr int kPieces = R * kHeads * kDim / 8 / kScoreThreads;   // 16-byte pieces per thread
    u32x4_t qt[kPieces];
#pragma unroll
    for (int c = 0; c < kPieces; ++c) {
        const int ci = tid + c * kScoreThreads;   // piece index: row, head, piece
        qt[c] = *(gptr<u32x4_t>)(a.q + ((int64_t)(row0 + (ci >> 10)) * kHeads + ((ci >> 4) & 63)) * kDim +
                                 8 * (ci & 15));
    }
#pragma unroll
    for (int c = 0; c < kPieces; ++c) {
        const int ci = tid + c * kScoreThreads;
        *(u32x4_t *)(lds_q + q_lds_off(ci >> 10, (ci >> 4) & 63, ci & 15)) = qt[c];
    }
}

// The linear term's A operand for row slot ur of a group whose q starts at LDS
// row slot q_slot: A row 4p + ur holds part p of u = sum_h (w[h]/2) q[h] (fp32),
// split into three bf16 parts hi + mid + lo (each residual exact in fp32, so
// the three carry u to fp32 precision).  One wave: lane l sums dims
// 8 (l % 16) .. +7 over the sixteen heads whose halved weights it holds for
// the epilogue, wh[hb][jj] for head 16 hb + 4 (l / 16) + jj -- one 16-byte LDS
// read per head and eight independent fma chains -- and two permlane swap
// rounds add the four lane rows' partial sums, after which lane row p (p < 3)
// writes part p of its eight dims as one 16-byte store.
__device__ __forceinline__ void linear_u(const unsigned char *lds_q, int q_slot, int ur, const f32x4_t (&wh)[4],
                                         __bf16 *t1_lds, int lane) {
    typedef __bf16 bf16x8l_t __attribute__((ext_vector_type(8)));
    const int pc = lane & 15, lr4 = lane >> 4;
    u32x4_t qv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        qv[i] = *(const u32x4_t *)(lds_q + q_lds_off(q_slot + ur, 16 * (i >> 2) + 4 * lr4 + (i & 3), pc));
    float u[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) u[e] = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float w = wh[i >> 2][i & 3];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            u[2 * e] = fmaf(w, __uint_as_float(qv[i][e] << 16), u[2 * e]);
            u[2 * e + 1] = fmaf(w, __uint_as_float(qv[i][e] & 0xffff0000u), u[2 * e + 1]);
        }
    }
    bf16x8l_t part;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const auto a32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(u[e]), __float_as_uint(u[e]), false, false);
        const float s2 = __uint_as_float(a32[0]) + __uint_as_float(a32[1]);
        const auto a16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(s2), __float_as_uint(s2), false, false);
        const float uu = __uint_as_float(a16[0]) + __uint_as_float(a16[1]);
        const __bf16 hi = (__bf16)uu;
        const float r1 = uu - (float)hi;
        const __bf16 mid = (__bf16)r1;
        const __bf16 lo = (__bf16)(r1 - (float)mid);
        part[e] = lr4 == 0 ? hi : (lr4 == 1 ? mid : lo);
    }
    // dims 8pc .. 8pc+7: K step pc % 4 of the A operand, lane row pc / 4
    if (lr4 < 3) *(bf16x8l_t *)(t1_lds + ((pc & 3) * 64 + lr4 * 4 + ur + 16 * (pc >> 2)) * 8) = part;
}

struct KeyGroup {
    u32x4_t lo, hi;   // 32 code bytes of key lane%16
    float scale;
    int ok;           // wave-uniform: the page id was in range
};

// What one wave scores: R rows (R = 1..4) over its share of the chunk's
// 16-key groups.  The chunk is cut into blocks of 16 groups (4 pages); wave w
// takes page w of each block, i.e. its i-th group is
// gbase + 16 * (i / 4) + i % 4 with gbase = (first group of the chunk) + 4w,
// so every 4 consecutive groups of a wave are one page: 64 consecutive keys.
struct WaveJob {
    int tid;         // thread index in the workgroup
    int lane;
    int c0;          // first key of the chunk (a multiple of 64)
    int chunk;       // keys per chunk
    int gbase;       // the wave's first 16-key group (index over the request's keys)
    int n_my;        // groups the wave takes
    int vpage;       // page id of the chunk's page number `lane` (-1: out of range)
    int row0;        // the wave's first row
    int bnd[kGroupRows];   // exclusive bounds of the wave's rows
    __device__ __forceinline__ int group(int i) const { return gbase + 16 * (i >> 2) + (i & 3); }
};

// Scores R rows of one wave.  A "unit" is (group, row); units run in order
// (group 0 row 0, group 0 row 1, group 1 row 0, ...).  In the step of unit u
// the 16 MFMAs of unit u, the epilogue of unit u-1 and (on a group's last
// row) the conversion of the next group and the refill of its ring slot are
// independent, and the scheduler interleaves them: one MFMA, then a few VALU
// ops.  A group's keys are converted once and used by all R rows.
template <int R, bool kHist, int kRing = ring_depth<R>()>
__device__ __forceinline__ void score_rows(const ScoreArgs &a, const WaveJob &j, unsigned char *lds_q,
                                           bf16_t *t1_lds, uint32_t *lds_cnt, int q_slot, bool staged,
                                           bool u_ready) {
    const int lane = j.lane;
    const int kig = lane & 15;      // key of the group this lane loads / scores
    const int lrow = lane >> 4;     // lane row: 32-byte quarter of the key, 4-head slice of D
    const uint32_t koff = (uint32_t)(kig * kDim + lrow * 32);
    const int gc0 = j.c0 / kKeysPerMfma;

    // Loads are unconditional: past the wave's last group they re-read that
    // group (always in range), so no branch separates a load from its use.
    // The group's base addresses are wave-uniform; each lane adds its fixed
    // 32-bit offset.
    auto load_group = [&](int i, KeyGroup &kg) {
        const int ic = max(min(i, j.n_my - 1), 0);   // in range also when n_my == 0
        const int g = j.group(ic);
        const int page = __builtin_amdgcn_readlane(j.vpage, (g - gc0) >> 2);
        kg.ok = page >= 0;
        const int64_t key0 = (int64_t)(kg.ok ? page : 0) * kPage + (g & 3) * kKeysPerMfma;
        gptr<uint8_t> kbase = scalar_ptr(a.k8 + key0 * kDim);
        gptr<float> sbase = scalar_ptr(a.kscale + key0);
        kg.lo = *(gptr<u32x4_t>)(kbase + koff);
        kg.hi = *(gptr<u32x4_t>)(kbase + koff + 16);
        kg.scale = sbase[kig];
    };

    // q of the group's rows sits in LDS, one 16 KB row after another from
    // row slot q_slot: staged with the workgroup's block of rows, or here
    // when the group's rows were not.  Each wave reads q back in MFMA
    // A-operand order (head 16*hb + lane%16, dims 32*(lane/16) + 8*ks +
    // [0, 8)) straight into the registers the MFMAs read.  The order of the
    // set-up favours the key stream: the key ring goes out first (the page
    // ids are in by now), then the q reads and the weights, the linear term
    // (LDS and VALU work) last; issuing the ring after the q reads cost
    // 0.2-0.8 us per launch.
    bf16x8_t qa[R][4][4];
    bf16x8_t t1a[4];      // A operand of the linear term (below)
    f32x4_t wv[R][4];
    KeyGroup kb[kRing];   // group g of the wave lives in slot g % kRing
    {
        const int tid = j.tid;
        const int wave_idx = tid >> 6;
        if (!staged) {   // q_slot is 0 here
            stage_q<R>(a, j.row0, tid, lds_q);
            lds_barrier();
        }
        // weights of the D rows a lane holds: heads 16*hb + 4*(lane/16) + jj
        // (issued ahead of the ring: loads complete in order, and the first
        // step's epilogue must not wait for the whole ring)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int hb = 0; hb < 4; ++hb)
                wv[r][hb] = *(gptr<f32x4_t>)(a.w + (int64_t)(j.row0 + r) * kHeads + 16 * hb + 4 * lrow) * 0.5f;
#pragma unroll
        for (int p = 0; p < kRing; ++p) load_group(p, kb[p]);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int hb = 0; hb < 4; ++hb)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    qa[r][hb][ks] = *(const bf16x8_t *)(lds_q + q_lds_off(q_slot + r, 16 * hb + kig, 4 * lrow + ks));
        // The linear term's A operand (linear_u): wave q_slot + r builds row
        // r's, unless the kernel built it while the page ids were in flight.
        const int ur = wave_idx - q_slot;
        if (!u_ready && ur >= 0 && ur < R) {
            f32x4_t wq[4];
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) {
                wq[hb] = wv[0][hb];
#pragma unroll
                for (int r = 1; r < R; ++r) wq[hb] = ur == r ? wv[r][hb] : wq[hb];
            }
            linear_u(lds_q, q_slot, ur, wq, t1_lds, lane);
        }
        lds_barrier();   // u is written; every wave is done reading q from LDS
        if (kHist) {     // the q region becomes the counters
            u32x4_t *c4 = (u32x4_t *)lds_cnt;
            const uint32_t z = (uint32_t)tid >> 16;   // 0, built here rather than kept live
            for (int i = tid; i < kHistLds / 4; i += kScoreThreads) c4[i] = u32x4_t{z, z, z, z};
        }
        const bool t1_row = (kig >> 2) < 3 && (kig & 3) < R;   // this lane's A row is used
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8_t v = *(const bf16x8_t *)(t1_lds + (ks * 64 + lane) * 8);
            t1a[ks] = t1_row ? v : bf16x8_t{};
        }
        // t1_lds may be written again by the next row group, and the
        // counters are clear before any wave adds to them
        lds_barrier();
    }
    if (j.n_my == 0) return;
    // q lives in AGPRs: the MFMA reads its A operand from there directly,
    // leaving the 256 architectural VGPRs to keys, results and weights
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                asm volatile("" : "+a"(qa[r][hb][ks]));

    auto convert = [&](const KeyGroup &kg, bf16x8_t (&kv)[4]) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const u32x4_t &src = ks < 2 ? kg.lo : kg.hi;
            kv[ks] = e4m3x8_to_bf16(src[(ks & 1) * 2], src[(ks & 1) * 2 + 1]);
        }
    };
    auto scale_of = [&](const KeyGroup &kg) { return kg.ok ? kg.scale : __builtin_nanf(""); };
    auto mfma_unit = [&](const bf16x8_t (&kv)[4], const bf16x8_t (&q)[4][4], f32x4_t (&acc)[4]) {
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) acc[hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int hb = 0; hb < 4; ++hb)
                acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q[hb][ks], kv[ks], acc[hb], 0, 0, 0);
    };
    // Epilogue.  sum_h w_h max(d_h, 0) = (1/2) sum_h w_h d_h + sum_h (w_h/2) |d_h|
    // (max(x, 0) = (x + |x|) / 2).  The first sum is linear in the key,
    // (1/2) sum_h w_h d_h = u . k with u = (1/2) sum_h w_h q_h, and comes from
    // one more MFMA block per 16-key group (A rows 4p + r: the bf16 parts of
    // row r's u; D element r of lane row p is part p's dot product).  The
    // second is one fma per element with the absolute value as a free source
    // modifier, instead of a max and an fma.
    // lane l holds D[head 16hb + 4(l/16) + jj][key l%16]: its sum over those
    // 16 heads (the other 48 heads of the key sit in the other lane rows),
    // started from this lane's part of the linear term
    auto partial = [&](const f32x4_t (&acc)[4], const f32x4_t (&w)[4], float init) {
        float part = init;
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                part = fmaf(w[hb][jj], fabsf(acc[hb][jj]), part);
        return part;
    };
    auto mfma_linear = [&](const bf16x8_t (&kv)[4], f32x4_t &t) {
        t = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t1a[ks], kv[ks], t, 0, 0, 0);
    };
    // Four groups form a block.  P[r][g & 3] is row r's partial of group g;
    // reduce4 turns a block's four partials into one register whose lane row
    // q holds the head sum of group 4m + q, which times the scale vector
    // sv (lane row q: scale of that group's key) is the block's scores.
    float P[R][4];
    // scale vectors: sv_fill collects the block being converted, sv_done
    // holds the last complete block until its flush.  A block is complete
    // when the first group of the next block is taken, which happens one
    // step before the flush of the complete block.
    float sv_fill = 0.0f, sv_done = 0.0f;
    // A block is one page of the wave: lane l holds the score of key
    // (first key of the page) + l, so each row's 64 scores go out as one
    // 256-byte store, masked at the row's bound, and (when counting) each
    // lane adds its score's first radix digit to its wave's counters.
    auto flush = [&](int g) {   // g: the wave's index of the block's last group
        const int iq = g - 3 + lrow;
        const int s = j.group(iq) * kKeysPerMfma + kig;
        const bool in_job = iq >= 0 && iq < j.n_my;
        const float scl = sv_done;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float out = reduce4(P[r][0], P[r][1], P[r][2], P[r][3]) * scl;
            // the row's keys [c0, bound) as a buffer: lanes past the bound or
            // outside the job fall outside it and the hardware drops their
            // stores, so no branch surrounds the store
            const int nrec = min(max(j.bnd[r] - j.c0, 0), j.chunk) * 4;
            const __amdgpu_buffer_rsrc_t row =
                __builtin_amdgcn_make_buffer_rsrc((void *)(a.scores + (int64_t)(j.row0 + r) * a.sstride + j.c0),
                                                  0, nrec, kBufferFlags);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(out), row, in_job ? (s - j.c0) * 4 : nrec, 0, kScoreStorePolicy);
            if (kHist) {   // every lane adds: 1 for a stored score, else 0 (no branch)
                const uint32_t d = radix_key(out) >> kDigit1Shift;
                atomicAdd(lds_cnt + (((j.tid >> 6) * kGroupRows + r) * kBins1 + d) * kCntCopies + lane % kCntCopies,
                          (in_job && s < j.bnd[r]) ? 1u : 0u);
            }
        }
    };
    // q = g & 3 must be a compile-time constant (g = i0 + p, i0 a multiple of 4)
    auto take_scale = [&](int q, const KeyGroup &kg) {
        if (q == 0) sv_done = sv_fill;
        sv_fill = lrow == q ? scale_of(kg) : sv_fill;
    };

    bf16x8_t kv[2][4];   // converted keys of group g in kv[g & 1]
    f32x4_t acc[2][4];   // D of unit u in acc[u & 1]
    f32x4_t t1[2];       // linear term of group g in t1[g & 1]
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) P[r][q] = 0.0f;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) acc[1][hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    t1[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    convert(kb[0], kv[0]);
    take_scale(0, kb[0]);   // (hands the empty block before group 0 to sv_done)
    load_group(kRing, kb[0]);

    const int n_iter = (j.n_my + kRing - 1) / kRing * kRing;
    for (int i0 = 0; i0 < n_iter; i0 += kRing) {
#pragma unroll
        for (int p = 0; p < kRing; ++p) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int u = p * R + r;
                mfma_unit(kv[p & 1], qa[r], acc[u & 1]);
                if (r == 0) mfma_linear(kv[p & 1], t1[p & 1]);
                // partial of the previous unit: row pr of group i0 + pp
                // (pp = -1 in the first step: a discarded value)
                const int pr = (r + R - 1) % R;
                const int pp = r == 0 ? p - 1 : p;
                P[pr][pp & 3] = partial(acc[(u + 1) & 1], wv[pr], t1[pp & 1][pr]);
                if (r == R - 1) {
                    KeyGroup &nx = kb[(p + 1) % kRing];
                    convert(nx, kv[(p + 1) & 1]);
                    take_scale((p + 1) & 3, nx);
                    load_group(i0 + p + 1 + kRing, nx);
                }
#pragma unroll
                for (int m = 0; m < (r == 0 ? 20 : 16); ++m) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // then up to four VALU
                }
                if (pr == R - 1 && (pp & 3) == 3) flush(i0 + pp);
                // nothing moves between steps: a step only reads results of
                // MFMAs issued in the step before
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    // partial of the last unit (row R-1 of group n_iter - 1; n_iter is a
    // multiple of 4, so this completes a block)
    P[R - 1][3] = partial(acc[1], wv[R - 1], t1[1][R - 1]);
    flush(n_iter - 1);
}

template <bool kHist>
__global__ __launch_bounds__(kScoreThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void score_kernel(ScoreArgs a) {
    // dynamic LDS: q of up to four rows (when counting, then the first-digit
    // counters [row][digit][64]) and the linear term's A operand
    extern __shared__ __align__(16) unsigned char lds_dyn[];
    unsigned char *lds_q = lds_dyn;
    bf16_t *t1_lds = (bf16_t *)(lds_dyn + kLdsQ);
    uint32_t *lds_cnt = (uint32_t *)lds_dyn;   // the q region, once q is in registers
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int yb = blockIdx.y * kGroupRows;   // first row of this block of rows

    // ---- row groups: up to 4 consecutive rows sharing a page-table row (a
    // run of equal page-table rows is cut into groups from its start).  This
    // workgroup scores the groups whose first row lies in its block of 4
    // rows: one group when requests' rows come in aligned fours, up to four.
    // One round of loads: lane l reads the page-table row of row yb+3-l (run
    // starts), lanes 0..6 the page-table rows and bounds of rows yb..yb+6
    // (group extents).
    const int back = yb + kGroupRows - 1 - lane;
    const int fwd = yb + lane;
    const bool fwd_ok = lane < 2 * kGroupRows - 1 && fwd < a.rows;
    const int v_back = (back >= 0 && back < a.rows) ? a.row_pt[back] : 0;
    const int v_fwd = fwd_ok ? a.row_pt[fwd] : 0;
    int v_bnd = fwd_ok ? a.row_bound[fwd] : 0;
    // q and w of the block's rows depend on nothing else: their loads go out
    // right behind the planning loads (q reaches LDS once the first group is
    // known to lie in the block).  Loads complete in order, so the planning
    // loads must be issued first for the planning to wait on them alone.
    __builtin_amdgcn_sched_barrier(0);
    // (piece c of every thread belongs to block row c / 4: rows past the last
    // are not loaded, so a block of one or two rows reads only their q and the
    // page-table load behind it returns sooner)
    static_assert(kScoreThreads * 4 == kHeads * kDim / 8, "four pieces per thread per row");
    const int rows_blk = min(a.rows - yb, kGroupRows);
    u32x4_t qt_blk[kBlockPieces];
#pragma unroll
    for (int c = 0; c < kBlockPieces; ++c) {
        const int ci = threadIdx.x + c * kScoreThreads;   // piece index: row, head, piece
        if ((c >> 2) < rows_blk)
            qt_blk[c] = *(gptr<u32x4_t>)(a.q + ((int64_t)(yb + (c >> 2)) * kHeads + ((ci >> 4) & 63)) * kDim +
                                         8 * (ci & 15));
    }
    // halved w of block row `wave` as linear_u takes it (heads 16 hb + 4 (lane / 16) + jj)
    f32x4_t wq_blk[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
        wq_blk[hb] = *(gptr<f32x4_t>)(a.w + (int64_t)min(yb + wave, a.rows - 1) * kHeads + 16 * hb + 4 * (lane >> 4)) * 0.5f;
    __builtin_amdgcn_sched_barrier(0);
    v_bnd = v_bnd < 0 ? 0 : (v_bnd > a.max_bound ? a.max_bound : v_bnd);
    // row `back` starts a run when it is row 0 or differs from row back-1
    // (lane 63 does not see its predecessor and never claims a start)
    const int v_prev = __shfl_down(v_back, 1);
    const uint64_t starts =
        __ballot(back == 0 || (back > 0 && back < a.rows && lane < 63 && v_prev != v_back));
    // No run start among rows yb-59 .. yb: row yb's run reaches back past
    // row yb-60 (lane 63), so walk back 64 rows per round.  Only block rows
    // whose window holds no start take this value.
    int rs_far = 0;
    if ((starts >> (kGroupRows - 1)) == 0) {
        const int pr_far = __builtin_amdgcn_readlane(v_back, kGroupRows - 1);   // row yb
        for (int base = yb - 60; base > 0; base -= 64) {
            const int idx = base - 1 - lane;
            const uint64_t m2 = __ballot(idx < 0 || a.row_pt[idx < 0 ? 0 : idx] != pr_far);
            if (m2) { rs_far = base - (__ffsll((unsigned long long)m2) - 1); break; }
        }
    }
    // The group led by block row bi, if any, with its row count and the
    // largest bound among its rows.
    const int c0 = blockIdx.x * a.chunk;
    auto group_at = [&](int bi, int &rg, int &gmax) {
        const int r0 = yb + bi;
        if (r0 >= a.rows) return false;
        const uint64_t m = starts >> (kGroupRows - 1 - bi);
        const int rs = m ? r0 - (__ffsll((unsigned long long)m) - 1) : rs_far;
        if ((r0 - rs) % kGroupRows != 0) return false;   // not the first row of a group
        const int pr0 = __builtin_amdgcn_readlane(v_fwd, bi);
        const uint64_t same = __ballot(fwd_ok && v_fwd == pr0) >> bi;
        rg = min(__ffsll((unsigned long long)~same) - 1, kGroupRows);
        gmax = 0;
        for (int j = 0; j < rg; ++j) gmax = max(gmax, __builtin_amdgcn_readlane(v_bnd, bi + j));
        return c0 < gmax;
    };
    // the chunk's page ids of a group, one per lane (a chunk spans at most 64
    // pages); a 16-key group picks its page with a lane read, so the loop
    // never waits on a scalar load.  Out-of-range ids become -1 (their keys
    // score NaN).
    auto load_pages = [&](int bi, int c1, int ln) {
        const int pr0 = __builtin_amdgcn_readlane(v_fwd, bi);
        const bool pt_ok = pr0 >= 0 && pr0 < a.pt_rows;
        const int npg = (c1 - c0 + kPage - 1) / kPage;
        const int32_t *pt = a.page_table + (int64_t)(pt_ok ? pr0 : 0) * a.pt_stride + c0 / kPage;
        return (pt_ok && ln < npg) ? pt[ln] : -1;
    };
    int bi_first = kGroupRows, rg_first = 0, gmax_first = 0;
    for (int bi = 0; bi < kGroupRows; ++bi) {
        int rg, gmax;
        if (group_at(bi, rg, gmax)) { bi_first = bi; rg_first = rg; gmax_first = gmax; break; }
    }
    if (bi_first == kGroupRows) return;
    // the first group's page ids go out before anything waits: page table ->
    // keys is the longest chain of dependent loads in the set-up
    const int v_pages_first = load_pages(bi_first, min(c0 + a.chunk, gmax_first), lane);
    // q staged with the block serves the first group when its rows lie in the block
    const bool staged_first = bi_first + rg_first <= kGroupRows;
    if (staged_first) {
#pragma unroll
        for (int c = 0; c < kBlockPieces; ++c) {
            const int ci = threadIdx.x + c * kScoreThreads;
            if ((c >> 2) < rows_blk) *(u32x4_t *)(lds_q + q_lds_off(ci >> 10, (ci >> 4) & 63, ci & 15)) = qt_blk[c];
        }
        lds_barrier();   // (the page ids may still be in flight)
        // the first group's linear term while the page ids are in flight:
        // block row `wave` is row wave - bi_first of the group
        const int ur = wave - bi_first;
        if (ur >= 0 && ur < rg_first) linear_u(lds_q, bi_first, ur, wq_blk, t1_lds, lane);
    }

    for (int bi = bi_first; bi < kGroupRows; ++bi) {
        int rg, gmax;
        if (bi == bi_first) { rg = rg_first; gmax = gmax_first; }
        else if (!group_at(bi, rg, gmax)) continue;
        const int r0 = yb + bi;
        const int c1 = min(c0 + a.chunk, gmax);
        if (bi != bi_first) lds_barrier();   // the previous group's write-out is done with LDS
        // the thread index passes through an empty asm per group: what the
        // group's code derives from it (LDS and key offsets) is recomputed in
        // each group instead of being kept live across all of them
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));

        // ---- wave roles: wave w takes page w of every block of four pages
        // of the chunk (4 consecutive 16-key groups), for all of the group's
        // rows
        const int nrows = rg;
        WaveJob job;
        job.tid = tid;
        job.lane = tid & 63;
        job.c0 = c0;
        job.chunk = a.chunk;
        job.row0 = r0;
#pragma unroll
        for (int r = 0; r < kGroupRows; ++r) job.bnd[r] = r < nrows ? __builtin_amdgcn_readlane(v_bnd, bi + r) : 0;
        const int myend = min(c1, max(max(job.bnd[0], job.bnd[1]), max(job.bnd[2], job.bnd[3])));
        job.gbase = c0 / kKeysPerMfma + 4 * wave;
        // groups of the chunk below the last bound, counted from the wave's
        // first: whole blocks of 16 give the wave 4 each, the last partial
        // block up to 4
        const int rem = (myend + kKeysPerMfma - 1) / kKeysPerMfma - job.gbase;
        job.n_my = rem > 0 ? 4 * (rem >> 4) + min(rem & 15, 4) : 0;
        const int v = bi == bi_first ? v_pages_first : load_pages(bi, c1, job.lane);
        job.vpage = (v >= 0 && v < a.num_pages) ? v : -1;
        const bool staged = bi == bi_first && staged_first;
        const int q_slot = staged ? bi : 0;
        switch (nrows) {   // every wave, also one with no groups (q staging)
        case 4: score_rows<4, kHist>(a, job, lds_q, t1_lds, lds_cnt, q_slot, staged, staged); break;
        case 3: score_rows<3, kHist>(a, job, lds_q, t1_lds, lds_cnt, q_slot, staged, staged); break;
        case 2: score_rows<2, kHist>(a, job, lds_q, t1_lds, lds_cnt, q_slot, staged, staged); break;
        default:
            if (job.n_my >= kDeepRingGroups) score_rows<1, kHist>(a, job, lds_q, t1_lds, lds_cnt, q_slot, staged, staged);
            else score_rows<1, kHist, 4>(a, job, lds_q, t1_lds, lds_cnt, q_slot, staged, staged);
            break;
        }

        // ---- add the chunk's first-digit counts to the row totals: wave r
        // sums row r's counters (lane = digit) into copy (workgroup % 16)
        if (kHist) {
            lds_barrier();
            const int hr = tid >> 6;   // row slot; lane = digit
            if (hr < rg) {
                uint32_t c = 0;
#pragma unroll
                for (int w = 0; w < kScoreThreads / 64; ++w) {
                    const u32x4_t v = *(const u32x4_t *)(lds_cnt + ((w * kGroupRows + hr) * kBins1 + job.lane) * kCntCopies);
                    c += v[0] + v[1] + v[2] + v[3];
                }
                if (c) atomicAdd(a.hist1 + ((int64_t)(r0 + hr) * kHist1Slots + blockIdx.x % kHist1Slots) * kBins1 + job.lane, c);
            }
        }
    }
}

// ===========================================================================
// One-row launches (a single query row: decode with no speculative rows).
// One row's q is 64 registers, so the wave fits in half the register file
// and each SIMD runs two waves: 8 waves per workgroup, wave w taking page w
// of every block of 8 pages of the chunk.  The loop is straight-line: while
// one wave converts keys and runs its epilogue, the other wave of the SIMD
// issues MFMAs and key loads.  The row needs no planning of row groups: its
// page-table row and bound are two scalar loads.
constexpr int kRowThreads = 512;
constexpr int kRowWaves = kRowThreads / 64;
constexpr int kRowRingPages = 1;                 // pages of keys in flight per wave
constexpr int kRowRing = 4 * kRowRingPages;      // 16-key groups in flight per wave
constexpr int kLdsQRow = kHeads * kDim * 2;      // 16 KB: q of the row, then the counters
constexpr int kHistLdsRow = kRowWaves * kBins1 * kCntCopies;
static_assert(kHistLdsRow * 4 <= kLdsQRow, "the counters reuse the q region");

template <bool kHist>
__global__ __launch_bounds__(kRowThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void score_row_kernel(ScoreArgs a) {
    extern __shared__ __align__(16) unsigned char lds_dyn[];
    unsigned char *lds_q = lds_dyn;
    bf16_t *t1_lds = (bf16_t *)(lds_dyn + kLdsQRow);
    uint32_t *lds_cnt = (uint32_t *)lds_dyn;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kig = lane & 15;
    const int lrow = lane >> 4;
    const uint32_t koff = (uint32_t)(kig * kDim + lrow * 32);

    // page-table row and bound first (the page ids wait on them), then q
    // (two 16-byte pieces per thread) and the weights, which wait on nothing
    const int pr = a.row_pt[0];
    int bnd = a.row_bound[0];
    __builtin_amdgcn_sched_barrier(0);
    constexpr int kPieces = kHeads * kDim / 8 / kRowThreads;
    static_assert(kPieces * kRowThreads * 8 == kHeads * kDim, "whole pieces per thread");
    u32x4_t qt[kPieces];
#pragma unroll
    for (int c = 0; c < kPieces; ++c) {
        const int ci = tid + c * kRowThreads;   // piece index: head ci / 16, piece ci % 16
        qt[c] = *(gptr<u32x4_t>)(a.q + (ci >> 4) * kDim + 8 * (ci & 15));
    }
    // weights (halved) of the D rows a lane holds: heads 16*hb + 4*(lane/16) + jj
    f32x4_t wv[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) wv[hb] = *(gptr<f32x4_t>)(a.w + 16 * hb + 4 * lrow) * 0.5f;

    __builtin_amdgcn_sched_barrier(0);
    bnd = bnd < 0 ? 0 : (bnd > a.max_bound ? a.max_bound : bnd);
    const int c0 = blockIdx.x * a.chunk;
    if (c0 >= bnd) return;   // (uniform over the workgroup)
    const int c1 = min(c0 + a.chunk, bnd);
    const int gc0 = c0 / kKeysPerMfma;
    int vpage;
    {
        const bool pt_ok = pr >= 0 && pr < a.pt_rows;
        const int npg = (c1 - c0 + kPage - 1) / kPage;
        const int32_t *pt = a.page_table + (int64_t)(pt_ok ? pr : 0) * a.pt_stride + c0 / kPage;
        const int v = (pt_ok && lane < npg) ? pt[lane] : -1;
        vpage = (v >= 0 && v < a.num_pages) ? v : -1;
    }
    // the wave's groups: its i-th is gbase + 32 * (i / 4) + i % 4, groups
    // below the chunk's end: 4 per whole block of 32, up to 4 of the last
    const int gbase = gc0 + 4 * wave;
    const int rem = (c1 + kKeysPerMfma - 1) / kKeysPerMfma - gbase;
    const int n_my = rem > 0 ? 4 * (rem >> 5) + min(rem & 31, 4) : 0;
    auto group = [&](int i) { return gbase + 32 * (i >> 2) + (i & 3); };
    // loads past the wave's last group re-read that group (no branch)
    auto load_group = [&](int i, KeyGroup &kg) {
        const int ic = max(min(i, n_my - 1), 0);
        const int g = group(ic);
        const int page = __builtin_amdgcn_readlane(vpage, (g - gc0) >> 2);
        kg.ok = page >= 0;
        const int64_t key0 = (int64_t)(kg.ok ? page : 0) * kPage + (g & 3) * kKeysPerMfma;
        gptr<uint8_t> kbase = scalar_ptr(a.k8 + key0 * kDim);
        gptr<float> sbase = scalar_ptr(a.kscale + key0);
        kg.lo = *(gptr<u32x4_t>)(kbase + koff);
        kg.hi = *(gptr<u32x4_t>)(kbase + koff + 16);
        kg.scale = sbase[kig];
    };
    KeyGroup kb[kRowRing];
#pragma unroll
    for (int p = 0; p < kRowRing; ++p) load_group(p, kb[p]);

    // q to LDS; the last wave builds the linear term's A operand (as in
    // score_rows, with one row: A row 4p holds part p of u) before its own q
    // read-back; then q goes back in MFMA A-operand order into AGPRs
#pragma unroll
    for (int c = 0; c < kPieces; ++c) {
        const int ci = tid + c * kRowThreads;
        *(u32x4_t *)(lds_q + q_lds_off(0, ci >> 4, ci & 15)) = qt[c];
    }
    lds_barrier();
    if (wave == kRowWaves - 1) linear_u(lds_q, 0, 0, wv, t1_lds, lane);
    bf16x8_t qa[4][4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qa[hb][ks] = *(const bf16x8_t *)(lds_q + q_lds_off(0, 16 * hb + kig, 4 * lrow + ks));
    lds_barrier();   // q in LDS is read and u is written
    bf16x8_t t1a[4];
    {
        const bool t1_row = (kig >> 2) < 3 && (kig & 3) == 0;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8_t v = *(const bf16x8_t *)(t1_lds + (ks * 64 + lane) * 8);
            t1a[ks] = t1_row ? v : bf16x8_t{};
        }
    }
    if (kHist) {   // the q region becomes the counters
        u32x4_t *c4 = (u32x4_t *)lds_cnt;
        const uint32_t z = (uint32_t)tid >> 16;   // 0, built here rather than kept live
        for (int i = tid; i < kHistLdsRow / 4; i += kRowThreads) c4[i] = u32x4_t{z, z, z, z};
        lds_barrier();
    }
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) asm volatile("" : "+a"(qa[hb][ks]));

    const int nrec = min(bnd - c0, a.chunk) * 4;   // the row's keys [c0, bound) of the chunk, in bytes
    const __amdgpu_buffer_rsrc_t out_row = __builtin_amdgcn_make_buffer_rsrc((void *)(a.scores + c0), 0, nrec, kBufferFlags);
    float P[4];
    float sv = 0.0f;   // lane l: scale of key l of the page being scored
    // one pass over the ring per kRowRingPages pages; the last pass stops
    // after the wave's last page
    for (int i0 = 0; i0 < n_my; i0 += kRowRing) {
#pragma unroll
        for (int pg = 0; pg < kRowRingPages; ++pg) {
            const int ip = i0 + 4 * pg;   // the page's first group (wave's index)
            if (pg > 0 && ip >= n_my) break;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                KeyGroup &kg = kb[4 * pg + p];
                bf16x8_t kv[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const u32x4_t &src = ks < 2 ? kg.lo : kg.hi;
                    kv[ks] = e4m3x8_to_bf16(src[(ks & 1) * 2], src[(ks & 1) * 2 + 1]);
                }
                sv = lrow == p ? (kg.ok ? kg.scale : __builtin_nanf("")) : sv;
                load_group(ip + p + kRowRing, kg);
                f32x4_t t1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) t1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t1a[ks], kv[ks], t1, 0, 0, 0);
                f32x4_t acc[4];
#pragma unroll
                for (int hb = 0; hb < 4; ++hb) acc[hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                    for (int hb = 0; hb < 4; ++hb)
                        acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[hb][ks], kv[ks], acc[hb], 0, 0, 0);
                // sum_h w_h max(d_h, 0) = u . k + sum_h (w_h / 2) |d_h| (the
                // epilogue of score_rows); lane l's 16 heads of key l % 16
                float part = t1[0];
#pragma unroll
                for (int hb = 0; hb < 4; ++hb)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) part = fmaf(wv[hb][jj], fabsf(acc[hb][jj]), part);
                P[p] = part;
                // groups stay in order: the other wave of the SIMD fills the
                // gaps (letting the compiler interleave groups cost ~0.5 us
                // per launch)
                __builtin_amdgcn_sched_barrier(0);
            }
            // the page's scores: lane l holds key l of the page; keys past the
            // bound or the wave's groups fall outside the buffer and are dropped
            const float out = reduce4(P[0], P[1], P[2], P[3]) * sv;
            const int s = group(ip) * kKeysPerMfma + lane;
            const bool in_job = ip + lrow < n_my;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(out), out_row, in_job ? (s - c0) * 4 : nrec, 0, kScoreStorePolicy);
            if (kHist) {
                const uint32_t d = radix_key(out) >> kDigit1Shift;
                atomicAdd(lds_cnt + (wave * kBins1 + d) * kCntCopies + lane % kCntCopies, (in_job && s < bnd) ? 1u : 0u);
            }
        }
    }
    if (kHist) {   // the row's counts (lane = digit) summed over the waves by the first wave
        lds_barrier();
        if (wave == 0) {
            uint32_t c = 0;
#pragma unroll
            for (int w = 0; w < kRowWaves; ++w) {
                const u32x4_t v4 = *(const u32x4_t *)(lds_cnt + (w * kBins1 + lane) * kCntCopies);
                c += v4[0] + v4[1] + v4[2] + v4[3];
            }
            if (c) atomicAdd(a.hist1 + (blockIdx.x % kHist1Slots) * kBins1 + lane, c);
        }
    }
}

hipError_t launch_score(const ScoreArgs &a, hipStream_t st) {
    if (a.max_bound <= 0) return hipSuccess;
    const int nchunks = (a.max_bound + a.chunk - 1) / a.chunk;
    dim3 grid(nchunks, (a.rows + kGroupRows - 1) / kGroupRows);
    if (a.rows == 1) {
        const size_t lds = (size_t)kLdsQRow + kLdsT1;
        if (a.hist1)
            hipLaunchKernelGGL(score_row_kernel<true>, grid, dim3(kRowThreads), lds, st, a);
        else
            hipLaunchKernelGGL(score_row_kernel<false>, grid, dim3(kRowThreads), lds, st, a);
        return hipGetLastError();
    }
    const size_t lds = (size_t)kLdsQ + kLdsT1;
    if (a.hist1)
        hipLaunchKernelGGL(score_kernel<true>, grid, dim3(kScoreThreads), lds, st, a);
    else
        hipLaunchKernelGGL(score_kernel<false>, grid, dim3(kScoreThreads), lds, st, a);
    return hipGetLastError();
}

}  // namespace fp8idx
