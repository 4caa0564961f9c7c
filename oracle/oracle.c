/*
 * Plain CPU oracle for the paged FP8-E4M3 decode indexer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code, header or table with the HIP library.
 *
 * What it computes (the indexer launch of the sglang pull request page
 * "sgl-project/sglang#48224", sgl-amd-mono #86 commit body, Motivation: every
 * cached key of each row is scored, then each row's exact top-k is selected):
 *
 *   for row r and logical key s < bound[r]:
 *     p = page_table[row_pt[r]][s / 64], o = s % 64
 *     d_h   = sum_{i<128} q[r][h][i] * dec(k8[p][o][i])          (fp64, i order)
 *     score = scale[p][o] * sum_{h<64} w[r][h] * max(d_h, 0)
 *     bnd   = scale[p][o] * sum_{h<64} |w[r][h]| * |d_h|          (tolerance scale)
 *
 * Keys at or past a row's bound are not scored (same page, #86 commit 2: the
 * store's mask drops keys at or past the row's bound, so the bound is
 * exclusive).  Top-k: descending by value, ties to the lower key index, NaN
 * below every number, -0 equal to +0; the first min(k, bound) of that order,
 * padded with -1.  The selection is a plain full sort (qsort) of all
 * (value, index) pairs.
 *
 * Plain C, fp64, one thread, no intrinsics.  Build: gcc -O2 -fPIC -shared
 * (no -ffast-math, so no floating-point reassociation).
 *
 * Return codes: 0 ok, -1 invalid argument, -2 page id / page-table row out of
 * range (nothing is read out of bounds).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_H 64
#define ORC_D 128
#define ORC_PAGE 64

/* OCP 8-bit floating point, E4M3 ("FN": no infinities, S.1111.111 is NaN):
 * exponent bias 7; exponent field 0 is subnormal (m/8) * 2^-6. */
static double e4m3_value(uint8_t b)
{
    int s = (b >> 7) & 1;
    int e = (b >> 3) & 15;
    int m = b & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
static double bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_e4m3_decode(uint8_t b) { return e4m3_value(b); }
double oracle_bf16_decode(uint16_t h) { return bf16_value(h); }

/* One key-row: score and tolerance scale.  qd is the row's q decoded to
 * fp64, [64][128].  Returns 0, or -2 if the page lookup is out of range. */
static int score_one(const double *qd, const float *w_r, const uint8_t *k8,
                     const float *kscale, int num_pages, const int32_t *pt_row,
                     int64_t s, double *score, double *bnd)
{
    int32_t page = pt_row[s / ORC_PAGE];
    int64_t slot = s % ORC_PAGE;
    const uint8_t *key;
    double kv[ORC_D];
    double c, acc = 0.0, accb = 0.0;
    int h, i;
    if (page < 0 || page >= num_pages)
        return -2;
    key = k8 + ((int64_t)page * ORC_PAGE + slot) * ORC_D;
    c = (double)kscale[(int64_t)page * ORC_PAGE + slot];
    for (i = 0; i < ORC_D; ++i)
        kv[i] = e4m3_value(key[i]);
    for (h = 0; h < ORC_H; ++h) {
        double d = 0.0;
        for (i = 0; i < ORC_D; ++i)
            d += qd[h * ORC_D + i] * kv[i];
        acc += (double)w_r[h] * (d > 0.0 ? d : 0.0);
        accb += fabs((double)w_r[h]) * fabs(d);
    }
    *score = c * acc;
    *bnd = c * accb;
    return 0;
}

static void decode_q_row(const uint16_t *q_r, double *qd)
{
    int i;
    for (i = 0; i < ORC_H * ORC_D; ++i)
        qd[i] = bf16_value(q_r[i]);
}

/* Scores of row r for keys s in [s0, s1) (clipped to the row's bound).
 * q: [rows][64][128] bf16 bits; w: [rows][64]; k8: [num_pages][64][128];
 * kscale: [num_pages][64]; page_table: [pt_rows][pt_stride].
 * out_score[s - s0], out_bnd[s - s0] (out_bnd may be NULL). */
int oracle_score_range(int r, int64_t s0, int64_t s1,
                       const uint16_t *q, const float *w,
                       const uint8_t *k8, const float *kscale, int num_pages,
                       const int32_t *page_table, int pt_rows, int pt_stride,
                       const int32_t *row_pt, const int32_t *row_bound,
                       double *out_score, double *out_bnd)
{
    double qd[ORC_H * ORC_D];
    int64_t s, b;
    int pr;
    if (!q || !w || !k8 || !kscale || !page_table || !row_pt || !row_bound || !out_score)
        return -1;
    if (r < 0 || s0 < 0 || s1 < s0)
        return -1;
    pr = row_pt[r];
    if (pr < 0 || pr >= pt_rows)
        return -2;
    b = row_bound[r];
    if (b > (int64_t)pt_stride * ORC_PAGE)
        return -1;
    if (s1 > b)
        s1 = b;
    decode_q_row(q + (int64_t)r * ORC_H * ORC_D, qd);
    for (s = s0; s < s1; ++s) {
        double sc, bd;
        int rc = score_one(qd, w + (int64_t)r * ORC_H, k8,
                           kscale, num_pages, page_table + (int64_t)pr * pt_stride, s,
                           &sc, &bd);
        if (rc)
            return rc;
        out_score[s - s0] = sc;
        if (out_bnd)
            out_bnd[s - s0] = bd;
    }
    return 0;
}

/* Scores for an explicit list of (row, key) samples. */
int oracle_score_samples(int64_t nsamp, const int32_t *samp_row, const int64_t *samp_key,
                         const uint16_t *q, const float *w,
                         const uint8_t *k8, const float *kscale, int num_pages,
                         const int32_t *page_table, int pt_rows, int pt_stride,
                         const int32_t *row_pt, const int32_t *row_bound,
                         double *out_score, double *out_bnd)
{
    double qd[ORC_H * ORC_D];
    int64_t i;
    for (i = 0; i < nsamp; ++i) {
        int r = samp_row[i];
        int64_t s = samp_key[i];
        int pr = row_pt[r];
        double sc, bd;
        int rc;
        if (pr < 0 || pr >= pt_rows)
            return -2;
        if (s < 0 || s >= row_bound[r] || s >= (int64_t)pt_stride * ORC_PAGE)
            return -1;
        decode_q_row(q + (int64_t)r * ORC_H * ORC_D, qd);
        rc = score_one(qd, w + (int64_t)r * ORC_H, k8, kscale,
                       num_pages, page_table + (int64_t)pr * pt_stride, s, &sc, &bd);
        if (rc)
            return rc;
        out_score[i] = sc;
        if (out_bnd)
            out_bnd[i] = bd;
    }
    return 0;
}

/* ---------------------------------------------------------------- top-k */

typedef struct {
    double v;
    int64_t i;
} orc_pair;

/* "a comes before b": larger value first; NaN after every number; equal
 * values (and -0 vs +0, and NaN vs NaN) by lower index. */
static int before(const orc_pair *a, const orc_pair *b)
{
    int an = isnan(a->v), bn = isnan(b->v);
    if (an != bn)
        return bn;                  /* the number comes first */
    if (!an && a->v != b->v)
        return a->v > b->v;
    return a->i < b->i;
}

static int cmp_pair(const void *pa, const void *pb)
{
    const orc_pair *a = (const orc_pair *)pa, *b = (const orc_pair *)pb;
    if (before(a, b))
        return -1;
    if (before(b, a))
        return 1;
    return 0;
}

static int topk_pairs(orc_pair *pr, int64_t n, int k, int32_t *out)
{
    int64_t i, take;
    qsort(pr, (size_t)n, sizeof *pr, cmp_pair);
    take = n < k ? n : k;
    for (i = 0; i < take; ++i)
        out[i] = (int32_t)pr[i].i;
    for (i = take; i < k; ++i)
        out[i] = -1;
    return 0;
}

/* Top-k of scores[0..n) given as fp32 (the GPU's own scores). */
int oracle_topk_f32(const float *scores, int64_t n, int k, int32_t *out)
{
    orc_pair *pr;
    int64_t i;
    if (n < 0 || k < 1 || !out || (n > 0 && !scores))
        return -1;
    pr = (orc_pair *)malloc(sizeof(orc_pair) * (size_t)(n > 0 ? n : 1));
    if (!pr)
        return -1;
    for (i = 0; i < n; ++i) {
        pr[i].v = (double)scores[i];
        pr[i].i = i;
    }
    topk_pairs(pr, n, k, out);
    free(pr);
    return 0;
}

/* Top-k of scores[0..n) given in fp64 (the oracle's own scores). */
int oracle_topk_f64(const double *scores, int64_t n, int k, int32_t *out)
{
    orc_pair *pr;
    int64_t i;
    if (n < 0 || k < 1 || !out || (n > 0 && !scores))
        return -1;
    pr = (orc_pair *)malloc(sizeof(orc_pair) * (size_t)(n > 0 ? n : 1));
    if (!pr)
        return -1;
    for (i = 0; i < n; ++i) {
        pr[i].v = scores[i];
        pr[i].i = i;
    }
    topk_pairs(pr, n, k, out);
    free(pr);
    return 0;
}

/* ---- New-key write (the same page, Modifications row 2 and the Reviewer
 * notes "New keys": a key the launch itself writes is taken from its row's
 * index_k8 pair, the key's E4M3 codes and scale, by every row of the request
 * in the launch).  The pages give no quantization rule; the plain per-key one
 * is taken: the scale is the key's largest magnitude over the largest finite
 * E4M3 value, and each element divided by the scale goes to the nearest E4M3
 * value.
 *
 *   amax  = max_i |k[i]|                 (the bf16 key decoded exactly)
 *   scale = amax / 448                   (one fp32 division, round to nearest even)
 *   x_i   = k[i] / scale                 (one fp32 division each)
 *   code_i = the finite E4M3 code nearest to x_i; a tie goes to the code with
 *            an even mantissa (its lowest bit clear); beyond 448 in magnitude
 *            the code of +-448; the sign bit is x_i's sign bit (so -0 -> 0x80)
 *   a key with amax == 0 gets scale 1 and all codes 0x00.
 *
 * The nearest code is found by looking at every non-negative finite code, as
 * the definition reads (no bit manipulation).  Inputs are finite. */
static uint8_t e4m3_nearest(float x)
{
    double a = fabs((double)x);
    int best = 0, c;
    double bestd = a;                 /* distance to code 0x00 (zero) */
    for (c = 1; c <= 0x7E; ++c) {     /* every positive finite code */
        double d = fabs(e4m3_value((uint8_t)c) - a);
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) != 0)) {
            best = c;
            bestd = d;
        }
    }
    if (a > 448.0)
        best = 0x7E;
    return (uint8_t)(best | (signbit(x) ? 0x80 : 0));
}

int oracle_quantize_key(const uint16_t *k_bf16, uint8_t *codes, float *scale_out)
{
    float kv[ORC_D], amax = 0.0f, scale;
    int i;
    if (!k_bf16 || !codes || !scale_out)
        return -1;
    for (i = 0; i < ORC_D; ++i) {
        kv[i] = (float)bf16_value(k_bf16[i]);
        if (fabsf(kv[i]) > amax)
            amax = fabsf(kv[i]);
    }
    if (amax == 0.0f) {
        memset(codes, 0, ORC_D);
        *scale_out = 1.0f;
        return 0;
    }
    scale = amax / 448.0f;
    for (i = 0; i < ORC_D; ++i) {
        volatile float x = kv[i] / scale;   /* an fp32 quotient, not a wider one */
        codes[i] = e4m3_nearest(x);
    }
    *scale_out = scale;
    return 0;
}

uint8_t oracle_e4m3_nearest(float x) { return e4m3_nearest(x); }

/*
 * Sparse attention over a row's selected keys: the step the indexer feeds
 * (the sglang pull request page, #86 commit body, Motivation: the launch
 * picks each row's exact top-2048 keys for the attention that follows; the
 * GLM-5.2 release test-suite page runs that step with an MLA sparse
 * attention backend over a DeepSeek-style latent cache).  The pages give
 * neither the formula nor the shapes; the reading used here is multi-head
 * latent attention in its absorbed decode form:
 *
 *   every key position s of a request holds one latent vector c_s of 576
 *   bf16 values (512 latent + 64 rotary), paged like the index keys (the
 *   same page table: page page_table[row_pt][s / 64], slot s % 64);
 *   row r has 16 query heads q_h of 576 bf16 values;
 *   for the row's selected positions J (its index list, -1 entries skipped;
 *   a position outside [0, max_bound) or on a page id out of range is
 *   skipped too):
 *     l_j   = sm_scale * sum_{i<576} q_h[i] * c_j[i]
 *     out_h = sum_j exp(l_j) * c_j[0..512) / sum_j exp(l_j)
 *     lse_h = log(sum_j exp(l_j))
 *   with no selected position: out_h = 0, lse_h = -inf.
 *
 * fp64 throughout; exp and log of fp64, the sums in index-list order, the
 * maximum logit subtracted before exp (exp(l - m) / sum exp(l - m) is the
 * same quotient).
 */
#define ORC_AH 16
#define ORC_AD 576
#define ORC_AV 512

int oracle_sparse_attention(const uint16_t *q_r, const uint16_t *kv, int num_pages,
                            const int32_t *page_table, int pt_rows, int pt_stride, int row_pt,
                            const int32_t *sel_r, int topk, int max_bound, double sm_scale,
                            double *out_r, double *lse_r)
{
    if (!q_r || !kv || !page_table || !sel_r || !out_r || !lse_r || topk < 0 || num_pages < 1)
        return -1;
    /* the selected positions' cache rows (NULL: skipped) */
    const uint16_t **rowp = (const uint16_t **)malloc(sizeof(const uint16_t *) * (size_t)(topk > 0 ? topk : 1));
    double *lg = (double *)malloc(sizeof(double) * (size_t)(topk > 0 ? topk : 1));
    if (!rowp || !lg) {
        free(rowp);
        free(lg);
        return -1;
    }
    for (int j = 0; j < topk; ++j) {
        const int32_t s = sel_r[j];
        rowp[j] = NULL;
        if (s < 0 || s >= max_bound || row_pt < 0 || row_pt >= pt_rows || s / ORC_PAGE >= pt_stride)
            continue;
        const int32_t pg = page_table[(int64_t)row_pt * pt_stride + s / ORC_PAGE];
        if (pg < 0 || pg >= num_pages)
            continue;
        rowp[j] = kv + ((int64_t)pg * ORC_PAGE + s % ORC_PAGE) * ORC_AD;
    }
    for (int h = 0; h < ORC_AH; ++h) {
        const uint16_t *q = q_r + (int64_t)h * ORC_AD;
        double m = -INFINITY;
        for (int j = 0; j < topk; ++j) {
            if (!rowp[j])
                continue;
            double d = 0.0;
            for (int i = 0; i < ORC_AD; ++i)
                d += bf16_value(q[i]) * bf16_value(rowp[j][i]);
            lg[j] = sm_scale * d;
            if (lg[j] > m)
                m = lg[j];
        }
        double *o = out_r + (int64_t)h * ORC_AV;
        for (int i = 0; i < ORC_AV; ++i)
            o[i] = 0.0;
        if (m == -INFINITY) {   /* nothing selected */
            lse_r[h] = -INFINITY;
            continue;
        }
        double den = 0.0;
        for (int j = 0; j < topk; ++j) {
            if (!rowp[j])
                continue;
            const double p = exp(lg[j] - m);
            den += p;
            for (int i = 0; i < ORC_AV; ++i)
                o[i] += p * bf16_value(rowp[j][i]);
        }
        for (int i = 0; i < ORC_AV; ++i)
            o[i] /= den;
        lse_r[h] = m + log(den);
    }
    free(rowp);
    free(lg);
    return 0;
}
