/*
 * nabla_oracle.c -- plain, slow CPU oracle for the NABLA hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls this file.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  It shares no source, header, table or helper with the HIP path.
 *
 * What it follows (page titles and sections, no code copied):
 *   [nabla]  FastVideo API page "nabla": source of nablaT_v2 (map estimation,
 *            map binarization, BlockMask creation), NablaAttentionImpl.forward
 *            and the NablaAttentionMetadata fields (sta_mask, P).
 *   [NABLA]  "NABLA: Neighborhood Adaptive Block-Level Attention" summary page,
 *            Technical Summary > Methodology (token reordering, pooling,
 *            reduced attention, CDF thresholding, expansion, STA union).
 *
 * Precision readings (the pages run the estimator in the input dtype and do
 * not fix rounding; these are the readings this oracle and the GPU both take):
 *   - pool:    fp32, sequential over the 64 tokens of a block, then * 2^-6.
 *   - score:   fp32, acc = fma(qa[d], ka[d], acc) for d = 0..D-1 from +0,
 *              then IEEE division by fl32(sqrt(D)); -0 is canonicalised to +0.
 *   - exp:     nexp(), a Cody-Waite reduction plus a degree-7 Taylor polynomial
 *              in Horner form with fused multiply-adds; 0 below x = -64.
 *   - softmax: e_j = nexp(s_j - max s); Z is the exact sum of e_j in 2^-48
 *              fixed point, rounded to fp32; p_j = e_j / Z (IEEE fp32 division).
 *   - CDF:     cumulative sums of p in 2^-48 fixed point (exact integer sums),
 *              compared with fl32(1 - thr) rounded up to the same grid.
 *   - order:   ascending by (s_j, j); among equal scores the lower block index
 *              comes first, i.e. is dropped first.
 *   - the last block in sorted order (the row's arg-max) is always kept.
 *   - attention: fp64 dense softmax over every key, with disallowed 64x64
 *              blocks at -inf; scale 1/sqrt(D).
 *   - training pass: lse (natural log) and the gradients dq, dk, dv of that
 *              dense masked softmax attention, fp64.
 *   - quantized variant (the sibling "sla" page, SageSLA forward): INT8 q and
 *              k - mean(k) per block, FP8 e4m3 v per channel (see O12 below),
 *              fp64 attention with FP8 weights e4m3(448 exp(z - rowmax)).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_BLK 64           /* tokens per block: 64 ([nabla] nablaT_v2, map estimation) */
#define ORC_TILE 8           /* spatial tile edge P = 8: a 1 x 8 x 8 tile holds one block */
#define ORC_FIX_BITS 48      /* fixed-point grid of the softmax sums: 2^-48 */

/* ------------------------------------------------------------------------- */
/* threads                                                                    */
/* ------------------------------------------------------------------------- */
void orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------- */
/* O1: fractal flattening ([NABLA] Methodology, "Token Reordering")           */
/* The tokens of each 8 x 8 spatial patch of one frame become a contiguous    */
/* run of 64; frames stay in time order; patches go in raster order (patch    */
/* row, patch column); inside a patch, raster order (row, column).            */
/* Grids whose H or W is not a multiple of 8 are padded to whole patches       */
/* (ceil(H/8) x ceil(W/8) per frame, the sibling "video_sparse_attn" page's    */
/* variable block sizes): the padded positions exist in the fractal order,    */
/* hold zeros, and are not tokens (see orc_token_valid).                       */
/* ------------------------------------------------------------------------- */
static int orc_tiles(int n) { return (n + ORC_TILE - 1) / ORC_TILE; }

int64_t orc_fractal_index(int t, int y, int x, int H, int W) {
    int Ht = orc_tiles(H), Wt = orc_tiles(W);
    int64_t tile = ((int64_t)t * Ht + y / ORC_TILE) * Wt + x / ORC_TILE;
    return tile * ORC_BLK + (y % ORC_TILE) * ORC_TILE + (x % ORC_TILE);
}

/* Sequence length of the fractal order of a T x H x W grid (padded to whole patches). */
int64_t orc_fractal_len(int T, int H, int W) {
    return (int64_t)T * orc_tiles(H) * orc_tiles(W) * ORC_BLK;
}

/* 1 if fractal position s (within one sequence) is a token of the T x H x W grid, 0 if it
 * is padding of a partial patch. */
int orc_token_valid(int64_t s, int H, int W) {
    int Ht = orc_tiles(H), Wt = orc_tiles(W);
    int64_t blk = s / ORC_BLK;
    int r = (int)(s % ORC_BLK);
    int ht = (int)((blk / Wt) % Ht), wt = (int)(blk % Wt);
    return ht * ORC_TILE + r / ORC_TILE < H && wt * ORC_TILE + r % ORC_TILE < W;
}

/* x, y: one token row = heads*D elements of esize bytes; S = orc_fractal_len(T, H, W).
 * inverse == 0: x natural [B][T][H][W][row] -> y fractal [B][S][row] (padding rows 0)
 * inverse != 0: x fractal -> y natural (padding rows are not read). */
void orc_fractal_permute(const uint8_t *x, uint8_t *y, int64_t esize, int B, int T, int H,
                         int W, int heads, int D, int inverse) {
    int64_t row = (int64_t)heads * D * esize;
    int64_t S = orc_fractal_len(T, H, W);
    if (!inverse) memset(y, 0, (size_t)(B * S * row));
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < T; ++t)
            for (int yy = 0; yy < H; ++yy)
                for (int xx = 0; xx < W; ++xx) {
                    int64_t nat = (((int64_t)b * T + t) * H + yy) * W + xx;
                    int64_t fra = (int64_t)b * S + orc_fractal_index(t, yy, xx, H, W);
                    if (!inverse)
                        memcpy(y + fra * row, x + nat * row, (size_t)row);
                    else
                        memcpy(y + nat * row, x + fra * row, (size_t)row);
                }
}

/* ------------------------------------------------------------------------- */
/* O2: STA block mask ([nabla] NablaAttentionMetadata.sta_mask, "precomputed  */
/* once per run"; [NABLA] Methodology, "Hybrid Integration with STA").         */
/* Reading: blocks i, j (tile coordinates (t, ht, wt)) are neighbours when    */
/* |dt| <= wt, |dh| <= wh and |dw| <= ww; the window is clipped at borders.   */
/* ------------------------------------------------------------------------- */
void orc_sta_mask(uint8_t *sta, int Tt, int Ht, int Wt, int win_t, int win_h, int win_w) {
    int64_t nb = (int64_t)Tt * Ht * Wt;
    for (int64_t i = 0; i < nb; ++i) {
        int ti = (int)(i / ((int64_t)Ht * Wt)), hi = (int)((i / Wt) % Ht), wi = (int)(i % Wt);
        for (int64_t j = 0; j < nb; ++j) {
            int tj = (int)(j / ((int64_t)Ht * Wt)), hj = (int)((j / Wt) % Ht), wj = (int)(j % Wt);
            sta[i * nb + j] = (uint8_t)(abs(ti - tj) <= win_t && abs(hi - hj) <= win_h &&
                                        abs(wi - wj) <= win_w);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* O3: block mean-pool ([nabla] nablaT_v2, map estimation: reshape to blocks  */
/* of 64 tokens and take the mean).  x [B][S][heads][D] (fp32 values; bf16    */
/* inputs are widened exactly by the caller) -> xa [B][heads][nb][D].         */
/* ------------------------------------------------------------------------- */
void orc_pool(const float *x, float *xa, int B, int S, int heads, int D) {
    int nb = S / ORC_BLK;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < heads; ++h)
            for (int i = 0; i < nb; ++i)
                for (int d = 0; d < D; ++d) {
                    float acc = 0.0f;
                    for (int r = 0; r < ORC_BLK; ++r) {
                        int64_t tok = (int64_t)b * S + (int64_t)i * ORC_BLK + r;
                        acc = acc + x[(tok * heads + h) * D + d];
                    }
                    xa[(((int64_t)b * heads + h) * nb + i) * D + d] = acc * 0.015625f;
                }
}

/* O3 on a padded grid: the mean over the block's tokens only (padding excluded): the sum
 * over its valid positions in fractal order, then an IEEE division by their count (for a
 * full block the count is 64 and this equals orc_pool).  x [B][S][heads][D] with
 * S = orc_fractal_len(T, H, W). */
void orc_pool_grid(const float *x, float *xa, int B, int T, int H, int W, int heads, int D) {
    int64_t S = orc_fractal_len(T, H, W);
    int nb = (int)(S / ORC_BLK);
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < heads; ++h)
            for (int i = 0; i < nb; ++i)
                for (int d = 0; d < D; ++d) {
                    float acc = 0.0f;
                    int cnt = 0;
                    for (int r = 0; r < ORC_BLK; ++r) {
                        int64_t s_ = (int64_t)i * ORC_BLK + r;
                        if (!orc_token_valid(s_, H, W)) continue;
                        int64_t tok = (int64_t)b * S + s_;
                        acc = acc + x[(tok * heads + h) * D + d];
                        ++cnt;
                    }
                    xa[(((int64_t)b * heads + h) * nb + i) * D + d] = acc / (float)cnt;
                }
}

/* ------------------------------------------------------------------------- */
/* O4: block scores ([nabla] nablaT_v2: qa @ ka^T, divided by sqrt(D)).       */
/* qa, ka [B][heads][nb][D] -> s [B][heads][nb][nb].                          */
/* ------------------------------------------------------------------------- */
static float orc_score_one(const float *a, const float *k, int D, float sqrt_d) {
    float acc = 0.0f;
    for (int d = 0; d < D; ++d) acc = fmaf(a[d], k[d], acc);
    float s = acc / sqrt_d;
    return s + 0.0f; /* -0 -> +0 */
}

void orc_scores(const float *qa, const float *ka, float *s, int B, int heads, int nb, int D) {
    float sqrt_d = (float)sqrt((double)D);
    int64_t rows = (int64_t)B * heads * nb;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t bh = r / nb;
        const float *a = qa + r * D;
        for (int j = 0; j < nb; ++j)
            s[r * nb + j] = orc_score_one(a, ka + (bh * nb + j) * D, D, sqrt_d);
    }
}

/* ------------------------------------------------------------------------- */
/* exp used by the softmax: Cody & Waite argument reduction                   */
/*   n = rint(x log2 e), r = (x - n ln2_hi) - n ln2_lo,                       */
/* then the Taylor series of e^r to degree 7 in Horner form (fused            */
/* multiply-add at every step), scaled by 2^n.  Valid for x <= 0; returns 0    */
/* for x < -64 (those weights fall below the 2^-48 grid anyway).              */
/* ------------------------------------------------------------------------- */
float orc_nexp(float x) {
    if (!(x >= -64.0f)) return 0.0f;
    const float log2e = 1.44269504088896341f;
    const float ln2_hi = 0.693145751953125f;      /* 15 significant bits: n*ln2_hi exact */
    const float ln2_lo = 1.42860682030941723e-6f; /* ln 2 - ln2_hi */
    float n = rintf(x * log2e);
    float r = fmaf(-n, ln2_hi, x);
    r = fmaf(-n, ln2_lo, r);
    /* e^r = sum_k r^k / k!, k = 0..7 */
    float p = 1.98412698412698413e-4f; /* 1/5040 */
    p = fmaf(p, r, 1.38888888888888889e-3f); /* 1/720 */
    p = fmaf(p, r, 8.33333333333333333e-3f); /* 1/120 */
    p = fmaf(p, r, 4.16666666666666667e-2f); /* 1/24 */
    p = fmaf(p, r, 1.66666666666666667e-1f); /* 1/6 */
    p = fmaf(p, r, 0.5f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    /* 2^n with n in [-93, 0]: a normal float built from its exponent field */
    int32_t bits = ((int32_t)n + 127) << 23;
    float two_n;
    memcpy(&two_n, &bits, sizeof two_n);
    return p * two_n;
}

void orc_nexp_vec(const float *x, float *y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = orc_nexp(x[i]);
}

/* ------------------------------------------------------------------------- */
/* O5: row softmax ([nabla] nablaT_v2: softmax over the last dimension).      */
/* e_j = nexp(s_j - m); Z = fl32(sum_j floor(e_j 2^48)) 2^-48; p_j = e_j / Z; */
/* P_j = floor(p_j 2^48) (the fixed-point weights the CDF adds up).            */
/* ------------------------------------------------------------------------- */
static int64_t orc_fix(float v) { /* floor(v * 2^48) for 0 <= v <= 1 */
    return (int64_t)ldexp((double)v, ORC_FIX_BITS);
}

void orc_softmax_row(const float *s, int nb, float *e, float *p, int64_t *P, double *Zout) {
    float m = s[0];
    for (int j = 1; j < nb; ++j)
        if (s[j] > m) m = s[j];
    int64_t ZE = 0;
    for (int j = 0; j < nb; ++j) {
        e[j] = orc_nexp(s[j] - m);
        ZE += orc_fix(e[j]);
    }
    float Z = (float)(double)ZE;
    Z = ldexpf(Z, -ORC_FIX_BITS);
    for (int j = 0; j < nb; ++j) {
        p[j] = e[j] / Z;
        P[j] = orc_fix(p[j]);
    }
    if (Zout) *Zout = (double)Z;
}

/* ------------------------------------------------------------------------- */
/* O6-O7: sort, cumulative sum, cut, un-sort ([nabla] nablaT_v2, map         */
/* binarization; [NABLA] Methodology, "CDF Thresholding").                    */
/* ------------------------------------------------------------------------- */
typedef struct { float s; int j; } orc_key;

static int orc_key_cmp(const void *a, const void *b) {
    const orc_key *x = (const orc_key *)a, *y = (const orc_key *)b;
    if (x->s < y->s) return -1;
    if (x->s > y->s) return 1;
    return (x->j > y->j) - (x->j < y->j);
}

/* The cut on the 2^-48 grid: ceil(fl32(1 - thr) * 2^48). */
int64_t orc_cut_fixed(double thr) {
    float cut = (float)(1.0 - thr);
    return (int64_t)ceil(ldexp((double)cut, ORC_FIX_BITS));
}

/* One row: kept[j] = 1 for kept blocks.  diag (optional, 3 int64):
 *   diag[0] = i0 (first kept position in sorted order),
 *   diag[1] = c_{i0-1} (0 when i0 == 0), diag[2] = c_{i0}, both on the 2^-48 grid. */
void orc_select_row(const float *s, int nb, double thr, uint8_t *kept, int64_t *diag) {
    float *e = (float *)malloc(sizeof(float) * (size_t)nb);
    float *p = (float *)malloc(sizeof(float) * (size_t)nb);
    int64_t *P = (int64_t *)malloc(sizeof(int64_t) * (size_t)nb);
    orc_key *key = (orc_key *)malloc(sizeof(orc_key) * (size_t)nb);
    uint8_t *ms = (uint8_t *)malloc((size_t)nb);
    orc_softmax_row(s, nb, e, p, P, NULL);
    /* vals, inds = map.sort(-1) */
    for (int j = 0; j < nb; ++j) { key[j].s = s[j]; key[j].j = j; }
    qsort(key, (size_t)nb, sizeof(orc_key), orc_key_cmp);
    /* cvals = cumsum(vals); mask = cvals >= 1 - thr */
    int64_t CUT = orc_cut_fixed(thr);
    int64_t c = 0, c_prev = 0, c_at = 0;
    int i0 = -1;
    for (int k = 0; k < nb; ++k) {
        int64_t before = c;
        c += P[key[k].j];
        ms[k] = (uint8_t)(c >= CUT);
        if (ms[k] && i0 < 0) { i0 = k; c_prev = before; c_at = c; }
    }
    /* the arg-max block is always kept (exact arithmetic gives c_last = 1) */
    if (!ms[nb - 1]) {
        ms[nb - 1] = 1;
        i0 = nb - 1;
        c_at = c;
        c_prev = c - P[key[nb - 1].j];
    }
    /* mask = mask.gather(-1, inds.argsort(-1)): back to block order */
    for (int k = 0; k < nb; ++k) kept[key[k].j] = ms[k];
    if (diag) { diag[0] = i0; diag[1] = c_prev; diag[2] = c_at; }
    free(e); free(p); free(P); free(key); free(ms);
}

/* ------------------------------------------------------------------------- */
/* O3-O9: the whole estimator.  q, k [B][S][heads][D] fp32 values.            */
/* sta [nb][nb] (NULL: STA off).  row_ids: the rows (b*heads + h)*nb + i to   */
/* evaluate (NULL: all rows, in order); output row r belongs to row_ids[r].   */
/*   kv_nb   [nrows]             number of kept blocks,                       */
/*   kv_inds [nrows][nb]         kept block indices ascending, then the       */
/*                               dropped ones ascending,                      */
/*   mnabla  [nrows][nb]         (optional) the mask before the STA union,    */
/*   diag    [nrows][3]          (optional) see orc_select_row.               */
/* Returns 0, or -1 on a bad argument.                                        */
/* ------------------------------------------------------------------------- */
/* gT, gH, gW: the latent grid of a padded layout (pooling over tokens only), or all 0 for
 * whole 64-token blocks. */
static int orc_block_mask_impl(const float *q, const float *k, int B, int S, int heads, int D,
                               int gT, int gH, int gW, const uint8_t *sta, double thr,
                               const int64_t *row_ids, int64_t nrows, int32_t *kv_nb,
                               int32_t *kv_inds, uint8_t *mnabla, int64_t *diag) {
    if (B <= 0 || heads <= 0 || D <= 0 || S <= 0 || S % ORC_BLK != 0) return -1;
    if (!(thr >= 0.0 && thr <= 1.0)) return -1;
    int nb = S / ORC_BLK;
    int64_t all = (int64_t)B * heads * nb;
    if (!row_ids) nrows = all;
    for (int64_t r = 0; r < nrows; ++r)
        if (row_ids && (row_ids[r] < 0 || row_ids[r] >= all)) return -1;
    int64_t nbd = (int64_t)B * heads * nb * D;
    float *qa = (float *)malloc(sizeof(float) * (size_t)nbd);
    float *ka = (float *)malloc(sizeof(float) * (size_t)nbd);
    if (gH > 0) {
        orc_pool_grid(q, qa, B, gT, gH, gW, heads, D);
        orc_pool_grid(k, ka, B, gT, gH, gW, heads, D);
    } else {
        orc_pool(q, qa, B, S, heads, D);
        orc_pool(k, ka, B, S, heads, D);
    }
    float sqrt_d = (float)sqrt((double)D);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t rr = 0; rr < nrows; ++rr) {
        int64_t id = row_ids ? row_ids[rr] : rr;
        int64_t bh = id / nb;
        int i = (int)(id % nb);
        float *srow = (float *)malloc(sizeof(float) * (size_t)nb);
        uint8_t *kept = (uint8_t *)malloc((size_t)nb);
        for (int j = 0; j < nb; ++j)
            srow[j] = orc_score_one(qa + id * D, ka + (bh * nb + j) * D, D, sqrt_d);
        orc_select_row(srow, nb, thr, kept, diag ? diag + rr * 3 : NULL);
        if (mnabla) memcpy(mnabla + rr * nb, kept, (size_t)nb);
        /* mask = logical_or(mask, sta) */
        if (sta)
            for (int j = 0; j < nb; ++j) kept[j] = (uint8_t)(kept[j] | (sta[(int64_t)i * nb + j] != 0));
        /* kv_nb = mask.sum(-1); kv_inds = mask.argsort(descending) */
        int n = 0;
        for (int j = 0; j < nb; ++j) n += kept[j];
        kv_nb[rr] = n;
        int32_t *row = kv_inds + rr * nb;
        int w = 0;
        for (int j = 0; j < nb; ++j)
            if (kept[j]) row[w++] = j;
        for (int j = 0; j < nb; ++j)
            if (!kept[j]) row[w++] = j;
        free(srow);
        free(kept);
    }
    free(qa);
    free(ka);
    return 0;
}

int orc_block_mask(const float *q, const float *k, int B, int S, int heads, int D,
                   const uint8_t *sta, double thr, const int64_t *row_ids, int64_t nrows,
                   int32_t *kv_nb, int32_t *kv_inds, uint8_t *mnabla, int64_t *diag) {
    return orc_block_mask_impl(q, k, B, S, heads, D, 0, 0, 0, sta, thr, row_ids, nrows, kv_nb,
                               kv_inds, mnabla, diag);
}

/* The estimator on the padded fractal layout of a T x H x W grid (S = orc_fractal_len). */
int orc_block_mask_grid(const float *q, const float *k, int B, int T, int H, int W, int heads,
                        int D, const uint8_t *sta, double thr, const int64_t *row_ids,
                        int64_t nrows, int32_t *kv_nb, int32_t *kv_inds, uint8_t *mnabla,
                        int64_t *diag) {
    if (T <= 0 || H <= 0 || W <= 0) return -1;
    return orc_block_mask_impl(q, k, B, (int)orc_fractal_len(T, H, W), heads, D, T, H, W, sta,
                               thr, row_ids, nrows, kv_nb, kv_inds, mnabla, diag);
}

/* ------------------------------------------------------------------------- */
/* O12: the top-k estimator variant ("sla" page, get_block_map: smooth-k,      */
/* mean-pooled q and k blocks, their dot products, the topk_ratio fraction of  */
/* key blocks with the largest scores per query block).  Readings:             */
/*   - blocks of 64 tokens for both q and k (the page's BLKQ = BLKK default);  */
/*   - smooth-k: km[d] = (sum_j ka_j[d], sequential in j, fp32) / nb (IEEE),   */
/*     ka'_j = ka_j - km; equal in exact arithmetic to pooling k - mean(k);    */
/*   - s_ij = sequential fma over d of qa_i[d] * ka'_j[d] from +0, no scale,   */
/*     -0 -> +0 (the page multiplies the pooled blocks, no softmax, no scale); */
/*   - k = min(nb, floor(ratio * nb)) with the product in double;             */
/*   - the k largest by (s_j, j): among equal scores the higher index wins     */
/*     (lower indices are dropped first, as in the CDF cut);                  */
/*   - optional STA union and ascending compaction as in orc_block_mask.       */
/* Selection is invariant to subtracting km in exact arithmetic (a per-row    */
/* constant); the step only changes rounding, so it is kept as the page has it.*/
/* ------------------------------------------------------------------------- */
int orc_topk_count(int nb, double ratio) {
    double x = ratio * (double)nb;
    int k = (int)x; /* truncation toward zero, x >= 0 */
    return k < nb ? k : nb;
}

static int orc_key_less(float sa, int ja, float sb, int jb) {
    return sa < sb || (sa == sb && ja < jb);
}

static int orc_block_mask_topk_impl(const float *q, const float *k, int B, int S, int heads,
                                    int D, int gT, int gH, int gW, const uint8_t *sta,
                                    double ratio, const int64_t *row_ids, int64_t nrows,
                                    int32_t *kv_nb, int32_t *kv_inds) {
    if (B <= 0 || heads <= 0 || D <= 0 || S <= 0 || S % ORC_BLK != 0) return -1;
    if (!(ratio >= 0.0 && ratio <= 1.0)) return -1;
    int nb = S / ORC_BLK;
    int64_t all = (int64_t)B * heads * nb;
    if (!row_ids) nrows = all;
    for (int64_t r = 0; r < nrows; ++r)
        if (row_ids && (row_ids[r] < 0 || row_ids[r] >= all)) return -1;
    int64_t nbd = (int64_t)B * heads * nb * D;
    float *qa = (float *)malloc(sizeof(float) * (size_t)nbd);
    float *ka = (float *)malloc(sizeof(float) * (size_t)nbd);
    if (gH > 0) {
        orc_pool_grid(q, qa, B, gT, gH, gW, heads, D);
        orc_pool_grid(k, ka, B, gT, gH, gW, heads, D);
    } else {
        orc_pool(q, qa, B, S, heads, D);
        orc_pool(k, ka, B, S, heads, D);
    }
    for (int64_t bh = 0; bh < (int64_t)B * heads; ++bh)
        for (int d = 0; d < D; ++d) {
            float sum = 0.0f;
            for (int j = 0; j < nb; ++j) sum = sum + ka[(bh * nb + j) * D + d];
            float km = sum / (float)nb;
            for (int j = 0; j < nb; ++j) ka[(bh * nb + j) * D + d] -= km;
        }
    const int kk = orc_topk_count(nb, ratio);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t rr = 0; rr < nrows; ++rr) {
        int64_t id = row_ids ? row_ids[rr] : rr;
        int64_t bh = id / nb;
        int i = (int)(id % nb);
        float *srow = (float *)malloc(sizeof(float) * (size_t)nb);
        uint8_t *kept = (uint8_t *)calloc((size_t)nb, 1);
        for (int j = 0; j < nb; ++j) {
            float acc = 0.0f;
            const float *a = qa + id * D, *b = ka + (bh * nb + j) * D;
            for (int d = 0; d < D; ++d) acc = fmaf(a[d], b[d], acc);
            srow[j] = acc + 0.0f;
        }
        /* j is among the k largest iff fewer than k keys are larger than (s_j, j) */
        for (int j = 0; j < nb; ++j) {
            int larger = 0;
            for (int t = 0; t < nb; ++t)
                if (orc_key_less(srow[j], j, srow[t], t)) ++larger;
            kept[j] = (uint8_t)(larger < kk);
        }
        if (sta)
            for (int j = 0; j < nb; ++j) kept[j] = (uint8_t)(kept[j] | (sta[(int64_t)i * nb + j] != 0));
        int n = 0;
        for (int j = 0; j < nb; ++j) n += kept[j];
        kv_nb[rr] = n;
        int32_t *row = kv_inds + rr * nb;
        int w = 0;
        for (int j = 0; j < nb; ++j)
            if (kept[j]) row[w++] = j;
        for (int j = 0; j < nb; ++j)
            if (!kept[j]) row[w++] = j;
        free(srow);
        free(kept);
    }
    free(qa);
    free(ka);
    return 0;
}

int orc_block_mask_topk(const float *q, const float *k, int B, int S, int heads, int D,
                        const uint8_t *sta, double ratio, const int64_t *row_ids, int64_t nrows,
                        int32_t *kv_nb, int32_t *kv_inds) {
    return orc_block_mask_topk_impl(q, k, B, S, heads, D, 0, 0, 0, sta, ratio, row_ids, nrows,
                                    kv_nb, kv_inds);
}

int orc_block_mask_topk_grid(const float *q, const float *k, int B, int T, int H, int W,
                             int heads, int D, const uint8_t *sta, double ratio,
                             const int64_t *row_ids, int64_t nrows, int32_t *kv_nb,
                             int32_t *kv_inds) {
    if (T <= 0 || H <= 0 || W <= 0) return -1;
    return orc_block_mask_topk_impl(q, k, B, (int)orc_fractal_len(T, H, W), heads, D, T, H, W,
                                    sta, ratio, row_ids, nrows, kv_nb, kv_inds);
}

/* ------------------------------------------------------------------------- */
/* O10: block-sparse attention as its plain dense definition                  */
/* ([nabla] NablaAttentionImpl.forward: flex attention with a block mask of   */
/* full 64 x 64 blocks; [NABLA] Methodology, "Expansion").  For each listed   */
/* q-block row id = (b*heads + h)*nb + i and each of its 64 query tokens:     */
/*   z_c = scale * <q, k_c> for every key c whose block is kept, -inf else;   */
/*   o = sum_c softmax(z)_c v_c, all in fp64.                                 */
/* o: [nrows][64][D] fp64.  A row whose list is empty yields 0.               */
/* ------------------------------------------------------------------------- */
/* gH, gW: the latent extents of a padded layout (padding positions are not keys), or 0. */
static int orc_attention_impl(const float *q, const float *k, const float *v, int B, int S,
                              int heads, int D, int gH, int gW, const int32_t *kv_nb,
                              const int32_t *kv_inds, double scale, const int64_t *row_ids,
                              int64_t nrows, double *o) {
    if (B <= 0 || heads <= 0 || D <= 0 || S <= 0 || S % ORC_BLK != 0) return -1;
    int nb = S / ORC_BLK;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t rr = 0; rr < nrows; ++rr) {
        int64_t id = row_ids[rr];
        if (id < 0 || id >= (int64_t)B * heads * nb) { bad = 1; continue; }
        int64_t b = id / ((int64_t)heads * nb);
        int h = (int)((id / nb) % heads);
        int i = (int)(id % nb);
        uint8_t *allowed = (uint8_t *)calloc((size_t)nb, 1);
        int n = kv_nb[id];
        if (n < 0 || n > nb) { bad = 1; free(allowed); continue; }
        for (int t = 0; t < n; ++t) {
            int j = kv_inds[id * nb + t];
            if (j < 0 || j >= nb) { bad = 1; break; }
            allowed[j] = 1;
        }
        double *z = (double *)malloc(sizeof(double) * (size_t)S);
        for (int r = 0; r < ORC_BLK; ++r) {
            int64_t qt = b * S + (int64_t)i * ORC_BLK + r;
            const float *qr = q + (qt * heads + h) * D;
            double *orow = o + (rr * ORC_BLK + r) * D;
            double zmax = -INFINITY;
            for (int64_t c = 0; c < S; ++c) {
                if (!allowed[c / ORC_BLK] || (gH > 0 && !orc_token_valid(c, gH, gW))) {
                    z[c] = -INFINITY;
                    continue;
                }
                const float *kc = k + ((b * S + c) * heads + h) * D;
                double acc = 0.0;
                for (int d = 0; d < D; ++d) acc += (double)qr[d] * (double)kc[d];
                z[c] = scale * acc;
                if (z[c] > zmax) zmax = z[c];
            }
            for (int d = 0; d < D; ++d) orow[d] = 0.0;
            if (zmax == -INFINITY) continue; /* empty list: O = 0 */
            double sum = 0.0;
            for (int64_t c = 0; c < S; ++c) {
                double w = (z[c] == -INFINITY) ? 0.0 : exp(z[c] - zmax);
                if (w == 0.0) continue;
                sum += w;
                const float *vc = v + ((b * S + c) * heads + h) * D;
                for (int d = 0; d < D; ++d) orow[d] += w * (double)vc[d];
            }
            for (int d = 0; d < D; ++d) orow[d] /= sum;
        }
        free(z);
        free(allowed);
    }
    return bad ? -1 : 0;
}

int orc_attention(const float *q, const float *k, const float *v, int B, int S, int heads,
                  int D, const int32_t *kv_nb, const int32_t *kv_inds, double scale,
                  const int64_t *row_ids, int64_t nrows, double *o) {
    return orc_attention_impl(q, k, v, B, S, heads, D, 0, 0, kv_nb, kv_inds, scale, row_ids,
                              nrows, o);
}

/* The attention on the padded fractal layout of a T x H x W grid: padding positions are
 * never keys (their query rows are computed too; the inverse permute drops them). */
int orc_attention_grid(const float *q, const float *k, const float *v, int B, int T, int H,
                       int W, int heads, int D, const int32_t *kv_nb, const int32_t *kv_inds,
                       double scale, const int64_t *row_ids, int64_t nrows, double *o) {
    if (T <= 0 || H <= 0 || W <= 0) return -1;
    return orc_attention_impl(q, k, v, B, (int)orc_fractal_len(T, H, W), heads, D, H, W, kv_nb,
                              kv_inds, scale, row_ids, nrows, o);
}

/* ------------------------------------------------------------------------- */
/* O11 attention statistics and gradients (the training pass)                 */
/* ------------------------------------------------------------------------- */
/*
 * The pages train with the same block-sparse attention ([NABLA] Results: the
 * training speed-up; [nabla] forward runs flex attention, whose backward is the
 * gradient of that dense masked softmax).  Per (b, h) and query row r, with A_r
 * the tokens of the blocks listed for r's block:
 *   z_rc  = scale * q_r . k_c            (c in A_r)
 *   lse_r = log sum_{c in A_r} exp(z_rc)            (natural log)
 *   P_rc  = exp(z_rc - lse_r),  o_r = sum_c P_rc v_c
 * and, for a given output gradient dO,
 *   dP_rc = dO_r . v_c,   Delta_r = sum_c P_rc dP_rc,   dZ_rc = P_rc (dP_rc - Delta_r)
 *   dq_r  = scale sum_c dZ_rc k_c
 *   dk_c  = scale sum_r dZ_rc q_r,   dv_c = sum_r P_rc dO_r   (r over rows with c in A_r).
 * fp64 throughout.  A row with no allowed key has lse = -inf and zero gradients.
 */

/* allowed[i * nb + j] = 1 iff block j is listed for query block i of slice (b, h) */
static int orc_slice_allowed(const int32_t *kv_nb, const int32_t *kv_inds, int64_t slice, int nb,
                             uint8_t *allowed) {
    memset(allowed, 0, (size_t)nb * nb);
    for (int i = 0; i < nb; ++i) {
        int64_t row = slice * nb + i;
        int n = kv_nb[row];
        if (n < 0 || n > nb) return -1;
        for (int t = 0; t < n; ++t) {
            int j = kv_inds[row * nb + t];
            if (j < 0 || j >= nb) return -1;
            allowed[(size_t)i * nb + j] = 1;
        }
    }
    return 0;
}

/* Row pass for query row r (token index within the sequence) of slice (b, h):
 * lse_r, Delta_r and (if dq_row) dq_r.  allowed_row = the row of `allowed` for
 * r's block; z is scratch of S doubles.  dout may be NULL (lse only). */
/* gH, gW: the latent extents of a padded layout (its padding positions are not keys), or 0. */
static void orc_row_pass(const float *q, const float *k, const float *v, const float *dout,
                         int64_t b, int h, int S, int heads, int D, int gH, int gW,
                         const uint8_t *allowed_row, double scale, int64_t r, double *z,
                         double *lse, double *delta, double *dq_row) {
    const int64_t tq = b * S + r;
    const float *qr = q + (tq * heads + h) * D;
    double zmax = -INFINITY;
    for (int64_t c = 0; c < S; ++c) {
        if (!allowed_row[c / ORC_BLK] || (gH > 0 && !orc_token_valid(c, gH, gW))) {
            z[c] = -INFINITY;
            continue;
        }
        const float *kc = k + ((b * S + c) * heads + h) * D;
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += (double)qr[d] * (double)kc[d];
        z[c] = scale * acc;
        if (z[c] > zmax) zmax = z[c];
    }
    if (dq_row) for (int d = 0; d < D; ++d) dq_row[d] = 0.0;
    if (zmax == -INFINITY) {
        *lse = -INFINITY;
        if (delta) *delta = 0.0;
        return;
    }
    double sum = 0.0;
    for (int64_t c = 0; c < S; ++c)
        if (z[c] != -INFINITY) sum += exp(z[c] - zmax);
    const double l = zmax + log(sum);
    *lse = l;
    if (!dout) return;
    const float *dor = dout + (tq * heads + h) * D;
    /* Delta_r = sum_c P_rc dP_rc; then dq_r = scale sum_c P_rc (dP_rc - Delta_r) k_c */
    double dl = 0.0;
    for (int64_t c = 0; c < S; ++c) {
        if (z[c] == -INFINITY) continue;
        const float *vc = v + ((b * S + c) * heads + h) * D;
        double dp = 0.0;
        for (int d = 0; d < D; ++d) dp += (double)dor[d] * (double)vc[d];
        dl += exp(z[c] - l) * dp;
    }
    *delta = dl;
    if (!dq_row) return;
    for (int64_t c = 0; c < S; ++c) {
        if (z[c] == -INFINITY) continue;
        const float *vc = v + ((b * S + c) * heads + h) * D;
        const float *kc = k + ((b * S + c) * heads + h) * D;
        double dp = 0.0;
        for (int d = 0; d < D; ++d) dp += (double)dor[d] * (double)vc[d];
        const double dz = exp(z[c] - l) * (dp - dl);
        for (int d = 0; d < D; ++d) dq_row[d] += scale * dz * (double)kc[d];
    }
}

/* lse of the 64 rows of each listed query block id = (b*heads + h)*nb + i: lse[rr*64 + r]. */
int orc_attention_lse(const float *q, const float *k, int B, int S, int heads, int D,
                      const int32_t *kv_nb, const int32_t *kv_inds, double scale,
                      const int64_t *row_ids, int64_t nrows, double *lse) {
    if (B <= 0 || heads <= 0 || D <= 0 || S <= 0 || S % ORC_BLK != 0) return -1;
    const int nb = S / ORC_BLK;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t rr = 0; rr < nrows; ++rr) {
        const int64_t id = row_ids[rr];
        if (id < 0 || id >= (int64_t)B * heads * nb) { bad = 1; continue; }
        const int64_t b = id / ((int64_t)heads * nb);
        const int h = (int)((id / nb) % heads);
        const int i = (int)(id % nb);
        uint8_t *allowed = (uint8_t *)calloc((size_t)nb, 1);
        double *z = (double *)malloc(sizeof(double) * (size_t)S);
        const int n = kv_nb[id];
        int ok = n >= 0 && n <= nb;
        for (int t = 0; ok && t < n; ++t) {
            const int j = kv_inds[id * nb + t];
            if (j < 0 || j >= nb) ok = 0; else allowed[j] = 1;
        }
        if (!ok) bad = 1;
        else
            for (int r = 0; r < ORC_BLK; ++r)
                orc_row_pass(q, k, NULL, NULL, b, h, S, heads, D, 0, 0, allowed, scale,
                             (int64_t)i * ORC_BLK + r, z, &lse[rr * ORC_BLK + r], NULL, NULL);
        free(z);
        free(allowed);
    }
    return bad ? -1 : 0;
}

/* dq of the 64 rows of each listed query block id: dq[(rr*64 + r)*D + d]. */
int orc_attention_dq(const float *q, const float *k, const float *v, const float *dout, int B,
                     int S, int heads, int D, const int32_t *kv_nb, const int32_t *kv_inds,
                     double scale, const int64_t *row_ids, int64_t nrows, double *dq) {
    if (B <= 0 || heads <= 0 || D <= 0 || S <= 0 || S % ORC_BLK != 0) return -1;
    const int nb = S / ORC_BLK;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t rr = 0; rr < nrows; ++rr) {
        const int64_t id = row_ids[rr];
        if (id < 0 || id >= (int64_t)B * heads * nb) { bad = 1; continue; }
        const int64_t b = id / ((int64_t)heads * nb);
        const int h = (int)((id / nb) % heads);
        const int i = (int)(id % nb);
        uint8_t *allowed = (uint8_t *)calloc((size_t)nb, 1);
        double *z = (double *)malloc(sizeof(double) * (size_t)S);
        const int n = kv_nb[id];
        int ok = n >= 0 && n <= nb;
        for (int t = 0; ok && t < n; ++t) {
            const int j = kv_inds[id * nb + t];
            if (j < 0 || j >= nb) ok = 0; else allowed[j] = 1;
        }
        if (!ok) bad = 1;
        else
            for (int r = 0; r < ORC_BLK; ++r) {
                double l, dl;
                orc_row_pass(q, k, v, dout, b, h, S, heads, D, 0, 0, allowed, scale,
                             (int64_t)i * ORC_BLK + r, z, &l, &dl, &dq[(rr * ORC_BLK + r) * D]);
            }
        free(z);
        free(allowed);
    }
    return bad ? -1 : 0;
}

/* Full training pass over every (b, h) slice: lse [B,heads,S]; dq, dk, dv [B,S,heads,D].
 * Row quantities first (parallel over rows), then dk and dv per key (parallel over keys):
 * key c of block j gathers from every row whose block lists j.  gH, gW: the latent extents
 * of a padded layout, whose padding positions are never keys (their dk and dv are 0; their
 * query rows are rows like any other), or 0. */
static int orc_attention_bwd_impl(const float *q, const float *k, const float *v,
                                  const float *dout, int B, int S, int heads, int D, int gH,
                                  int gW, const int32_t *kv_nb, const int32_t *kv_inds,
                                  double scale, double *lse, double *dq, double *dk,
                                  double *dv) {
    if (B <= 0 || heads <= 0 || D <= 0 || S <= 0 || S % ORC_BLK != 0) return -1;
    const int nb = S / ORC_BLK;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
    uint8_t *allowed = (uint8_t *)malloc((size_t)nb * nb);
    double *delta = (double *)malloc(sizeof(double) * (size_t)S);
    if (!allowed || !delta) { free(allowed); free(delta); return -1; }
    int bad = 0;
    for (int64_t b = 0; b < B && !bad; ++b)
        for (int h = 0; h < heads && !bad; ++h) {
            const int64_t slice = b * heads + h;
            if (orc_slice_allowed(kv_nb, kv_inds, slice, nb, allowed) != 0) { bad = 1; break; }
            double *lse_s = lse + slice * S;
#pragma omp parallel
            {
                double *z = (double *)malloc(sizeof(double) * (size_t)S);
#pragma omp for schedule(dynamic, 16)
                for (int64_t r = 0; r < S; ++r)
                    orc_row_pass(q, k, v, dout, b, h, S, heads, D, gH, gW,
                                 allowed + (size_t)(r / ORC_BLK) * nb, scale, r, z, &lse_s[r],
                                 &delta[r], dq + ((b * S + r) * heads + h) * D);
                free(z);
            }
#pragma omp parallel for schedule(dynamic, 16)
            for (int64_t c = 0; c < S; ++c) {
                const int j = (int)(c / ORC_BLK);
                const float *kc = k + ((b * S + c) * heads + h) * D;
                const float *vc = v + ((b * S + c) * heads + h) * D;
                double *dkc = dk + ((b * S + c) * heads + h) * D;
                double *dvc = dv + ((b * S + c) * heads + h) * D;
                for (int d = 0; d < D; ++d) { dkc[d] = 0.0; dvc[d] = 0.0; }
                if (gH > 0 && !orc_token_valid(c, gH, gW)) continue; /* not a key */
                for (int i = 0; i < nb; ++i) {
                    if (!allowed[(size_t)i * nb + j]) continue;
                    for (int rb = 0; rb < ORC_BLK; ++rb) {
                        const int64_t r = (int64_t)i * ORC_BLK + rb;
                        const float *qr = q + ((b * S + r) * heads + h) * D;
                        const float *dor = dout + ((b * S + r) * heads + h) * D;
                        double zz = 0.0, dp = 0.0;
                        for (int d = 0; d < D; ++d) {
                            zz += (double)qr[d] * (double)kc[d];
                            dp += (double)dor[d] * (double)vc[d];
                        }
                        const double p = exp(scale * zz - lse_s[r]);
                        const double dz = p * (dp - delta[r]);
                        for (int d = 0; d < D; ++d) {
                            dvc[d] += p * (double)dor[d];
                            dkc[d] += scale * dz * (double)qr[d];
                        }
                    }
                }
            }
        }
    free(allowed);
    free(delta);
    return bad ? -1 : 0;
}

int orc_attention_bwd(const float *q, const float *k, const float *v, const float *dout, int B,
                      int S, int heads, int D, const int32_t *kv_nb, const int32_t *kv_inds,
                      double scale, double *lse, double *dq, double *dk, double *dv) {
    return orc_attention_bwd_impl(q, k, v, dout, B, S, heads, D, 0, 0, kv_nb, kv_inds, scale,
                                  lse, dq, dk, dv);
}

/* dk and dv of the 64 keys of each listed key block id = (b*heads + h)*nb + j only
 * (dk[(cc*64 + c)*D + d], likewise dv), for checks at sizes where the full pass is too
 * slow.  The definition is the one above: key c of block j gathers, in ascending row
 * order, from every query row whose block lists j, with that row's lse and Delta taken
 * from its own full row pass.  Per (b, h) slice, only the rows of blocks that list one of
 * the requested key blocks get a row pass.  Returns 0, or -1 on a bad argument. */
int orc_attention_dkdv(const float *q, const float *k, const float *v, const float *dout,
                       int B, int S, int heads, int D, const int32_t *kv_nb,
                       const int32_t *kv_inds, double scale, const int64_t *col_ids,
                       int64_t ncols, double *dk, double *dv) {
    if (B <= 0 || heads <= 0 || D <= 0 || S <= 0 || S % ORC_BLK != 0 || ncols < 0) return -1;
    const int nb = S / ORC_BLK;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
    for (int64_t cc = 0; cc < ncols; ++cc)
        if (col_ids[cc] < 0 || col_ids[cc] >= (int64_t)B * heads * nb) return -1;
    uint8_t *allowed = (uint8_t *)malloc((size_t)nb * nb);
    uint8_t *need = (uint8_t *)malloc((size_t)nb);
    double *lse = (double *)malloc(sizeof(double) * (size_t)S);
    double *delta = (double *)malloc(sizeof(double) * (size_t)S);
    if (!allowed || !need || !lse || !delta) {
        free(allowed); free(need); free(lse); free(delta);
        return -1;
    }
    int bad = 0;
    for (int64_t slice = 0; slice < (int64_t)B * heads && !bad; ++slice) {
        int any = 0;
        for (int64_t cc = 0; cc < ncols; ++cc) any |= col_ids[cc] / nb == slice;
        if (!any) continue;
        const int64_t b = slice / heads;
        const int h = (int)(slice % heads);
        if (orc_slice_allowed(kv_nb, kv_inds, slice, nb, allowed) != 0) { bad = 1; break; }
        /* the query blocks whose lists hold a requested key block of this slice */
        memset(need, 0, (size_t)nb);
        for (int64_t cc = 0; cc < ncols; ++cc) {
            if (col_ids[cc] / nb != slice) continue;
            const int j = (int)(col_ids[cc] % nb);
            for (int i = 0; i < nb; ++i) need[i] |= allowed[(size_t)i * nb + j];
        }
#pragma omp parallel
        {
            double *z = (double *)malloc(sizeof(double) * (size_t)S);
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < S; ++r)
                if (need[r / ORC_BLK])
                    orc_row_pass(q, k, v, dout, b, h, S, heads, D, 0, 0,
                                 allowed + (size_t)(r / ORC_BLK) * nb, scale, r, z, &lse[r],
                                 &delta[r], NULL);
            free(z);
        }
#pragma omp parallel for schedule(dynamic, 4) collapse(2)
        for (int64_t cc = 0; cc < ncols; ++cc)
            for (int kc = 0; kc < ORC_BLK; ++kc) {
                if (col_ids[cc] / nb != slice) continue;
                const int j = (int)(col_ids[cc] % nb);
                const int64_t c = (int64_t)j * ORC_BLK + kc;
                const float *kr = k + ((b * S + c) * heads + h) * D;
                const float *vr = v + ((b * S + c) * heads + h) * D;
                double *dkc = dk + (cc * ORC_BLK + kc) * D;
                double *dvc = dv + (cc * ORC_BLK + kc) * D;
                for (int d = 0; d < D; ++d) { dkc[d] = 0.0; dvc[d] = 0.0; }
                for (int i = 0; i < nb; ++i) {
                    if (!allowed[(size_t)i * nb + j]) continue;
                    for (int rb = 0; rb < ORC_BLK; ++rb) {
                        const int64_t r = (int64_t)i * ORC_BLK + rb;
                        const float *qr = q + ((b * S + r) * heads + h) * D;
                        const float *dor = dout + ((b * S + r) * heads + h) * D;
                        double zz = 0.0, dp = 0.0;
                        for (int d = 0; d < D; ++d) {
                            zz += (double)qr[d] * (double)kr[d];
                            dp += (double)dor[d] * (double)vr[d];
                        }
                        const double p = exp(scale * zz - lse[r]);
                        const double dz = p * (dp - delta[r]);
                        for (int d = 0; d < D; ++d) {
                            dvc[d] += p * (double)dor[d];
                            dkc[d] += scale * dz * (double)qr[d];
                        }
                    }
                }
            }
    }
    free(allowed);
    free(need);
    free(lse);
    free(delta);
    return bad ? -1 : 0;
}

/* The training pass on the padded fractal layout of a T x H x W grid (the gradient of
 * orc_attention_grid's output): padding positions are never keys. */
int orc_attention_bwd_grid(const float *q, const float *k, const float *v, const float *dout,
                           int B, int T, int H, int W, int heads, int D, const int32_t *kv_nb,
                           const int32_t *kv_inds, double scale, double *lse, double *dq,
                           double *dk, double *dv) {
    if (T <= 0 || H <= 0 || W <= 0) return -1;
    return orc_attention_bwd_impl(q, k, v, dout, B, (int)orc_fractal_len(T, H, W), heads, D, H,
                                  W, kv_nb, kv_inds, scale, lse, dq, dk, dv);
}

/* ------------------------------------------------------------------------- */
/* O12 the quantized attention variant (the sibling "sla" backend page, the    */
/* SageSLA forward: Q and K to INT8 with one scale per block after the mean of */
/* K over the sequence is subtracted, V to FP8 e4m3 with one scale per channel */
/* (scale maximum 2.25, the value that page passes), then the block-sparse     */
/* attention on the codes).  Readings (the page shows the calls, not their     */
/* arithmetic):                                                               */
/*   - blocks: the 64-token blocks of the kv lists, for q and for k;          */
/*   - k_mean[d] = (sum over blocks j of bs_j[d]) / S, bs_j[d] the sum of the  */
/*     block's 64 tokens; both sums sequential in fp32 from +0, then an IEEE   */
/*     fp32 division by S; k' = k - k_mean (fp32);                            */
/*   - INT8: scale = amax / 127 (fp32), code = clamp(rint(x / scale), +-127)   */
/*     with an IEEE fp32 division and round-half-even; amax = 0 gives scale 0  */
/*     and codes 0;                                                           */
/*   - FP8 V: scale[d] = amax_d / 2.25 over all S tokens of channel d,        */
/*     code = e4m3(v / scale) (fp32 division, then round-to-nearest-even to   */
/*     OCP FP8 e4m3fn: 3 mantissa bits, bias 7, largest finite 448, no        */
/*     infinities);                                                           */
/*   - scores z = scale_sm * qs_i * ks_j * <q8, k8> (the integer dot exact);   */
/*   - P = exp(z - rowmax) is stored as e4m3(448 P) (the FP8 P of that page's  */
/*     "sv_f8" kernels, full range at P = 1); the row sum is taken over the    */
/*     same quantized weights, so o is a convex combination of the V codes:   */
/*     o[d] = vs[d] * sum_c p8_c v8_cd / sum_c p8_c, all in fp64;             */
/*   - padded layouts (Q9): padding positions are not tokens, so they are left */
/*     out of the k mean (divided by the token count) and of every maximum,  */
/*     their codes are 0, and they are never keys.                            */
/* ------------------------------------------------------------------------- */

/* OCP FP8 e4m3fn encoding of x, round to nearest, ties to the even code;     */
/* |x| > 448 saturates to 448 (never reached by the method's inputs); NaN     */
/* gives 0x7f with x's sign.                                                  */
uint8_t orc_fp8_e4m3(double x) {
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs(x);
    if (a != a) return sign | 0x7f;
    if (a >= 448.0) return sign | 0x7e;
    if (a < 0.015625) { /* below 2^-6: subnormal codes m * 2^-9, m = 0..8 (8 = 2^-6) */
        double m = rint(a * 512.0); /* exact scaling; rint rounds half to even */
        return sign | (uint8_t)m;
    }
    int e2;
    double fr = frexp(a, &e2);        /* a = fr * 2^e2, fr in [0.5, 1) */
    int e = e2 - 1;                   /* a = (2 fr) * 2^e, 2 fr in [1, 2) */
    double m = rint((2.0 * fr - 1.0) * 8.0); /* 3 mantissa bits, half to even */
    if (m == 8.0) { m = 0.0; e += 1; }
    int code = ((e + 7) << 3) | (int)m;
    if (code > 0x7e) code = 0x7e;
    return sign | (uint8_t)code;
}

double orc_fp8_e4m3_value(uint8_t c) {
    double s = (c & 0x80) ? -1.0 : 1.0;
    int E = (c >> 3) & 15, m = c & 7;
    if (E == 15 && m == 7) return NAN;
    if (E == 0) return s * ldexp((double)m, -9);
    return s * ldexp(1.0 + m / 8.0, E - 7);
}

void orc_fp8_e4m3_vec(const double *x, uint8_t *y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = orc_fp8_e4m3(x[i]);
}

static int8_t orc_int8_code(float x, float scale) {
    if (scale == 0.0f) return 0;
    float r = rintf(x / scale);
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    return (int8_t)r;
}

/* q8, k8: [B][heads][nb][64][D] int8; qs, ks: [B][heads][nb]; v8: [B][heads][nb][D][64]   */
/* e4m3 codes (each block transposed); vs, km: [B][heads][D]. */
/* gH, gW: the latent extents of a padded layout, whose padding positions are not tokens
 * (Q9): they are left out of the k mean (its divisor is the token count) and of every
 * maximum, and their codes are 0.  0: every position is a token. */
static int orc_quant_qkv_impl(const float *q, const float *k, const float *v, int B, int S,
                              int heads, int D, int gH, int gW, int8_t *q8, float *qs,
                              int8_t *k8, float *ks, uint8_t *v8, float *vs, float *km) {
    if (B <= 0 || heads <= 0 || D <= 0 || S <= 0 || S % ORC_BLK != 0) return -1;
    int nb = S / ORC_BLK;
    uint8_t *tok = (uint8_t *)malloc((size_t)S);
    if (!tok) return -1;
    int64_t ntok = 0;
    for (int64_t s = 0; s < S; ++s) {
        tok[s] = (uint8_t)(gH <= 0 || orc_token_valid(s, gH, gW));
        ntok += tok[s];
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < (int64_t)B * heads; ++bh) {
        int64_t b = bh / heads;
        int h = (int)(bh % heads);
        float *kmean = km + bh * D;
        /* k_mean: block sums over the tokens, then their sum, then / the token count */
        for (int d = 0; d < D; ++d) {
            float tot = 0.0f;
            for (int j = 0; j < nb; ++j) {
                float bs = 0.0f;
                for (int r = 0; r < ORC_BLK; ++r)
                    if (tok[(int64_t)j * ORC_BLK + r])
                        bs += k[((b * S + (int64_t)j * ORC_BLK + r) * heads + h) * D + d];
                tot += bs;
            }
            kmean[d] = tot / (float)ntok;
        }
        /* q and k' = k - k_mean per block */
        float *xs = (float *)malloc(sizeof(float) * ORC_BLK * D);
        for (int which = 0; which < 2; ++which) {
            const float *x = which == 0 ? q : k;
            int8_t *x8 = which == 0 ? q8 : k8;
            float *xsc = which == 0 ? qs : ks;
            for (int j = 0; j < nb; ++j) {
                float amax = 0.0f;
                for (int r = 0; r < ORC_BLK; ++r)
                    for (int d = 0; d < D; ++d) {
                        float val = 0.0f;
                        if (tok[(int64_t)j * ORC_BLK + r]) {
                            val = x[((b * S + (int64_t)j * ORC_BLK + r) * heads + h) * D + d];
                            if (which == 1) val = val - kmean[d];
                        }
                        xs[r * D + d] = val;
                        if (fabsf(val) > amax) amax = fabsf(val);
                    }
                float sc = amax / 127.0f;
                xsc[bh * nb + j] = sc;
                int8_t *dst = x8 + (bh * nb + j) * (int64_t)ORC_BLK * D;
                for (int e = 0; e < ORC_BLK * D; ++e) dst[e] = orc_int8_code(xs[e], sc);
            }
        }
        free(xs);
        /* v: per-channel scale over the whole sequence, then codes, blocks transposed */
        for (int d = 0; d < D; ++d) {
            float amax = 0.0f;
            for (int64_t s = 0; s < S; ++s) {
                if (!tok[s]) continue;
                float a = fabsf(v[((b * S + s) * heads + h) * D + d]);
                if (a > amax) amax = a;
            }
            float sc = amax / 2.25f;
            vs[bh * D + d] = sc;
            for (int64_t s = 0; s < S; ++s) {
                float val = tok[s] ? v[((b * S + s) * heads + h) * D + d] : 0.0f;
                float r = sc == 0.0f ? 0.0f : val / sc;
                int64_t j = s / ORC_BLK, key = s % ORC_BLK;
                v8[((bh * nb + j) * D + d) * ORC_BLK + key] = orc_fp8_e4m3((double)r);
            }
        }
    }
    free(tok);
    return 0;
}

int orc_quant_qkv(const float *q, const float *k, const float *v, int B, int S, int heads, int D,
                  int8_t *q8, float *qs, int8_t *k8, float *ks, uint8_t *v8, float *vs,
                  float *km) {
    return orc_quant_qkv_impl(q, k, v, B, S, heads, D, 0, 0, q8, qs, k8, ks, v8, vs, km);
}

/* The quantizer on the padded fractal layout of a T x H x W grid (Q9). */
int orc_quant_qkv_grid(const float *q, const float *k, const float *v, int B, int T, int H,
                       int W, int heads, int D, int8_t *q8, float *qs, int8_t *k8, float *ks,
                       uint8_t *v8, float *vs, float *km) {
    if (T <= 0 || H <= 0 || W <= 0) return -1;
    return orc_quant_qkv_impl(q, k, v, B, (int)orc_fractal_len(T, H, W), heads, D, H, W, q8,
                              qs, k8, ks, v8, vs, km);
}

/* The attention on the codes for the q-block rows row_ids (as orc_attention); o [nrows][64][D].
 * gH, gW: the latent extents of a padded layout (padding positions are never keys), or 0. */
static int orc_attention_q8_impl(const int8_t *q8, const float *qs, const int8_t *k8,
                                 const float *ks, const uint8_t *v8, const float *vs, int B,
                                 int S, int heads, int D, int gH, int gW, const int32_t *kv_nb,
                                 const int32_t *kv_inds, double scale, const int64_t *row_ids,
                                 int64_t nrows, double *o) {
    if (B <= 0 || heads <= 0 || D <= 0 || S <= 0 || S % ORC_BLK != 0) return -1;
    int nb = S / ORC_BLK;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
    double vdec[256];
    for (int c = 0; c < 256; ++c) vdec[c] = orc_fp8_e4m3_value((uint8_t)c);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t rr = 0; rr < nrows; ++rr) {
        int64_t id = row_ids[rr];
        if (id < 0 || id >= (int64_t)B * heads * nb) { bad = 1; continue; }
        int64_t bh = id / nb;
        int i = (int)(id % nb);
        int n = kv_nb[id];
        if (n < 0 || n > nb) { bad = 1; continue; }
        uint8_t *allowed = (uint8_t *)calloc((size_t)nb, 1);
        for (int t = 0; t < n; ++t) {
            int j = kv_inds[id * nb + t];
            if (j < 0 || j >= nb) { bad = 1; break; }
            allowed[j] = 1;
        }
        double *z = (double *)malloc(sizeof(double) * (size_t)S);
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
        for (int r = 0; r < ORC_BLK; ++r) {
            const int8_t *qr = q8 + ((bh * nb + i) * ORC_BLK + r) * (int64_t)D;
            double *orow = o + (rr * ORC_BLK + r) * D;
            double zmax = -INFINITY;
            for (int64_t c = 0; c < S; ++c) {
                int j = (int)(c / ORC_BLK);
                if (!allowed[j] || (gH > 0 && !orc_token_valid(c, gH, gW))) {
                    z[c] = -INFINITY;
                    continue;
                }
                const int8_t *kc = k8 + (bh * nb * ORC_BLK + c) * (int64_t)D;
                int64_t dot = 0;
                for (int d = 0; d < D; ++d) dot += (int64_t)qr[d] * (int64_t)kc[d];
                z[c] = scale * (double)qs[bh * nb + i] * (double)ks[bh * nb + j] * (double)dot;
                if (z[c] > zmax) zmax = z[c];
            }
            for (int d = 0; d < D; ++d) { orow[d] = 0.0; acc[d] = 0.0; }
            if (zmax == -INFINITY) continue; /* empty list: O = 0 */
            double wsum = 0.0;
            for (int64_t c = 0; c < S; ++c) {
                if (z[c] == -INFINITY) continue;
                double w = vdec[orc_fp8_e4m3(448.0 * exp(z[c] - zmax))];
                if (w == 0.0) continue;
                wsum += w;
                int64_t j = c / ORC_BLK, key = c % ORC_BLK;
                const uint8_t *vb = v8 + (bh * nb + j) * (int64_t)D * ORC_BLK;
                for (int d = 0; d < D; ++d) acc[d] += w * vdec[vb[d * ORC_BLK + key]];
            }
            for (int d = 0; d < D; ++d) orow[d] = (double)vs[bh * D + d] * acc[d] / wsum;
        }
        free(acc);
        free(z);
        free(allowed);
    }
    return bad ? -1 : 0;
}

int orc_attention_q8(const int8_t *q8, const float *qs, const int8_t *k8, const float *ks,
                     const uint8_t *v8, const float *vs, int B, int S, int heads, int D,
                     const int32_t *kv_nb, const int32_t *kv_inds, double scale,
                     const int64_t *row_ids, int64_t nrows, double *o) {
    return orc_attention_q8_impl(q8, qs, k8, ks, v8, vs, B, S, heads, D, 0, 0, kv_nb, kv_inds,
                                 scale, row_ids, nrows, o);
}

/* The attention on the codes of a padded T x H x W grid: padding positions are never keys. */
int orc_attention_q8_grid(const int8_t *q8, const float *qs, const int8_t *k8, const float *ks,
                          const uint8_t *v8, const float *vs, int B, int T, int H, int W,
                          int heads, int D, const int32_t *kv_nb, const int32_t *kv_inds,
                          double scale, const int64_t *row_ids, int64_t nrows, double *o) {
    if (T <= 0 || H <= 0 || W <= 0) return -1;
    return orc_attention_q8_impl(q8, qs, k8, ks, v8, vs, B, (int)orc_fractal_len(T, H, W), heads,
                                 D, H, W, kv_nb, kv_inds, scale, row_ids, nrows, o);
}
