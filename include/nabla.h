/*
 * nabla.h -- C ABI of libnabla.so, the MI355X (gfx950) NABLA hot path.
 *
 * NABLA ("NABLA: Neighborhood Adaptive Block-Level Attention"; FastVideo API
 * page "nabla") is data-dependent block-sparse attention for video DiTs:
 *   1. tokens are put in fractal order (each 8 x 8 spatial patch of a frame
 *      becomes a contiguous run of 64 tokens),
 *   2. an estimator mean-pools Q and K over 64-token blocks, softmaxes the
 *      scaled block-score map per row, keeps the top-mass blocks of each row
 *      through a sorted-CDF cut at 1 - thr, ORs in a static spatio-temporal
 *      window (STA) mask, and emits per-row kv block counts and indices,
 *   3. attention is computed over exactly those 64 x 64 blocks.
 *
 * Conventions for every call
 *   - Tensors are device pointers in HBM, contiguous, row-major, owned by the
 *     caller.  Inputs are never written.  The library allocates nothing: the
 *     calls that need scratch memory take a caller-owned workspace.
 *   - q, k, v, o use [B, S, heads, head_dim] (the layout of the pages'
 *     attention forward), S = T*H*W in fractal token order, S % 64 == 0.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on that stream and returns.  The library keeps no state
 *     between calls beyond a per-device cache of the GPU's compute-unit count,
 *     so calls on different streams (with separate workspaces) may run
 *     concurrently.
 *   - Every call validates its arguments on the host before any launch and
 *     returns a nabla_status; nothing is enqueued unless the result is
 *     NABLA_OK.  NABLA_ERR_HIP reports a failed launch (hipGetLastError).
 *   - dtype NABLA_BF16 (bfloat16) or NABLA_FP32; outputs of the attention
 *     have the input dtype.  Attention runs on bf16 MFMA with fp32
 *     accumulation (fp32 inputs are rounded to bf16, nearest-even, first).
 */
#ifndef NABLA_H
#define NABLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NABLA_OK = 0,
    NABLA_ERR_INVALID_ARG = 1, /* null pointer, bad shape, thr outside [0,1] or NaN */
    NABLA_ERR_UNSUPPORTED = 2, /* valid request this build does not implement */
    NABLA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
    NABLA_ERR_HIP = 4          /* a HIP launch failed */
} nabla_status;

typedef enum { NABLA_FP32 = 0, NABLA_BF16 = 1 } nabla_dtype;

/* Version of this ABI (incremented on any signature change). */
int nabla_abi_version(void);

/* Static description of a status code (never NULL). */
const char *nabla_status_string(nabla_status s);

/*
 * Fractal token reordering (NABLA summary page, Technical Summary >
 * Methodology, "Token Reordering"; the "nabla" page's forward expects q/k/v
 * "fractal-ordered by the model").
 *
 * With Ht = ceil(H/8), Wt = ceil(W/8) and S = T * Ht * Wt * 64:
 * inverse == 0: x is [B, T, H, W, heads, head_dim] (natural order), y is
 *   [B, S, heads, head_dim] with token (t, yy, xx) at
 *   s = ((t*Ht + yy/8) * Wt + xx/8) * 64 + (yy%8)*8 + xx%8:
 *   frames stay in time order, 8 x 8 patches in raster order, and the 64
 *   tokens of a patch in raster order; each 64-token block is one patch.
 *   When 8 does not divide H or W, the last patch row / column is partial
 *   (the sibling "video_sparse_attn" page's variable block sizes): its padding
 *   positions are written as 0 and are not tokens (S > T*H*W).
 * inverse != 0: the inverse (x fractal [B, S, ...], y natural), e.g. for O;
 *   padding positions are not read.
 * x and y must not overlap.  Errors: INVALID_ARG if a pointer is NULL or a
 * size is < 1; UNSUPPORTED if heads*head_dim*sizeof(dtype) is not a multiple
 * of 16 bytes or B * T * Ht * Wt exceeds 2^24 - 1 patches (one launch of
 * 256-lane workgroups, one per patch).
 */
nabla_status nabla_fractal_permute(const void *x, void *y, nabla_dtype dtype, int B, int T,
                                   int H, int W, int heads, int head_dim, int inverse,
                                   void *stream);

/*
 * STA block mask ("nabla" page, NablaAttentionMetadata.sta_mask: a block-level
 * window mask of S/64 x S/64, precomputed once per run; NABLA summary page,
 * Methodology, "Hybrid Integration with STA").
 *
 * sta[i*nb + j] = 1 when blocks i and j (tile coordinates (t, h, w), block
 * index i = (t*Ht + h)*Wt + w, nb = Tt*Ht*Wt) satisfy |dt| <= win_t,
 * |dh| <= win_h and |dw| <= win_w, else 0.  The window is clipped at the
 * borders.  sta: device buffer of nb*nb bytes.  Errors: INVALID_ARG for a NULL
 * pointer, a tile count < 1 or a negative window.
 */
nabla_status nabla_sta_mask(uint8_t *sta, int Tt, int Ht, int Wt, int win_t, int win_h,
                            int win_w, void *stream);

/* Bytes of workspace nabla_block_mask needs: pooled Q and K in fp32,
 * 2 * B * heads * (S/64) * head_dim * 4, and for rows of 513 to 2048 blocks the block scores
 * (B * heads * (S/64)^2 * 4; the selection then runs as a second launch).  0 if the sizes are
 * invalid. */
size_t nabla_block_mask_workspace(int B, int S, int heads, int head_dim);

/*
 * The NABLA block-mask estimator ("nabla" page, nablaT_v2: map estimation,
 * map binarization, BlockMask creation; NABLA summary page, Methodology,
 * "Adaptive Mask Construction" and "Hybrid Integration with STA").
 *
 * For every (b, head, query block i), with nb = S/64:
 *   qa_i = mean of the 64 query tokens of block i (fp32; likewise ka_j),
 *   s_ij = <qa_i, ka_j> / sqrt(head_dim)     (fp32, fixed reduction order),
 *   p_ij = softmax_j(s_ij),
 *   blocks sorted ascending by (s_ij, j); block j is kept when the
 *   cumulative p up to and including it is >= fl32(1 - thr); the row's
 *   largest block is always kept; finally kept |= sta[i][j].
 * The cumulative sums are exact on a 2^-48 grid, so the decision does not
 * depend on summation order.
 *
 * q, k:     [B, S, heads, head_dim] (bf16 or fp32), fractal order.
 * sta:      [nb, nb] uint8 (nonzero = in window), shared by all (b, head);
 *           NULL means no STA union.
 * thr:      kept probability mass, in [0, 1] (the pages' default is 0.9).
 * kv_nb:    out [B, heads, nb] int32, number of kept blocks of each row (>= 1).
 * kv_inds:  out [B, heads, nb, nb] int32; the first kv_nb entries of each row
 *           are the kept block indices in ascending order; the rest of the
 *           row is left untouched (unspecified).
 * ws:       device workspace of at least nabla_block_mask_workspace() bytes.
 * Errors: INVALID_ARG (NULL q/k/kv_nb/kv_inds, sizes < 1, S % 64 != 0, thr
 * NaN or outside [0,1]); UNSUPPORTED (head_dim not 64 or 128, nb > 4096, or
 * B * heads > 65535); WORKSPACE (ws NULL or ws_bytes too small).
 */
nabla_status nabla_block_mask(const void *q, const void *k, nabla_dtype dtype, int B, int S,
                              int heads, int head_dim, const uint8_t *sta, double thr,
                              int32_t *kv_nb, int32_t *kv_inds, void *ws, size_t ws_bytes,
                              void *stream);

/*
 * The top-k estimator variant (the sibling "sla" backend page, get_block_map:
 * smooth-k, mean-pooled q and k blocks, their dot products, and per query block
 * the topk_ratio fraction of key blocks with the largest scores), on 64-token
 * blocks, with the same list format and optional STA union as nabla_block_mask:
 *   qa_i, ka_j = block means (fp32, as nabla_block_mask);
 *   km = (sum over j of ka_j, sequential in j) / nb;  ka'_j = ka_j - km;
 *   s_ij = <qa_i, ka'_j> (sequential fma over d, no scale);
 *   k = min(nb, int(topk_ratio * nb)) (double product, truncated);
 *   block j is kept when it is among the k largest by (s_ij, j) (on equal scores
 *   the higher index wins), then kept |= sta[i][j].
 * Every row keeps exactly k blocks before the union (0 when k = 0: with no STA the
 * lists are empty and the attention gives o = 0 for them).
 * q, k, sta, kv_nb, kv_inds, ws: as for nabla_block_mask (same workspace size).
 * Errors: INVALID_ARG (NULL q/k/kv_nb/kv_inds, sizes < 1, S % 64 != 0, topk_ratio
 * NaN or outside [0, 1]); UNSUPPORTED (head_dim not 64 or 128, or nb > 2048);
 * WORKSPACE (ws NULL or ws_bytes too small).
 */
nabla_status nabla_block_mask_topk(const void *q, const void *k, nabla_dtype dtype, int B,
                                   int S, int heads, int head_dim, const uint8_t *sta,
                                   double topk_ratio, int32_t *kv_nb, int32_t *kv_inds, void *ws,
                                   size_t ws_bytes, void *stream);

/*
 * Either estimator on the fractal layout of a T x H x W latent grid whose H or W need
 * not be multiples of 8 (S = T * ceil(H/8) * ceil(W/8) * 64, as nabla_fractal_permute
 * writes it; the sibling "video_sparse_attn" page's variable block sizes): a block's
 * mean is taken over its tokens only (their sum in fractal order divided by their
 * count min(8, H - 8 ht) * min(8, W - 8 wt)); everything else is nabla_block_mask
 * (topk_ratio < 0; thr as there) or nabla_block_mask_topk (topk_ratio in [0, 1]; thr
 * not used).  On a grid of whole patches the lists equal those of the plain calls.
 * Workspace: nabla_block_mask_workspace(B, S, heads, head_dim).
 * Errors: those of the chosen estimator; INVALID_ARG also for T, H or W < 1 or a NaN
 * topk_ratio.
 */
nabla_status nabla_block_mask_grid(const void *q, const void *k, nabla_dtype dtype, int B,
                                   int T, int H, int W, int heads, int head_dim,
                                   const uint8_t *sta, double thr, double topk_ratio,
                                   int32_t *kv_nb, int32_t *kv_inds, void *ws, size_t ws_bytes,
                                   void *stream);

/*
 * Either estimator on q and k left in natural order, with the fractal permute folded into
 * the pooling's addressing (the "nabla" page's fractal flattening reorders tokens only, so
 * each 64-token block is read where the permute would take its rows from, in the same
 * order).  H and W must be multiples of 8 (whole patches); S = T * H * W.
 * q, k:     [B, T, H, W, heads, head_dim] (bf16 or fp32), natural order.
 * The block indices, lists, sta, thr / topk_ratio (as nabla_block_mask_grid) and the
 * workspace (nabla_block_mask_workspace(B, S, heads, head_dim)) are those of the fractal
 * layout: the lists are identical to nabla_block_mask_grid's on the permuted q and k.
 * Errors: those of nabla_block_mask_grid; UNSUPPORTED also for H or W not a multiple of 8,
 * 8 * W * heads * head_dim * element size >= 2^32, or more than 4096 blocks (S/64).
 */
nabla_status nabla_block_mask_natural(const void *q, const void *k, nabla_dtype dtype, int B,
                                      int T, int H, int W, int heads, int head_dim,
                                      const uint8_t *sta, double thr, double topk_ratio,
                                      int32_t *kv_nb, int32_t *kv_inds, void *ws,
                                      size_t ws_bytes, void *stream);

/*
 * Bytes of workspace nabla_sparse_attn_fwd needs for the same (B, S, heads) and tile
 * grid: 256 + 2 * round_up(4 * ngroups, 256), where ngroups = B * heads *
 * ceil(Tt/2) * Ht * ceil(Wt/2) (tile grid known) or B * heads * ceil(S/256)
 * (unknown grid).  0 if the sizes or the grid are invalid.
 */
size_t nabla_sparse_attn_workspace(int B, int S, int heads, int Tt, int Ht, int Wt);

/*
 * Block-sparse attention forward over the kept blocks ("nabla" page,
 * NablaAttentionImpl.forward: flex attention with a block mask of full
 * 64 x 64 blocks, no intra-block masking; NABLA summary page, Methodology,
 * "Expansion").
 *
 * For each (b, head, query block i) and each of its 64 query rows:
 *   o = softmax(scale * q K_J^T) V_J, J = the tokens of the blocks
 *   kv_inds[b, head, i, 0 .. kv_nb[b, head, i] - 1].
 * A row with kv_nb == 0 gets o = 0.  Non-causal only; one kv head per head.
 *
 * q, k, v:  [B, S, heads, head_dim] (bf16 or fp32), fractal order.
 * kv_nb, kv_inds: as produced by nabla_block_mask (or any lists with
 *           0 <= kv_nb <= nb and entries in [0, nb) without repeats, in any
 *           order; a repeated entry counts once).
 * scale:    softmax scale; <= 0 selects 1/sqrt(head_dim).
 * Tt, Ht, Wt: the tile grid of the blocks (the pages' visual_shape divided
 *           by (1, 8, 8)), Tt*Ht*Wt == S/64; it only decides which query
 *           blocks share K/V tiles on chip.  All three 0 = unknown (blocks
 *           are then grouped in runs of consecutive indices).
 * o:        out [B, S, heads, head_dim], same dtype as q; must not overlap inputs.
 * ws:       device workspace of at least nabla_sparse_attn_workspace() bytes
 *           (the call's work schedule; overwritten, no contents carried between
 *           calls).  Calls that share one workspace must be on one stream.
 * Errors: INVALID_ARG (NULL pointer, sizes < 1, S % 64 != 0, NaN scale, a
 * tile grid that does not multiply to S/64); UNSUPPORTED (head_dim not 64 or
 * 128, or S/64 > 4096); WORKSPACE (ws NULL or ws_bytes too small).  List
 * contents are not checked on the host; entries outside [0, nb) are clamped by
 * the kernel.
 */
nabla_status nabla_sparse_attn_fwd(const void *q, const void *k, const void *v,
                                   nabla_dtype dtype, int B, int S, int heads, int head_dim,
                                   const int32_t *kv_nb, const int32_t *kv_inds, float scale,
                                   int Tt, int Ht, int Wt, void *o, void *ws, size_t ws_bytes,
                                   void *stream);

/*
 * nabla_sparse_attn_fwd without allocation or a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  The call's only scratch memory, its work schedule, lives in a static
 * 1 MiB device array that the library holds on every GPU it runs on until the process ends
 * (its address is looked up once per device, on the first call there).  The call itself
 * allocates nothing.
 * Arguments, layouts, results and the other errors are those of nabla_sparse_attn_fwd; the
 * output equals nabla_sparse_attn_fwd's bit for bit.
 * Limit: the schedule, nabla_sparse_attn_workspace(B, S, heads, Tt, Ht, Wt) bytes, must fit
 * in 1 MiB (up to 131 008 groups of query blocks, e.g. B * heads <= 545 on the 720p tile grid
 * 16 x 6 x 10, whose 960 blocks form 240 groups per head), else NABLA_ERR_WORKSPACE.  NABLA_ERR_HIP also if the array's address
 * cannot be looked up.
 * Every call on one GPU shares that GPU's array and overwrites it (nothing is carried between
 * calls): calls that overlap on one GPU, e.g. on two streams, race and must be serialized by
 * the caller.
 */
nabla_status nabla_sparse_attn_fwd_noalloc(const void *q, const void *k, const void *v,
                                           nabla_dtype dtype, int B, int S, int heads,
                                           int head_dim, const int32_t *kv_nb,
                                           const int32_t *kv_inds, float scale, int Tt, int Ht,
                                           int Wt, void *o, void *stream);

/*
 * The same forward, also writing each row's log-sum-exp, which the backward needs
 * (the training pass of the same attention: NABLA summary page, Results, training
 * speed-up; the "nabla" page's forward runs flex attention, whose backward is the
 * gradient of that masked softmax).
 *
 * lse:      out [B, heads, S] fp32: log(sum over the row's allowed keys c of
 *           exp(scale * q . k_c)), natural log; -inf for a row with kv_nb == 0.
 *           Computed from the same bf16 products and weights as o.
 * Everything else, the workspace and the errors are those of nabla_sparse_attn_fwd
 * (lse NULL behaves exactly like nabla_sparse_attn_fwd).
 */
nabla_status nabla_sparse_attn_fwd_lse(const void *q, const void *k, const void *v,
                                       nabla_dtype dtype, int B, int S, int heads, int head_dim,
                                       const int32_t *kv_nb, const int32_t *kv_inds, float scale,
                                       int Tt, int Ht, int Wt, void *o, float *lse, void *ws,
                                       size_t ws_bytes, void *stream);

/* Bytes of workspace nabla_sparse_attn_fwd_grid needs for a T x H x W grid (the tile grid
 * is (T, ceil(H/8), ceil(W/8))).  0 if the sizes are invalid. */
size_t nabla_sparse_attn_workspace_grid(int B, int T, int H, int W, int heads);

/*
 * The forward (with optional lse) on the fractal layout of a T x H x W latent grid whose
 * H or W need not be multiples of 8 (S = T * ceil(H/8) * ceil(W/8) * 64; tile grid
 * (T, ceil(H/8), ceil(W/8))): the padding positions of partial patches are never keys.
 * Query rows at padding positions are computed as well (their q is 0 as the permute
 * writes it) and are dropped by the inverse permute.  Everything else is
 * nabla_sparse_attn_fwd_lse; on a grid of whole patches the result equals it.
 * Errors: those of nabla_sparse_attn_fwd_lse; INVALID_ARG also for T, H or W < 1.
 */
nabla_status nabla_sparse_attn_fwd_grid(const void *q, const void *k, const void *v,
                                        nabla_dtype dtype, int B, int T, int H, int W, int heads,
                                        int head_dim, const int32_t *kv_nb,
                                        const int32_t *kv_inds, float scale, void *o, float *lse,
                                        void *ws, size_t ws_bytes, void *stream);

/*
 * The forward (with optional lse) on q, k, v and o in natural order, with the fractal
 * permute and its inverse folded into the kernel's addressing: every token row is read
 * and written where the permutes would have moved it, so o equals, bit for bit, the
 * inverse permute of nabla_sparse_attn_fwd_lse's output on the permuted inputs (tile grid
 * (T, H/8, W/8)).  H and W must be multiples of 8; S = T * H * W.
 * q, k, v:  [B, T, H, W, heads, head_dim] (bf16 or fp32), natural order.
 * kv_nb, kv_inds: lists over fractal block indices, as nabla_block_mask_natural writes them.
 * o:        out [B, T, H, W, heads, head_dim], natural order; must not overlap inputs.
 * lse:      out [B, heads, S] fp32 in fractal order (as nabla_sparse_attn_fwd_lse), or NULL.
 * ws:       nabla_sparse_attn_workspace_grid(B, T, H, W, heads) bytes.
 * Errors: those of nabla_sparse_attn_fwd_grid; UNSUPPORTED also for H or W not a multiple
 * of 8, 8 * W * heads * head_dim * element size >= 2^32, or
 * more than 4096 blocks (S/64).
 */
nabla_status nabla_sparse_attn_fwd_natural(const void *q, const void *k, const void *v,
                                           nabla_dtype dtype, int B, int T, int H, int W,
                                           int heads, int head_dim, const int32_t *kv_nb,
                                           const int32_t *kv_inds, float scale, void *o,
                                           float *lse, void *ws, size_t ws_bytes,
                                           void *stream);

/*
 * Bytes of workspace nabla_sparse_attn_bwd needs: round_up(4 B heads S, 256) +
 * round_up(4 B heads nb, 256) + round_up(4 B heads nb^2, 256) + round_up(B heads nb^2,
 * 256) + 2 round_up(4 B heads nb, 256), nb = S/64 (row deltas, the transposed lists and
 * their byte matrix, the two gradient kernels' launch orders).  0 if the sizes are
 * invalid.
 */
size_t nabla_sparse_attn_bwd_workspace(int B, int S, int heads);

/*
 * Backward of nabla_sparse_attn_fwd: the gradients of o with respect to q, k and v for
 * a given output gradient dO, over the same lists (fixed; the mask is not
 * differentiated).  With P = exp(scale q k^T - lse) on the allowed blocks (0 elsewhere),
 * dP = dO V^T and Delta = rowsum(dO * o):
 *   dS = P (dP - Delta),   dq = scale dS K,   dk = scale dS^T Q,   dv = P^T dO.
 *
 * q, k, v, o, dout: [B, S, heads, head_dim] bf16, fractal order; o and lse as written
 *           by nabla_sparse_attn_fwd_lse for the same q, k, v, lists and scale.  Whole
 *           64-token blocks (padded layouts: nabla_sparse_attn_bwd_grid).
 * lse:      [B, heads, S] fp32.
 * kv_nb, kv_inds, scale: as for the forward.
 * dq, dk, dv: out [B, S, heads, head_dim] bf16; must not overlap the inputs or each
 *           other.  Every element is written (rows and keys no list touches get 0).
 * ws:       device workspace of at least nabla_sparse_attn_bwd_workspace() bytes
 *           (overwritten; no contents carried between calls; calls sharing one
 *           workspace must be on one stream).
 * Deterministic: no atomics; each output element is reduced in a fixed order.
 * Errors: INVALID_ARG (NULL pointer, sizes < 1, S % 64 != 0, NaN scale);
 * UNSUPPORTED (dtype not bf16, head_dim not 64 or 128, or S/64 > 4096);
 * WORKSPACE (ws NULL or ws_bytes too small).
 */
nabla_status nabla_sparse_attn_bwd(const void *q, const void *k, const void *v, const void *o,
                                   const void *dout, const float *lse, nabla_dtype dtype, int B,
                                   int S, int heads, int head_dim, const int32_t *kv_nb,
                                   const int32_t *kv_inds, float scale, void *dq, void *dk,
                                   void *dv, void *ws, size_t ws_bytes, void *stream);

/*
 * The backward of nabla_sparse_attn_fwd_grid: the training pass on the fractal layout of a
 * T x H x W latent grid whose H or W need not be multiples of 8 (S = T * ceil(H/8) *
 * ceil(W/8) * 64; the sibling "video_sparse_attn" page's variable block sizes).  The
 * padding positions of partial patches are never keys: their dk and dv are 0.  Query rows
 * at padding positions are rows like any other (with dO = 0 there, as nabla_fractal_permute
 * writes a permuted gradient, their dq is 0 and they add nothing to dk or dv).  o and lse
 * as written by nabla_sparse_attn_fwd_grid.  Everything else is nabla_sparse_attn_bwd; the
 * workspace is nabla_sparse_attn_bwd_workspace(B, S, heads) for that S.  On a grid of
 * whole patches the result equals nabla_sparse_attn_bwd.
 * Errors: those of nabla_sparse_attn_bwd; INVALID_ARG also for T, H or W < 1.
 */
nabla_status nabla_sparse_attn_bwd_grid(const void *q, const void *k, const void *v,
                                        const void *o, const void *dout, const float *lse,
                                        nabla_dtype dtype, int B, int T, int H, int W, int heads,
                                        int head_dim, const int32_t *kv_nb,
                                        const int32_t *kv_inds, float scale, void *dq, void *dk,
                                        void *dv, void *ws, size_t ws_bytes, void *stream);

/*
 * The quantized variant (the sibling "sla" backend page, the SageSLA forward: Q and K
 * in INT8 with one scale per block after the mean of K over the sequence is
 * subtracted, V in FP8 e4m3 with one scale per channel, then the block-sparse
 * attention on the codes with FP8 weights).  Blocks are the 64-token blocks of the
 * kv lists.
 *
 * Bytes of workspace nabla_quant_qkv needs: round_up(4 * B * heads * (S/64) * head_dim,
 * 256) + round_up(4 * B * heads * ceil(S/1024) * head_dim, 256) (block sums of k, partial
 * channel maxima of v).  0 if the sizes are invalid.
 */
size_t nabla_quant_qkv_workspace(int B, int S, int heads, int head_dim);
/*
 * Quantizes q, k, v ([B, S, heads, head_dim], bf16 or fp32, fractal order).  With
 * nb = S/64, per (b, head):
 *   k_mean[d] = (sum over blocks j of bs_j[d]) / S, bs_j[d] the sum of block j's 64
 *               tokens (both sums sequential in fp32 from +0; IEEE fp32 division);
 *   per block, for x = q and for x = k - k_mean (fp32):
 *               scale = amax|x| / 127 (fp32), code = clamp(rint(x / scale), -127, 127)
 *               (IEEE fp32 division, round half to even; amax = 0 gives scale 0, code 0);
 *   per channel d of v, over all S tokens:
 *               v_scale[d] = amax|v[:, d]| / 2.25, code = e4m3fn(v / v_scale[d]) (round to
 *               nearest even; OCP FP8 e4m3, largest finite 448; scale 0 gives code 0).
 * The codes and scales are exactly reproducible (fixed rounding and summation order).
 * Outputs (device, caller-owned, must not overlap the inputs):
 *   q8, k8:           [B, heads, nb, 64, head_dim] int8 (each block's rows in token order)
 *   q_scale, k_scale: [B, heads, nb] fp32
 *   v8:               [B, heads, nb, head_dim, 64] uint8 e4m3 codes (each block transposed)
 *   v_scale, k_mean:  [B, heads, head_dim] fp32
 * ws: device workspace of at least nabla_quant_qkv_workspace() bytes (overwritten).
 * Errors: INVALID_ARG (NULL pointer, sizes < 1, S % 64 != 0); UNSUPPORTED (head_dim not
 * 64 or 128); WORKSPACE (ws NULL or ws_bytes too small).
 */
nabla_status nabla_quant_qkv(const void *q, const void *k, const void *v, nabla_dtype dtype,
                             int B, int S, int heads, int head_dim, int8_t *q8, float *q_scale,
                             int8_t *k8, float *k_scale, uint8_t *v8, float *v_scale,
                             float *k_mean, void *ws, size_t ws_bytes, void *stream);
/*
 * The quantizer on the fractal layout of a T x H x W latent grid whose H or W need not be
 * multiples of 8 (S = T * ceil(H/8) * ceil(W/8) * 64; the sibling "video_sparse_attn"
 * page's variable block sizes).  Padding positions of partial patches are not tokens:
 * they are left out of the block sums and the k mean, whose divisor is the token count
 * T * H * W, and out of every block and channel maximum; their codes are 0 whatever the
 * inputs hold there.  Everything else is nabla_quant_qkv (its workspace for this S); on a
 * grid of whole patches the result equals it.
 * Errors: those of nabla_quant_qkv; INVALID_ARG also for T, H or W < 1.
 */
nabla_status nabla_quant_qkv_grid(const void *q, const void *k, const void *v,
                                  nabla_dtype dtype, int B, int T, int H, int W, int heads,
                                  int head_dim, int8_t *q8, float *q_scale, int8_t *k8,
                                  float *k_scale, uint8_t *v8, float *v_scale, float *k_mean,
                                  void *ws, size_t ws_bytes, void *stream);
/* Bytes of workspace nabla_sparse_attn_fwd_q8 needs (its work schedule; the same formula
 * as nabla_sparse_attn_workspace).  0 if the sizes or the grid are invalid. */
size_t nabla_sparse_attn_q8_workspace(int B, int S, int heads, int Tt, int Ht, int Wt);
/*
 * Block-sparse attention on the codes of nabla_quant_qkv (INT8 Q K^T with exact int32
 * sums, FP8 P V with fp32 accumulation).  For each (b, head, query block i) and query
 * row, over the keys c of the blocks j listed in kv_inds[b, head, i, 0 .. kv_nb - 1]:
 *   z_c  = scale * q_scale_i * k_scale_j * <q8_row, k8_c>
 *   w_c  = e4m3(C * exp(z_c - m))   with m within log(4) of the row maximum (the
 *          reference is raised lazily) and C * exp(z_c - m) <= 448
 *   o[d] = v_scale[d] * (sum_c w_c v8_cd) / (sum_c w_c)
 * A row with kv_nb == 0 gets o = 0.  The rounding of the weights depends on the
 * reference, so o matches the plain definition (weights rounded against the row
 * maximum) to within the weights' e4m3 rounding, not bit for bit.
 * q8 .. v_scale: as written by nabla_quant_qkv.
 * kv_nb, kv_inds, Tt, Ht, Wt: as for nabla_sparse_attn_fwd.
 * scale:    softmax scale; <= 0 selects 1/sqrt(head_dim).
 * o:        out [B, S, heads, head_dim] bf16.
 * ws:       device workspace of at least nabla_sparse_attn_q8_workspace() bytes.
 * Errors: INVALID_ARG (NULL pointer, sizes < 1, S % 64 != 0, NaN scale, a tile grid that
 * does not multiply to S/64); UNSUPPORTED (head_dim not 64 or 128, or S/64 > 4096);
 * WORKSPACE (ws NULL or ws_bytes too small).
 */
nabla_status nabla_sparse_attn_fwd_q8(const int8_t *q8, const float *q_scale, const int8_t *k8,
                                      const float *k_scale, const uint8_t *v8,
                                      const float *v_scale, int B, int S, int heads,
                                      int head_dim, const int32_t *kv_nb, const int32_t *kv_inds,
                                      float scale, int Tt, int Ht, int Wt, void *o, void *ws,
                                      size_t ws_bytes, void *stream);

/*
 * The quantized attention on the codes of nabla_quant_qkv_grid for a T x H x W grid
 * (S = T * ceil(H/8) * ceil(W/8) * 64; tile grid (T, ceil(H/8), ceil(W/8))): padding
 * positions of partial patches are never keys (their weights are 0).  Query rows at
 * padding positions are computed too and are dropped by the inverse permute.  Everything
 * else is nabla_sparse_attn_fwd_q8 with that tile grid (workspace:
 * nabla_sparse_attn_q8_workspace(B, S, heads, T, ceil(H/8), ceil(W/8))); on a grid of
 * whole patches the result equals it.
 * Errors: those of nabla_sparse_attn_fwd_q8; INVALID_ARG also for T, H or W < 1.
 */
nabla_status nabla_sparse_attn_fwd_q8_grid(const int8_t *q8, const float *q_scale,
                                           const int8_t *k8, const float *k_scale,
                                           const uint8_t *v8, const float *v_scale, int B, int T,
                                           int H, int W, int heads, int head_dim,
                                           const int32_t *kv_nb, const int32_t *kv_inds,
                                           float scale, void *o, void *ws, size_t ws_bytes,
                                           void *stream);

/*
 * The quantizer on q, k, v in natural order [B, T, H, W, heads, head_dim] (H, W multiples of
 * 8; S = T * H * W), with the fractal permute folded into its reads: the codes, scales and
 * k mean (in the fractal block layout of nabla_quant_qkv) are bit-identical to
 * nabla_quant_qkv's on the permuted tensors.  Workspace: nabla_quant_qkv_workspace(B, S,
 * heads, head_dim).  Errors: those of nabla_quant_qkv; INVALID_ARG also for T, H or W < 1;
 * UNSUPPORTED also for H or W not a multiple of 8, 8 * W * heads * head_dim * element
 * size >= 2^32, or more than 4096 blocks (S/64).
 */
nabla_status nabla_quant_qkv_natural(const void *q, const void *k, const void *v,
                                     nabla_dtype dtype, int B, int T, int H, int W, int heads,
                                     int head_dim, int8_t *q8, float *q_scale, int8_t *k8,
                                     float *k_scale, uint8_t *v8, float *v_scale, float *k_mean,
                                     void *ws, size_t ws_bytes, void *stream);

/*
 * The quantized forward writing o in natural order [B, T, H, W, heads, head_dim] bf16 (H, W
 * multiples of 8; tile grid (T, H/8, W/8)), with the inverse permute folded into its stores:
 * o is bit-identical to the inverse permute of nabla_sparse_attn_fwd_q8's output on the same
 * codes and lists.  Codes, scales, lists and workspace
 * (nabla_sparse_attn_q8_workspace(B, S, heads, T, H/8, W/8)) as for nabla_sparse_attn_fwd_q8.
 * Errors: those of nabla_sparse_attn_fwd_q8; INVALID_ARG also for T, H or W < 1;
 * UNSUPPORTED also for H or W not a multiple of 8, or more than 4096 blocks (S/64).
 */
nabla_status nabla_sparse_attn_fwd_q8_natural(const int8_t *q8, const float *q_scale,
                                              const int8_t *k8, const float *k_scale,
                                              const uint8_t *v8, const float *v_scale, int B,
                                              int T, int H, int W, int heads, int head_dim,
                                              const int32_t *kv_nb, const int32_t *kv_inds,
                                              float scale, void *o, void *ws, size_t ws_bytes,
                                              void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NABLA_H */
