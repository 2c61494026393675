// nabla_abi.hip -- the extern "C" entry points of libnabla.so (declared in
// include/nabla.h).  Host-side validation happens before any launch; nothing is
// enqueued unless the call returns NABLA_OK.
#include <math.h>

#include <mutex>

#include "../../include/nabla.h"
#include "nabla_launch.h"

namespace {

constexpr int kAbiVersion = 11;
constexpr int kBlock = 64;
constexpr int kTile = 8;
constexpr int kMaxBlocks = 4096;  // longest list row the kernels support (64 x 64-bit words)
constexpr int kMaxTopkBlocks = 2048;  // rows the top-k selection holds (one wave per row)

size_t dtype_bytes(nabla_dtype dt) { return dt == NABLA_BF16 ? 2 : 4; }
bool dtype_ok(nabla_dtype dt) { return dt == NABLA_BF16 || dt == NABLA_FP32; }
hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }
nabla_status from_hip(hipError_t e) { return e == hipSuccess ? NABLA_OK : NABLA_ERR_HIP; }

// B*S*heads*head_dim must stay addressable with 64-bit offsets (always) and the
// number of query blocks must fit a 1-D grid.
bool sizes_ok(int B, int S, int heads, int head_dim) {
    if (B < 1 || S < 1 || heads < 1 || head_dim < 1) return false;
    const long long rows = (long long)B * heads * (S / kBlock);
    return rows <= 0x7fffffffLL;
}

// Patches along an axis of n latent positions (the last one partial when 8 does not divide n).
long long tiles(int n) { return ((long long)n + kTile - 1) / kTile; }

// A tile grid is either all zero (unknown) or positive and multiplies to S/64.
bool grid_ok(int S, int Tt, int Ht, int Wt) {
    if (Tt == 0 && Ht == 0 && Wt == 0) return true;
    return Tt >= 1 && Ht >= 1 && Wt >= 1 && (long long)Tt * Ht * Wt == (long long)(S / kBlock);
}

}  // namespace

extern "C" {

int nabla_abi_version(void) { return kAbiVersion; }

const char *nabla_status_string(nabla_status s) {
    switch (s) {
        case NABLA_OK: return "ok";
        case NABLA_ERR_INVALID_ARG: return "invalid argument";
        case NABLA_ERR_UNSUPPORTED: return "unsupported configuration";
        case NABLA_ERR_WORKSPACE: return "workspace missing or too small";
        case NABLA_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

nabla_status nabla_fractal_permute(const void *x, void *y, nabla_dtype dtype, int B, int T,
                                   int H, int W, int heads, int head_dim, int inverse,
                                   void *stream) {
    if (!x || !y || !dtype_ok(dtype)) return NABLA_ERR_INVALID_ARG;
    if (B < 1 || T < 1 || H < 1 || W < 1 || heads < 1 || head_dim < 1)
        return NABLA_ERR_INVALID_ARG;
    const long long row_bytes = (long long)heads * head_dim * (long long)dtype_bytes(dtype);
    if (row_bytes % 16) return NABLA_ERR_UNSUPPORTED;
    if (row_bytes / 16 > 0x7fffffffLL / kBlock) return NABLA_ERR_UNSUPPORTED;
    const long long nb = (long long)T * tiles(H) * tiles(W);
    // one 256-lane workgroup per patch: the launch's lane count must fit 32 bits
    if ((long long)B * nb * 256 > 0xffffffffLL) return NABLA_ERR_UNSUPPORTED;
    return from_hip(nabla::launch_fractal_permute(x, y, (int)dtype_bytes(dtype), B, T, H, W,
                                                  heads * head_dim, inverse != 0,
                                                  as_stream(stream)));
}

nabla_status nabla_sta_mask(uint8_t *sta, int Tt, int Ht, int Wt, int win_t, int win_h,
                            int win_w, void *stream) {
    if (!sta || Tt < 1 || Ht < 1 || Wt < 1 || win_t < 0 || win_h < 0 || win_w < 0)
        return NABLA_ERR_INVALID_ARG;
    const long long nb = (long long)Tt * Ht * Wt;
    if (nb > (1LL << 20)) return NABLA_ERR_UNSUPPORTED;
    return from_hip(nabla::launch_sta_mask(sta, Tt, Ht, Wt, win_t, win_h, win_w,
                                           as_stream(stream)));
}

size_t nabla_block_mask_workspace(int B, int S, int heads, int head_dim) {
    if (!sizes_ok(B, S, heads, head_dim) || S % kBlock) return 0;
    const size_t nb = (size_t)(S / kBlock);
    const size_t pooled = 2ull * (size_t)B * heads * nb * head_dim * sizeof(float);
    const size_t scores =
        nabla::mask_scores_split((int)nb) ? (size_t)B * heads * nb * nb * sizeof(float) : 0;
    return pooled + scores;
}

}  // extern "C"

namespace {

// Both estimators; ratio < 0 selects the CDF cut (thr), ratio >= 0 the top-k variant.
// H, W > 0: the latent grid of a padded fractal layout (pooling over tokens only), or with
// natural, the grid of q and k in natural order.
nabla_status estimate(const void *q, const void *k, nabla_dtype dtype, int B, int S, int heads,
                      int head_dim, int H, int W, bool natural, const uint8_t *sta, double thr,
                      double ratio,
                      int32_t *kv_nb, int32_t *kv_inds, void *ws, size_t ws_bytes,
                      void *stream) {
    if (!q || !k || !kv_nb || !kv_inds || !dtype_ok(dtype)) return NABLA_ERR_INVALID_ARG;
    if (!sizes_ok(B, S, heads, head_dim) || S % kBlock) return NABLA_ERR_INVALID_ARG;
    const bool topk = ratio >= 0.0;
    if (!topk && !(thr >= 0.0 && thr <= 1.0)) return NABLA_ERR_INVALID_ARG;  // also NaN
    if (topk && !(ratio <= 1.0)) return NABLA_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128) return NABLA_ERR_UNSUPPORTED;
    // the selection grid has B * heads workgroups along y
    if ((long long)B * heads > 65535) return NABLA_ERR_UNSUPPORTED;
    const int nb = S / kBlock;
    if (nb > (topk ? kMaxTopkBlocks : kMaxBlocks)) return NABLA_ERR_UNSUPPORTED;
    const size_t need = nabla_block_mask_workspace(B, S, heads, head_dim);
    if (!ws || ws_bytes < need) return NABLA_ERR_WORKSPACE;
    float *qa = static_cast<float *>(ws);
    float *ka = qa + (size_t)B * heads * nb * head_dim;
    if (topk) {
        // k = min(nb, int(ratio * nb)): the product in double, truncated
        const double x = ratio * (double)nb;
        const int kk = x >= (double)nb ? nb : (int)x;
        return from_hip(nabla::launch_block_mask_topk(q, k, dtype == NABLA_BF16, B, S, heads,
                                                      head_dim, H, W, natural, sta, kk, kv_nb,
                                                      kv_inds,
                                                      qa, ka, as_stream(stream)));
    }
    // cut on the 2^-48 grid: ceil(fl32(1 - thr) * 2^48), exact in double
    const float cut32 = (float)(1.0 - thr);
    const int64_t cut_fixed = (int64_t)ceil(ldexp((double)cut32, 48));
    const float sqrt_d = (float)sqrt((double)head_dim);
    float *sbuf = ka + (size_t)B * heads * nb * head_dim;  // the score buffer, if any
    return from_hip(nabla::launch_block_mask(q, k, dtype == NABLA_BF16, B, S, heads, head_dim,
                                             H, W, natural, sta, cut_fixed, sqrt_d, kv_nb,
                                             kv_inds, qa, ka, sbuf, as_stream(stream)));
}

// S of the padded fractal layout of a T x H x W grid, or -1 when the sizes are invalid.
long long grid_len(int B, int T, int H, int W, int heads, int head_dim) {
    if (B < 1 || T < 1 || H < 1 || W < 1 || heads < 1 || head_dim < 1) return -1;
    const long long S = (long long)T * tiles(H) * tiles(W) * kBlock;
    if (S > 0x7fffffffLL || !sizes_ok(B, (int)S, heads, head_dim)) return -1;
    return S;
}

// S = T*H*W of a natural-order [B][T][H][W][heads][head_dim] grid read in place of its
// fractal permute; -1 when the sizes are invalid, -2 when the grid has partial patches, a
// patch's rows lie too far apart for the kernels' 32-bit in-tile offsets, or the sequence
// has more than kMaxBlocks blocks (the kernels find a block's patch row j / Wt by a
// multiply-high that is exact while j * Wt < 2^32; j < 4096 and Wt < 2^20 keep it so).
long long natural_len(int B, int T, int H, int W, int heads, int head_dim, size_t esize) {
    const long long S = grid_len(B, T, H, W, heads, head_dim);
    if (S < 0) return -1;
    if (H % kTile || W % kTile) return -2;
    if (((long long)kTile * W) * heads * head_dim * (long long)esize > 0xffffffffLL) return -2;
    if (S / kBlock > kMaxBlocks || W / kTile >= (1 << 20)) return -2;
    return S;
}

}  // namespace

extern "C" {

nabla_status nabla_block_mask(const void *q, const void *k, nabla_dtype dtype, int B, int S,
                              int heads, int head_dim, const uint8_t *sta, double thr,
                              int32_t *kv_nb, int32_t *kv_inds, void *ws, size_t ws_bytes,
                              void *stream) {
    return estimate(q, k, dtype, B, S, heads, head_dim, 0, 0, false, sta, thr, -1.0, kv_nb,
                    kv_inds, ws, ws_bytes, stream);
}

nabla_status nabla_block_mask_topk(const void *q, const void *k, nabla_dtype dtype, int B,
                                   int S, int heads, int head_dim, const uint8_t *sta,
                                   double topk_ratio, int32_t *kv_nb, int32_t *kv_inds, void *ws,
                                   size_t ws_bytes, void *stream) {
    if (!(topk_ratio >= 0.0 && topk_ratio <= 1.0)) return NABLA_ERR_INVALID_ARG;  // also NaN
    return estimate(q, k, dtype, B, S, heads, head_dim, 0, 0, false, sta, 0.0, topk_ratio,
                    kv_nb, kv_inds, ws, ws_bytes, stream);
}

nabla_status nabla_block_mask_grid(const void *q, const void *k, nabla_dtype dtype, int B,
                                   int T, int H, int W, int heads, int head_dim,
                                   const uint8_t *sta, double thr, double topk_ratio,
                                   int32_t *kv_nb, int32_t *kv_inds, void *ws, size_t ws_bytes,
                                   void *stream) {
    const long long S = grid_len(B, T, H, W, heads, head_dim);
    if (S < 0 || topk_ratio != topk_ratio) return NABLA_ERR_INVALID_ARG;
    return estimate(q, k, dtype, B, (int)S, heads, head_dim, H, W, false, sta, thr,
                    topk_ratio < 0.0 ? -1.0 : topk_ratio, kv_nb, kv_inds, ws, ws_bytes, stream);
}

nabla_status nabla_block_mask_natural(const void *q, const void *k, nabla_dtype dtype, int B,
                                      int T, int H, int W, int heads, int head_dim,
                                      const uint8_t *sta, double thr, double topk_ratio,
                                      int32_t *kv_nb, int32_t *kv_inds, void *ws,
                                      size_t ws_bytes, void *stream) {
    if (!dtype_ok(dtype)) return NABLA_ERR_INVALID_ARG;
    const long long S = natural_len(B, T, H, W, heads, head_dim, dtype_bytes(dtype));
    if (S == -1 || topk_ratio != topk_ratio) return NABLA_ERR_INVALID_ARG;
    if (S < 0) return NABLA_ERR_UNSUPPORTED;
    return estimate(q, k, dtype, B, (int)S, heads, head_dim, H, W, true, sta, thr,
                    topk_ratio < 0.0 ? -1.0 : topk_ratio, kv_nb, kv_inds, ws, ws_bytes, stream);
}

size_t nabla_sparse_attn_workspace(int B, int S, int heads, int Tt, int Ht, int Wt) {
    if (!sizes_ok(B, S, heads, 1) || S % kBlock || !grid_ok(S, Tt, Ht, Wt)) return 0;
    return nabla::sparse_attn_workspace_bytes(B, S, heads, Tt, Ht, Wt);
}

nabla_status nabla_sparse_attn_fwd(const void *q, const void *k, const void *v,
                                   nabla_dtype dtype, int B, int S, int heads, int head_dim,
                                   const int32_t *kv_nb, const int32_t *kv_inds, float scale,
                                   int Tt, int Ht, int Wt, void *o, void *ws, size_t ws_bytes,
                                   void *stream) {
    return nabla_sparse_attn_fwd_lse(q, k, v, dtype, B, S, heads, head_dim, kv_nb, kv_inds,
                                     scale, Tt, Ht, Wt, o, nullptr, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

// Every check of the forward's arguments except the workspace.
nabla_status attn_fwd_check(const void *q, const void *k, const void *v, nabla_dtype dtype, int B,
                            int S, int heads, int head_dim, const int32_t *kv_nb,
                            const int32_t *kv_inds, float scale, int Tt, int Ht, int Wt,
                            const void *o) {
    if (!q || !k || !v || !kv_nb || !kv_inds || !o || !dtype_ok(dtype))
        return NABLA_ERR_INVALID_ARG;
    if (!sizes_ok(B, S, heads, head_dim) || S % kBlock) return NABLA_ERR_INVALID_ARG;
    if (scale != scale) return NABLA_ERR_INVALID_ARG;
    if (!grid_ok(S, Tt, Ht, Wt)) return NABLA_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128) return NABLA_ERR_UNSUPPORTED;
    if (S / kBlock > kMaxBlocks) return NABLA_ERR_UNSUPPORTED;
    return NABLA_OK;
}

nabla_status attn_fwd(const void *q, const void *k, const void *v, nabla_dtype dtype, int B,
                      int S, int heads, int head_dim, const int32_t *kv_nb,
                      const int32_t *kv_inds, float scale, int Tt, int Ht, int Wt, int H, int W,
                      bool natural, void *o, float *lse, void *ws, size_t ws_bytes,
                      void *stream) {
    const nabla_status st = attn_fwd_check(q, k, v, dtype, B, S, heads, head_dim, kv_nb,
                                           kv_inds, scale, Tt, Ht, Wt, o);
    if (st != NABLA_OK) return st;
    if (!ws || ws_bytes < nabla::sparse_attn_workspace_bytes(B, S, heads, Tt, Ht, Wt))
        return NABLA_ERR_WORKSPACE;
    if (!(scale > 0.0f)) scale = (float)(1.0 / sqrt((double)head_dim));
    return from_hip(nabla::launch_sparse_attn(q, k, v, dtype == NABLA_BF16, B, S, heads,
                                              head_dim, Tt, Ht, Wt, H, W, natural, kv_nb,
                                              kv_inds, scale, o, lse, ws, as_stream(stream)));
}

}  // namespace

namespace {

// Hv > 0: a padded layout (Hv x Wv latents, tile grid (., Ht, Wt)); 0: whole blocks.
nabla_status attn_bwd(const void *q, const void *k, const void *v, const void *o,
                      const void *dout, const float *lse, nabla_dtype dtype, int B, int S,
                      int heads, int head_dim, const int32_t *kv_nb, const int32_t *kv_inds,
                      float scale, void *dq, void *dk, void *dv, int Ht, int Wt, int Hv, int Wv,
                      void *ws, size_t ws_bytes, void *stream) {
    if (!q || !k || !v || !o || !dout || !lse || !kv_nb || !kv_inds || !dq || !dk || !dv ||
        !dtype_ok(dtype))
        return NABLA_ERR_INVALID_ARG;
    if (!sizes_ok(B, S, heads, head_dim) || S % kBlock) return NABLA_ERR_INVALID_ARG;
    if (scale != scale) return NABLA_ERR_INVALID_ARG;
    if (dtype != NABLA_BF16) return NABLA_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return NABLA_ERR_UNSUPPORTED;
    if (S / kBlock > kMaxBlocks) return NABLA_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < nabla::sparse_attn_bwd_workspace_bytes(B, S, heads))
        return NABLA_ERR_WORKSPACE;
    if (!(scale > 0.0f)) scale = (float)(1.0 / sqrt((double)head_dim));
    return from_hip(nabla::launch_sparse_attn_bwd(q, k, v, o, dout, lse, B, S, heads, head_dim,
                                                  kv_nb, kv_inds, scale, dq, dk, dv, Ht, Wt, Hv,
                                                  Wv, ws, as_stream(stream)));
}

}  // namespace

extern "C" {

nabla_status nabla_sparse_attn_fwd_lse(const void *q, const void *k, const void *v,
                                       nabla_dtype dtype, int B, int S, int heads, int head_dim,
                                       const int32_t *kv_nb, const int32_t *kv_inds, float scale,
                                       int Tt, int Ht, int Wt, void *o, float *lse, void *ws,
                                       size_t ws_bytes, void *stream) {
    return attn_fwd(q, k, v, dtype, B, S, heads, head_dim, kv_nb, kv_inds, scale, Tt, Ht, Wt, 0,
                    0, false, o, lse, ws, ws_bytes, stream);
}

size_t nabla_sparse_attn_workspace_grid(int B, int T, int H, int W, int heads) {
    const long long S = grid_len(B, T, H, W, heads, 1);
    if (S < 0) return 0;
    return nabla_sparse_attn_workspace(B, (int)S, heads, T, (int)tiles(H), (int)tiles(W));
}

nabla_status nabla_sparse_attn_fwd_grid(const void *q, const void *k, const void *v,
                                        nabla_dtype dtype, int B, int T, int H, int W, int heads,
                                        int head_dim, const int32_t *kv_nb,
                                        const int32_t *kv_inds, float scale, void *o, float *lse,
                                        void *ws, size_t ws_bytes, void *stream) {
    const long long S = grid_len(B, T, H, W, heads, head_dim);
    if (S < 0) return NABLA_ERR_INVALID_ARG;
    return attn_fwd(q, k, v, dtype, B, (int)S, heads, head_dim, kv_nb, kv_inds, scale, T,
                    (int)tiles(H), (int)tiles(W), H, W, false, o, lse, ws, ws_bytes, stream);
}

nabla_status nabla_sparse_attn_fwd_natural(const void *q, const void *k, const void *v,
                                           nabla_dtype dtype, int B, int T, int H, int W,
                                           int heads, int head_dim, const int32_t *kv_nb,
                                           const int32_t *kv_inds, float scale, void *o,
                                           float *lse, void *ws, size_t ws_bytes,
                                           void *stream) {
    if (!dtype_ok(dtype)) return NABLA_ERR_INVALID_ARG;
    const long long S = natural_len(B, T, H, W, heads, head_dim, dtype_bytes(dtype));
    if (S == -1) return NABLA_ERR_INVALID_ARG;
    if (S < 0) return NABLA_ERR_UNSUPPORTED;
    return attn_fwd(q, k, v, dtype, B, (int)S, heads, head_dim, kv_nb, kv_inds, scale, T,
                    H / kTile, W / kTile, 0, 0, true, o, lse, ws, ws_bytes, stream);
}

size_t nabla_sparse_attn_bwd_workspace(int B, int S, int heads) {
    if (!sizes_ok(B, S, heads, 1) || S % kBlock || S / kBlock > kMaxBlocks) return 0;
    return nabla::sparse_attn_bwd_workspace_bytes(B, S, heads);
}

nabla_status nabla_sparse_attn_bwd(const void *q, const void *k, const void *v, const void *o,
                                   const void *dout, const float *lse, nabla_dtype dtype, int B,
                                   int S, int heads, int head_dim, const int32_t *kv_nb,
                                   const int32_t *kv_inds, float scale, void *dq, void *dk,
                                   void *dv, void *ws, size_t ws_bytes, void *stream) {
    return attn_bwd(q, k, v, o, dout, lse, dtype, B, S, heads, head_dim, kv_nb, kv_inds, scale,
                    dq, dk, dv, 0, 0, 0, 0, ws, ws_bytes, stream);
}

nabla_status nabla_sparse_attn_bwd_grid(const void *q, const void *k, const void *v,
                                        const void *o, const void *dout, const float *lse,
                                        nabla_dtype dtype, int B, int T, int H, int W, int heads,
                                        int head_dim, const int32_t *kv_nb,
                                        const int32_t *kv_inds, float scale, void *dq, void *dk,
                                        void *dv, void *ws, size_t ws_bytes, void *stream) {
    const long long S = grid_len(B, T, H, W, heads, head_dim);
    if (S < 0) return NABLA_ERR_INVALID_ARG;
    return attn_bwd(q, k, v, o, dout, lse, dtype, B, (int)S, heads, head_dim, kv_nb, kv_inds,
                    scale, dq, dk, dv, (int)tiles(H), (int)tiles(W), H, W, ws, ws_bytes, stream);
}

size_t nabla_quant_qkv_workspace(int B, int S, int heads, int head_dim) {
    if (!sizes_ok(B, S, heads, head_dim) || S % kBlock) return 0;
    return nabla::quant_workspace_bytes(B, S, heads, head_dim);
}

}  // extern "C"

namespace {

// T, Hv > 0: a padded layout (T frames of Hv x Wv latents); Hv = 0: whole blocks.
nabla_status quant_qkv(const void *q, const void *k, const void *v, nabla_dtype dtype, int B,
                       int S, int heads, int head_dim, int8_t *q8, float *q_scale, int8_t *k8,
                       float *k_scale, uint8_t *v8, float *v_scale, float *k_mean, int T,
                       int Hv, int Wv, int natW, void *ws, size_t ws_bytes, void *stream) {
    if (!q || !k || !v || !q8 || !q_scale || !k8 || !k_scale || !v8 || !v_scale || !k_mean ||
        !dtype_ok(dtype))
        return NABLA_ERR_INVALID_ARG;
    if (!sizes_ok(B, S, heads, head_dim) || S % kBlock) return NABLA_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128) return NABLA_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < nabla::quant_workspace_bytes(B, S, heads, head_dim))
        return NABLA_ERR_WORKSPACE;
    return from_hip(nabla::launch_quant_qkv(q, k, v, dtype == NABLA_BF16, B, S, heads, head_dim,
                                            q8, q_scale, k8, k_scale, v8, v_scale, k_mean, T, Hv,
                                            Wv, natW, ws, as_stream(stream)));
}

nabla_status attn_fwd_q8(const int8_t *q8, const float *q_scale, const int8_t *k8,
                         const float *k_scale, const uint8_t *v8, const float *v_scale, int B,
                         int S, int heads, int head_dim, const int32_t *kv_nb,
                         const int32_t *kv_inds, float scale, int Tt, int Ht, int Wt, int Hv,
                         int Wv, bool natural, void *o, void *ws, size_t ws_bytes,
                         void *stream) {
    if (!q8 || !q_scale || !k8 || !k_scale || !v8 || !v_scale || !kv_nb || !kv_inds || !o)
        return NABLA_ERR_INVALID_ARG;
    if (!sizes_ok(B, S, heads, head_dim) || S % kBlock) return NABLA_ERR_INVALID_ARG;
    if (scale != scale) return NABLA_ERR_INVALID_ARG;
    if (!grid_ok(S, Tt, Ht, Wt)) return NABLA_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128) return NABLA_ERR_UNSUPPORTED;
    if (S / kBlock > kMaxBlocks) return NABLA_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < nabla::sparse_attn_q8_workspace_bytes(B, S, heads, Tt, Ht, Wt))
        return NABLA_ERR_WORKSPACE;
    if (!(scale > 0.0f)) scale = (float)(1.0 / sqrt((double)head_dim));
    return from_hip(nabla::launch_sparse_attn_q8(q8, q_scale, k8, k_scale, v8, v_scale, B, S,
                                                 heads, head_dim, Tt, Ht, Wt, kv_nb, kv_inds,
                                                 scale, Hv, Wv, natural, o, ws,
                                                 as_stream(stream)));
}

}  // namespace

extern "C" {

nabla_status nabla_quant_qkv(const void *q, const void *k, const void *v, nabla_dtype dtype,
                             int B, int S, int heads, int head_dim, int8_t *q8, float *q_scale,
                             int8_t *k8, float *k_scale, uint8_t *v8, float *v_scale,
                             float *k_mean, void *ws, size_t ws_bytes, void *stream) {
    return quant_qkv(q, k, v, dtype, B, S, heads, head_dim, q8, q_scale, k8, k_scale, v8,
                     v_scale, k_mean, 0, 0, 0, 0, ws, ws_bytes, stream);
}

nabla_status nabla_quant_qkv_natural(const void *q, const void *k, const void *v,
                                     nabla_dtype dtype, int B, int T, int H, int W, int heads,
                                     int head_dim, int8_t *q8, float *q_scale, int8_t *k8,
                                     float *k_scale, uint8_t *v8, float *v_scale, float *k_mean,
                                     void *ws, size_t ws_bytes, void *stream) {
    if (!dtype_ok(dtype)) return NABLA_ERR_INVALID_ARG;
    const long long S = natural_len(B, T, H, W, heads, head_dim, dtype_bytes(dtype));
    if (S == -1) return NABLA_ERR_INVALID_ARG;
    if (S < 0) return NABLA_ERR_UNSUPPORTED;
    return quant_qkv(q, k, v, dtype, B, (int)S, heads, head_dim, q8, q_scale, k8, k_scale, v8,
                     v_scale, k_mean, 0, 0, 0, W, ws, ws_bytes, stream);
}

nabla_status nabla_quant_qkv_grid(const void *q, const void *k, const void *v,
                                  nabla_dtype dtype, int B, int T, int H, int W, int heads,
                                  int head_dim, int8_t *q8, float *q_scale, int8_t *k8,
                                  float *k_scale, uint8_t *v8, float *v_scale, float *k_mean,
                                  void *ws, size_t ws_bytes, void *stream) {
    const long long S = grid_len(B, T, H, W, heads, head_dim);
    if (S < 0) return NABLA_ERR_INVALID_ARG;
    return quant_qkv(q, k, v, dtype, B, (int)S, heads, head_dim, q8, q_scale, k8, k_scale, v8,
                     v_scale, k_mean, T, H, W, 0, ws, ws_bytes, stream);
}

size_t nabla_sparse_attn_q8_workspace(int B, int S, int heads, int Tt, int Ht, int Wt) {
    if (!sizes_ok(B, S, heads, 1) || S % kBlock || !grid_ok(S, Tt, Ht, Wt)) return 0;
    return nabla::sparse_attn_q8_workspace_bytes(B, S, heads, Tt, Ht, Wt);
}

nabla_status nabla_sparse_attn_fwd_q8(const int8_t *q8, const float *q_scale, const int8_t *k8,
                                      const float *k_scale, const uint8_t *v8,
                                      const float *v_scale, int B, int S, int heads,
                                      int head_dim, const int32_t *kv_nb, const int32_t *kv_inds,
                                      float scale, int Tt, int Ht, int Wt, void *o, void *ws,
                                      size_t ws_bytes, void *stream) {
    return attn_fwd_q8(q8, q_scale, k8, k_scale, v8, v_scale, B, S, heads, head_dim, kv_nb,
                       kv_inds, scale, Tt, Ht, Wt, 0, 0, false, o, ws, ws_bytes, stream);
}

nabla_status nabla_sparse_attn_fwd_q8_natural(const int8_t *q8, const float *q_scale,
                                              const int8_t *k8, const float *k_scale,
                                              const uint8_t *v8, const float *v_scale, int B,
                                              int T, int H, int W, int heads, int head_dim,
                                              const int32_t *kv_nb, const int32_t *kv_inds,
                                              float scale, void *o, void *ws, size_t ws_bytes,
                                              void *stream) {
    const long long S = natural_len(B, T, H, W, heads, head_dim, 2);
    if (S == -1) return NABLA_ERR_INVALID_ARG;
    if (S < 0) return NABLA_ERR_UNSUPPORTED;
    return attn_fwd_q8(q8, q_scale, k8, k_scale, v8, v_scale, B, (int)S, heads, head_dim, kv_nb,
                       kv_inds, scale, T, H / kTile, W / kTile, 0, 0, true, o, ws, ws_bytes,
                       stream);
}

nabla_status nabla_sparse_attn_fwd_q8_grid(const int8_t *q8, const float *q_scale,
                                           const int8_t *k8, const float *k_scale,
                                           const uint8_t *v8, const float *v_scale, int B, int T,
                                           int H, int W, int heads, int head_dim,
                                           const int32_t *kv_nb, const int32_t *kv_inds,
                                           float scale, void *o, void *ws, size_t ws_bytes,
                                           void *stream) {
    const long long S = grid_len(B, T, H, W, heads, head_dim);
    if (S < 0) return NABLA_ERR_INVALID_ARG;
    return attn_fwd_q8(q8, q_scale, k8, k_scale, v8, v_scale, B, (int)S, heads, head_dim, kv_nb,
                       kv_inds, scale, T, (int)tiles(H), (int)tiles(W), H, W, false, o, ws,
                       ws_bytes, stream);
}

}  // extern "C"

// ---- the forward without allocation.  Its only scratch memory, the work schedule (take
// counter, group costs, group order), lives in a file-scope device array: every GPU the
// library runs on holds its own copy until the process ends.  Host code never passes the
// array's name to a kernel (on the host it only stands for the symbol): the device address
// comes from hipGetSymbolAddress, once per device, and is kept per device.
namespace {

constexpr size_t kScratchBytes = (size_t)1 << 20;  // 1 MiB: up to 131 008 query-block groups
constexpr int kMaxScratchDevices = 64;

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxScratchDevices];  // device address of `scratch` per device, or null

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// The current device's address of `scratch`, looked up on the first call on that device.
nabla_status scratch_for_current_device(void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices)
        return NABLA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return NABLA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return NABLA_OK;
}

}  // namespace

extern "C" {

nabla_status nabla_sparse_attn_fwd_noalloc(const void *q, const void *k, const void *v,
                                           nabla_dtype dtype, int B, int S, int heads,
                                           int head_dim, const int32_t *kv_nb,
                                           const int32_t *kv_inds, float scale, int Tt, int Ht,
                                           int Wt, void *o, void *stream) {
    const nabla_status st = attn_fwd_check(q, k, v, dtype, B, S, heads, head_dim, kv_nb,
                                           kv_inds, scale, Tt, Ht, Wt, o);
    if (st != NABLA_OK) return st;
    if (nabla::sparse_attn_workspace_bytes(B, S, heads, Tt, Ht, Wt) > kScratchBytes)
        return NABLA_ERR_WORKSPACE;
    void *ws = nullptr;
    const nabla_status got = scratch_for_current_device(&ws);
    if (got != NABLA_OK) return got;
    return attn_fwd(q, k, v, dtype, B, S, heads, head_dim, kv_nb, kv_inds, scale, Tt, Ht, Wt, 0,
                    0, false, o, nullptr, ws, kScratchBytes, stream);
}

}  // extern "C"
