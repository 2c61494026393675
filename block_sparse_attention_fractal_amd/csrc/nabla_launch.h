// nabla_launch.h -- host launchers of the libnabla kernels (internal; the public
// C ABI is include/nabla.h).  Arguments are validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <atomic>
#include <stdint.h>

namespace nabla {

hipError_t launch_fractal_permute(const void *x, void *y, int elem_bytes, int B, int T, int H,
                                  int W, int row_elems, bool inverse, hipStream_t stream);

hipError_t launch_sta_mask(uint8_t *sta, int Tt, int Ht, int Wt, int win_t, int win_h,
                           int win_w, hipStream_t stream);

// Pooled blocks [B*heads][nb][D] fp32 of q (qa) and k (ka), then per-row
// selection; cut_fixed = ceil(fl32(1 - thr) * 2^48).  H, W > 0: the latent grid of a
// padded fractal layout (blocks average their tokens only); 0: whole 64-token blocks.
// natural: q and k are in natural order [B][T][H][W][heads][D] (H, W multiples of 8,
// S = T*H*W), read in place of their fractal permute.
hipError_t launch_block_mask(const void *q, const void *k, bool bf16_in, int B, int S,
                             int heads, int D, int H, int W, bool natural, const uint8_t *sta,
                             int64_t cut_fixed, float sqrt_d, int32_t *kv_nb, int32_t *kv_inds,
                             float *qa, float *ka, float *sbuf, hipStream_t stream);
// Rows whose selection runs from a score buffer of B * heads * nb * nb floats in the
// workspace (scores and selection in two launches): 513 to 2048 blocks.
inline bool mask_scores_split(int nb) { return nb > 512 && nb <= 2048; }

// The top-k variant: pooled blocks, smooth-k, the topk largest scores per row (k <= nb,
// nb <= 2048), STA union.  H, W as for launch_block_mask.
hipError_t launch_block_mask_topk(const void *q, const void *k, bool bf16_in, int B, int S,
                                  int heads, int D, int H, int W, bool natural,
                                  const uint8_t *sta, int topk,
                                  int32_t *kv_nb, int32_t *kv_inds, float *qa, float *ka,
                                  hipStream_t stream);

// Workgroups of kernel K (of `threads` lanes) the device holds at once (occupancy x CUs),
// cached per device and kernel; 0 if the query fails.
// The cache entries are atomics: calls on different streams or threads may query and fill
// them at the same time; a racing first call computes and stores the same value.
template <auto K>
int resident_workgroups(int threads) {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];  // 0 = not yet known
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    const int known = cache[dev].load(std::memory_order_relaxed);
    if (known > 0) return known;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, K, threads, 0) != hipSuccess)
        return 0;
    const int value = cus * (per_cu > 0 ? per_cu : 1);
    cache[dev].store(value, std::memory_order_relaxed);
    return value;
}

// The attention walk's schedule (groups of neighbouring query blocks, phases of a few
// heads, longest first): plan kernels write the group order and reset the take counter
// in a workspace of attn_schedule_bytes(); the walk kernel takes groups from it.
struct AttnSchedule {
    int groups_per_bh, ngroups, grid;
    int32_t *order, *counter;
};
int attn_groups_per_bh(int S, int Tt, int Ht, int Wt);
// order[0 .. n) = 0 .. n-1 arranged longest first (by cost[], each in [0, maxcost], maxcost
// < 4096) within phases of per_phase consecutive items (the remainder joins the last phase).
hipError_t launch_longest_first(const int32_t *cost, int n, int per_phase, int maxcost,
                                int32_t *order, hipStream_t stream);
size_t attn_schedule_bytes(int B, int S, int heads, int Tt, int Ht, int Wt);
// resident: workgroups of the walk kernel the device holds at once (sets the phase size).
AttnSchedule launch_attn_plan(const int32_t *kv_nb, const int32_t *kv_inds, int B, int S,
                              int heads, int Tt, int Ht, int Wt, int resident, void *ws,
                              hipStream_t stream);

// Tt, Ht, Wt: tile grid of the query blocks (Tt*Ht*Wt == S/64), or all 0 if unknown.
// ws: sparse_attn_workspace_bytes() bytes (schedule: counter, group costs, order).
size_t sparse_attn_workspace_bytes(int B, int S, int heads, int Tt, int Ht, int Wt);
// lse: [B*heads][S] fp32 natural-log log-sum-exp of each row's scaled scores, or null.
// H, W > 0: the latent grid of a padded fractal layout over the tile grid (Tt, Ht, Wt):
// padding positions of partial patches are never keys.  0: whole blocks.
// natural: q, k, v and o are in natural order [B][T][H][W][heads][D] (whole patches,
// H = 8 Ht, W = 8 Wt); lse stays in fractal order.
hipError_t launch_sparse_attn(const void *q, const void *k, const void *v, bool bf16_in,
                              int B, int S, int heads, int D, int Tt, int Ht, int Wt, int H,
                              int W, bool natural, const int32_t *kv_nb,
                              const int32_t *kv_inds, float scale, void *o, float *lse, void *ws,
                              hipStream_t stream);

// Backward (bf16 tensors): dq, dk, dv from q, k, v, o, dO, lse and the kv lists.
// Hv > 0: a padded layout of Hv x Wv latents on a tile grid (., Ht, Wt), whose padding
// positions are not keys; Hv = 0: whole blocks (Ht, Wt unused).
// ws: sparse_attn_bwd_workspace_bytes() bytes (row deltas, transposed lists).
size_t sparse_attn_bwd_workspace_bytes(int B, int S, int heads);
hipError_t launch_sparse_attn_bwd(const void *q, const void *k, const void *v, const void *o,
                                  const void *dout, const float *lse, int B, int S, int heads,
                                  int D, const int32_t *kv_nb, const int32_t *kv_inds,
                                  float scale, void *dq, void *dk, void *dv, int Ht, int Wt,
                                  int Hv, int Wv, void *ws, hipStream_t stream);

// The quantized variant.  Codes and scales of q, k, v (layouts in nabla.h,
// nabla_quant_qkv); ws: quant_workspace_bytes() bytes (k block sums, partial v maxima).
size_t quant_workspace_bytes(int B, int S, int heads, int D);
// Hv > 0: a padded layout of T frames of Hv x Wv latents, whose padding positions are not
// tokens; Hv = 0: whole blocks (T unused).  natW > 0 (with Hv = 0): q, k, v in natural order
// with rows of natW tokens (whole patches), read in place of their fractal permute.
hipError_t launch_quant_qkv(const void *q, const void *k, const void *v, bool bf16_in, int B,
                            int S, int heads, int D, int8_t *q8, float *qs, int8_t *k8,
                            float *ks, uint8_t *v8, float *vs, float *km, int T, int Hv, int Wv,
                            int natW, void *ws, hipStream_t stream);
// The attention on those codes (bf16 o); ws: sparse_attn_q8_workspace_bytes() bytes.
// natural (with Hv = 0): o is written in natural order (rows of 8 Wt tokens).
size_t sparse_attn_q8_workspace_bytes(int B, int S, int heads, int Tt, int Ht, int Wt);
hipError_t launch_sparse_attn_q8(const int8_t *q8, const float *qs, const int8_t *k8,
                                 const float *ks, const uint8_t *v8, const float *vs, int B,
                                 int S, int heads, int D, int Tt, int Ht, int Wt,
                                 const int32_t *kv_nb, const int32_t *kv_inds, float scale,
                                 int Hv, int Wv, bool natural, void *o, void *ws,
                                 hipStream_t stream);

}  // namespace nabla
