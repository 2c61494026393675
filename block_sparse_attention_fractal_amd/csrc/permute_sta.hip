// permute_sta.hip -- fractal token reordering and the STA block mask.
//
// Fractal reordering (NABLA summary page, Technical Summary > Methodology,
// "Token Reordering"): every 8 x 8 spatial patch of a frame becomes one run of
// 64 tokens; frames stay in time order, patches in raster order, tokens in a
// patch in raster order.  Pure data movement: one workgroup moves the 64 token
// rows of one patch with 16-byte accesses; the fractal side is one contiguous
// 64-row run, the natural side is 8 runs of 8 contiguous rows.
//
// STA mask ("nabla" page, NablaAttentionMetadata.sta_mask; NABLA summary page,
// Methodology, "Hybrid Integration with STA"): blocks are neighbours when their
// tile coordinates differ by at most (win_t, win_h, win_w), clipped at borders.
#include "nabla_device.h"
#include "nabla_launch.h"

namespace nabla {

// grid.x = B * nb (one 64-token patch each); row_chunks = 16-byte chunks per token row.
// Lane work item id in [0, 64*row_chunks): token w = id / row_chunks of the patch,
// chunk c = id % row_chunks of its row.
__device__ __forceinline__ void permute_addr(int id, int row_chunks, int64_t nat_row0, int W,
                                             int64_t frac0, bool inverse, int64_t &src,
                                             int64_t &dst) {
    const int w = id / row_chunks;
    const int c = id - w * row_chunks;
    // natural token of patch row (w / 8), column (w % 8)
    const int64_t nat = (nat_row0 + (int64_t)(w >> 3) * W + (w & 7)) * row_chunks + c;
    const int64_t fra = frac0 + id;
    src = inverse ? fra : nat;
    dst = inverse ? nat : fra;
}

// H and W need not be multiples of 8: each frame is padded to ceil(H/8) x ceil(W/8)
// patches (the sibling "video_sparse_attn" page's variable block sizes).  A padding
// position of a partial patch is written as 0 going to fractal order and is not read
// going back.  Whole patches take the unchecked path.
template <bool kFull>
__global__ __launch_bounds__(256) void fractal_permute_kernel(const uint4 *__restrict__ x,
                                                              uint4 *__restrict__ y,
                                                              int T, int H, int W,
                                                              int row_chunks, int inverse) {
    constexpr int U = 8;
    const int Ht = (H + kTile - 1) / kTile, Wt = (W + kTile - 1) / kTile;
    const int nb = T * Ht * Wt;
    const int b = blockIdx.x / nb;
    const int tile = blockIdx.x % nb;
    const int t = tile / (Ht * Wt);
    const int th = (tile / Wt) % Ht;
    const int tw = tile % Wt;
    const int64_t S = (int64_t)nb * kBlock;
    const int64_t frac0 = ((int64_t)b * S + (int64_t)tile * kBlock) * row_chunks;
    const int64_t nat_row0 = (((int64_t)b * T + t) * H + th * kTile) * W + tw * kTile;
    const int total = kBlock * row_chunks;
    const int vrows = H - th * kTile, vcols = W - tw * kTile;  // >= 1; >= 8 on whole patches
    if (vrows < kTile || vcols < kTile) {  // partial patch (workgroup-uniform)
        for (int id = threadIdx.x; id < total; id += 256) {
            const int w = id / row_chunks;
            const bool tok = (w >> 3) < vrows && (w & 7) < vcols;
            int64_t s, d;
            permute_addr(id, row_chunks, nat_row0, W, frac0, inverse, s, d);
            if (tok)
                y[d] = x[s];
            else if (!inverse)
                y[d] = make_uint4(0u, 0u, 0u, 0u);
        }
        return;
    }
    if constexpr (kFull) {  // total is a multiple of 256 * U
        for (int base = threadIdx.x; base < total; base += 256 * U) {
            uint4 v0, v1, v2, v3, v4, v5, v6, v7;
            int64_t s0, s1, s2, s3, s4, s5, s6, s7, d0, d1, d2, d3, d4, d5, d6, d7;
            permute_addr(base + 0 * 256, row_chunks, nat_row0, W, frac0, inverse, s0, d0);
            permute_addr(base + 1 * 256, row_chunks, nat_row0, W, frac0, inverse, s1, d1);
            permute_addr(base + 2 * 256, row_chunks, nat_row0, W, frac0, inverse, s2, d2);
            permute_addr(base + 3 * 256, row_chunks, nat_row0, W, frac0, inverse, s3, d3);
            permute_addr(base + 4 * 256, row_chunks, nat_row0, W, frac0, inverse, s4, d4);
            permute_addr(base + 5 * 256, row_chunks, nat_row0, W, frac0, inverse, s5, d5);
            permute_addr(base + 6 * 256, row_chunks, nat_row0, W, frac0, inverse, s6, d6);
            permute_addr(base + 7 * 256, row_chunks, nat_row0, W, frac0, inverse, s7, d7);
            v0 = x[s0]; v1 = x[s1]; v2 = x[s2]; v3 = x[s3];
            v4 = x[s4]; v5 = x[s5]; v6 = x[s6]; v7 = x[s7];
            y[d0] = v0; y[d1] = v1; y[d2] = v2; y[d3] = v3;
            y[d4] = v4; y[d5] = v5; y[d6] = v6; y[d7] = v7;
        }
    } else {
        for (int id = threadIdx.x; id < total; id += 256) {
            int64_t s, d;
            permute_addr(id, row_chunks, nat_row0, W, frac0, inverse, s, d);
            y[d] = x[s];
        }
    }
}

hipError_t launch_fractal_permute(const void *x, void *y, int elem_bytes, int B, int T, int H,
                                  int W, int row_elems, bool inverse, hipStream_t stream) {
    const int row_chunks = row_elems * elem_bytes / 16;
    const int nb = T * ((H + kTile - 1) / kTile) * ((W + kTile - 1) / kTile);
    const int64_t grid = (int64_t)B * nb;
    if ((kBlock * row_chunks) % (256 * 8) == 0)
        hipLaunchKernelGGL(fractal_permute_kernel<true>, dim3((unsigned)grid), dim3(256), 0,
                           stream, (const uint4 *)x, (uint4 *)y, T, H, W, row_chunks,
                           inverse ? 1 : 0);
    else
        hipLaunchKernelGGL(fractal_permute_kernel<false>, dim3((unsigned)grid), dim3(256), 0,
                           stream, (const uint4 *)x, (uint4 *)y, T, H, W, row_chunks,
                           inverse ? 1 : 0);
    return hipGetLastError();
}

// One thread per (i, j) byte of the nb x nb mask.
__global__ __launch_bounds__(256) void sta_mask_kernel(uint8_t *__restrict__ sta, int Tt, int Ht,
                                                       int Wt, int win_t, int win_h, int win_w) {
    const int64_t nb = (int64_t)Tt * Ht * Wt;
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= nb * nb) return;
    const int i = (int)(id / nb), j = (int)(id % nb);
    const int ti = i / (Ht * Wt), hi = (i / Wt) % Ht, wi = i % Wt;
    const int tj = j / (Ht * Wt), hj = (j / Wt) % Ht, wj = j % Wt;
    sta[id] = (uint8_t)(abs(ti - tj) <= win_t && abs(hi - hj) <= win_h && abs(wi - wj) <= win_w);
}

hipError_t launch_sta_mask(uint8_t *sta, int Tt, int Ht, int Wt, int win_t, int win_h,
                           int win_w, hipStream_t stream) {
    const int64_t nb = (int64_t)Tt * Ht * Wt;
    const int64_t grid = (nb * nb + 255) / 256;
    hipLaunchKernelGGL(sta_mask_kernel, dim3((unsigned)grid), dim3(256), 0, stream, sta, Tt, Ht,
                       Wt, win_t, win_h, win_w);
    return hipGetLastError();
}

}  // namespace nabla
