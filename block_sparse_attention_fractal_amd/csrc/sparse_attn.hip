// sparse_attn.hip -- NABLA block-sparse attention forward on gfx950.
//
// Computes, for each (b, head, query block i) and each of its 64 query rows,
// softmax(scale * q K_J^T) V_J over the tokens J of the kv blocks listed in
// kv_inds[b, head, i, 0 .. kv_nb - 1]; every listed block is a full 64 x 64
// block ("nabla" page, NablaAttentionImpl.forward and nablaT_v2's BlockMask
// creation: full blocks only, no per-element mask; NABLA summary page,
// Methodology, "Expansion").  Scale defaults to 1/sqrt(D) (the flex-attention
// default; the forward passes none).
//
// Design (CDNA4):
//   * one workgroup = 4 waves = one query block; wave w owns query rows
//     16w .. 16w+15 and keeps them in registers as MFMA operands;
//   * v_mfma_f32_16x16x32_bf16 throughout, fp32 accumulation;
//   * scores are formed transposed, S^T = K Q^T, so the MFMA output puts one
//     query row per lane column: the row max needs two lane swaps and the row
//     sum stays lane-local until the end;
//   * the K rows feeding score tile mt are permuted (sigma below) so that the
//     fp32 score registers, packed to bf16, are directly the B operand of the
//     P V product, whose A operand reads V^T rows of 8 consecutive keys;
//   * K and V^T tiles are double-buffered in LDS; the next tile's global
//     loads are issued before the current tile's MFMAs;
//   * online softmax in fp32 with exp2 and the scale folded into log2 units.
#include "nabla_device.h"
#include "nabla_launch.h"

namespace nabla {

// MFMA k-slot -> key row of score tile mt (0..3) for output row m (0..15):
// m = 4g + u maps to key 32*(mt/2) + 8g + 4*(mt%2) + u.
__device__ __forceinline__ int sigma_row(int mt, int m) {
    return 32 * (mt >> 1) + 8 * (m >> 2) + 4 * (mt & 1) + (m & 3);
}

template <int D, typename Tin>
__global__ __launch_bounds__(256, 2) void sparse_attn_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
    Tin *__restrict__ o, int S, int heads, int nrows, const int32_t *__restrict__ kv_nb,
    const int32_t *__restrict__ kv_inds, float scale_log2) {
    constexpr int KS = D / 32;               // MFMA k-steps of the score product
    constexpr int DT = D / 16;               // output d-tiles
    constexpr int LDK = D + 8;               // K tile row pitch (bf16)
    constexpr int LDV = kBlock + 8;          // V^T tile row pitch (bf16)
    constexpr int KCH = kBlock * D / 8 / 256;  // 16-byte K chunks per thread
    constexpr int DG = D / 8;                // 8-wide d groups of a V row

    __shared__ __attribute__((aligned(16))) bf16 Ks[2][kBlock * LDK];
    __shared__ __attribute__((aligned(16))) bf16 Vt[2][D * LDV];

    const int nb = S / kBlock;
    const int row = xcd_contiguous(blockIdx.x, nrows);
    const int i = row % nb;
    const int bh = row / nb;
    const int h = bh % heads;
    const int b = bh / heads;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, l16 = lane & 15;

    const int64_t tok = (int64_t)heads * D;  // elements between consecutive tokens
    const int64_t head0 = (int64_t)b * S * tok + (int64_t)h * D;

    int n = kv_nb[row];
    n = n < 0 ? 0 : (n > nb ? nb : n);
    const int32_t *list = kv_inds + (int64_t)row * nb;

    const int qtok = i * kBlock + w * 16 + l16;
    Tin *orow = o + head0 + (int64_t)qtok * tok;

    if (n == 0) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int u = 0; u < 4; ++u) orow[16 * dt + 4 * g + u] = (Tin)0.0f;
        return;
    }

    // Q rows of this wave as B operands: lane holds Q[qtok][32ks + 8g .. +7]
    bf16x8 qf[KS];
    {
        const Tin *qrow = q + head0 + (int64_t)qtok * tok;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = load8_bf16(qrow + 32 * ks + 8 * g);
    }

    // staging registers for one K tile and one V tile
    bf16x8 kreg[KCH];
    bf16x8 vreg[4];
    const int kvg = tid & 15, dg = tid >> 4;  // V: keys 4kvg..4kvg+3, dims 8dg..8dg+7
    const bool v_active = dg < DG;

    auto clampj = [&](int j) { return j < 0 ? 0 : (j >= nb ? nb - 1 : j); };
    auto fetch = [&](int j) {
        const Tin *kb = k + head0 + (int64_t)j * kBlock * tok;
        const Tin *vb = v + head0 + (int64_t)j * kBlock * tok;
#pragma unroll
        for (int it = 0; it < KCH; ++it) {
            const int id = it * 256 + tid;
            const int kr = id / DG, kc = id - kr * DG;
            kreg[it] = load8_bf16(kb + (int64_t)kr * tok + 8 * kc);
        }
        if (v_active) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                vreg[rr] = load8_bf16(vb + (int64_t)(4 * kvg + rr) * tok + 8 * dg);
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int it = 0; it < KCH; ++it) {
            const int id = it * 256 + tid;
            const int kr = id / DG, kc = id - kr * DG;
            *reinterpret_cast<bf16x8 *>(&Ks[buf][kr * LDK + 8 * kc]) = kreg[it];
        }
        if (v_active) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                bf16x4 col;
                col[0] = vreg[0][u];
                col[1] = vreg[1][u];
                col[2] = vreg[2][u];
                col[3] = vreg[3][u];
                *reinterpret_cast<bf16x4 *>(&Vt[buf][(8 * dg + u) * LDV + 4 * kvg]) = col;
            }
        }
    };

    f32x4 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    fetch(clampj(list[0]));
    stash(0);
    __syncthreads();

    for (int t = 0; t < n; ++t) {
        const int buf = t & 1;
        if (t + 1 < n) fetch(clampj(list[t + 1]));

        // S^T tiles: sacc[mt] holds keys sigma(mt, 4g+u), query l16
        f32x4 sacc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            sacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const bf16 *krow = &Ks[buf][sigma_row(mt, l16) * LDK + 8 * g];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(krow + 32 * ks);
                sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks], sacc[mt], 0, 0, 0);
            }
        }

        // online softmax (log2 units)
        float mloc = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                sacc[mt][u] *= scale_log2;
                mloc = fmaxf(mloc, sacc[mt][u]);
            }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        const float m_new = fmaxf(m_run, mloc);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        float psum = 0.0f;
        bf16x8 pb[2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float p = __builtin_amdgcn_exp2f(sacc[mt][u] - m_new);
                psum += p;
                pb[mt >> 1][4 * (mt & 1) + u] = (bf16)p;
            }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;

        // O^T += V^T P^T
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const bf16 *vrow = &Vt[buf][(16 * dt + l16) * LDV + 8 * g];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(vrow + 32 * kk);
                oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[kk], oacc[dt], 0, 0, 0);
            }
        }

        if (t + 1 < n) stash(buf ^ 1);
        __syncthreads();
    }

    float lsum = l_run + __shfl_xor(l_run, 16);
    lsum += __shfl_xor(lsum, 32);
    const float inv = 1.0f / lsum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        if constexpr (sizeof(Tin) == 2) {
            bf16x4 r;
#pragma unroll
            for (int u = 0; u < 4; ++u) r[u] = (bf16)(oacc[dt][u] * inv);
            *reinterpret_cast<bf16x4 *>(orow + 16 * dt + 4 * g) = r;
        } else {
            *reinterpret_cast<float4 *>(orow + 16 * dt + 4 * g) =
                make_float4(oacc[dt][0] * inv, oacc[dt][1] * inv, oacc[dt][2] * inv,
                            oacc[dt][3] * inv);
        }
    }
}

template <int D, typename Tin>
static hipError_t launch_attn_t(const void *q, const void *k, const void *v, int B, int S,
                                int heads, const int32_t *kv_nb, const int32_t *kv_inds,
                                float scale_log2, void *o, hipStream_t stream) {
    const int nrows = B * heads * (S / kBlock);
    hipLaunchKernelGGL((sparse_attn_kernel<D, Tin>), dim3(nrows), dim3(256), 0, stream,
                       (const Tin *)q, (const Tin *)k, (const Tin *)v, (Tin *)o, S, heads, nrows,
                       kv_nb, kv_inds, scale_log2);
    return hipGetLastError();
}

hipError_t launch_sparse_attn(const void *q, const void *k, const void *v, bool bf16_in,
                              int B, int S, int heads, int D, const int32_t *kv_nb,
                              const int32_t *kv_inds, float scale, void *o,
                              hipStream_t stream) {
    const float scale_log2 = scale * 1.4426950408889634f;
    if (D == 128)
        return bf16_in ? launch_attn_t<128, bf16>(q, k, v, B, S, heads, kv_nb, kv_inds,
                                                  scale_log2, o, stream)
                       : launch_attn_t<128, float>(q, k, v, B, S, heads, kv_nb, kv_inds,
                                                   scale_log2, o, stream);
    return bf16_in ? launch_attn_t<64, bf16>(q, k, v, B, S, heads, kv_nb, kv_inds, scale_log2, o,
                                             stream)
                   : launch_attn_t<64, float>(q, k, v, B, S, heads, kv_nb, kv_inds, scale_log2,
                                              o, stream);
}

}  // namespace nabla
