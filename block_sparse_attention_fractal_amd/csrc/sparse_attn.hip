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
// Design (CDNA4 / gfx950):
//   * K/V reuse across query blocks.  The lists of neighbouring query blocks
//     overlap heavily (the STA window, and content that changes slowly in time
//     and space).  One workgroup takes a group of G query blocks -- G = 2: the
//     same tile in two consecutive frames; G = 4: a 2 (time) x 1 x 2 (width)
//     box; consecutive blocks when the tile grid is unknown -- and walks the
//     union of their lists once in ascending block order.  Each K/V tile is
//     fetched from HBM/L2 once per group and shared through LDS by every member
//     that lists it.
//   * 2G waves = G query blocks x 2 halves of 32 query rows; a wave keeps its
//     32 query rows in registers as MFMA operands for the whole walk and skips
//     the tiles its block does not list.  With G = 2 two workgroups share a CU,
//     so each SIMD runs waves of two independent walks.
//   * v_mfma_f32_32x32x16_bf16, fp32 accumulation.  Scores are formed
//     transposed, S^T = K Q^T, so each lane owns one query row and 32 keys of a
//     tile (the other 32 sit in lane ^ 32): the row max is in-lane work plus
//     one lane swap, the row sum stays lane-local until the end.
//   * K rows are read from LDS in a permuted order (sigma) chosen so that the
//     fp32 score registers j = 8p .. 8p+7, packed to bf16, are the B operand
//     of the P V product for 16 consecutive keys; V is read back transposed
//     with ds_read_b64_tr_b16 as the A operand of O^T = V^T P^T.
//   * Tiles move global -> registers (16-byte loads, fp32 inputs rounded to
//     bf16 here) -> LDS (XOR-swizzled 16-byte chunks, two stages): the loads
//     for tile u+2 are in flight while tile u is computed.
//   * Online softmax in fp32, log2 domain: Q is pre-multiplied by
//     scale * log2(e), the score accumulators start at minus the row's
//     reference max, so exp2 reads the MFMA output directly.  The reference is
//     only raised when a tile exceeds it by more than 16 (and on the row's
//     first tile), so the O rescale is rare.  The row sum is a bf16 dot
//     product of the packed weights with ones (the same weights P V uses).
#include "nabla_device.h"
#include "nabla_launch.h"

namespace nabla {

typedef float f32x16 __attribute__((ext_vector_type(16)));
#define NABLA_LDS __attribute__((address_space(3)))

#ifndef NABLA_ATTN_GROUP
#define NABLA_ATTN_GROUP 4
#endif
constexpr int kGroup = NABLA_ATTN_GROUP;  // query blocks per workgroup (2 or 4)
constexpr int kAttnWaves = 2 * kGroup;
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr int kMaxWords = 4096 / 64;  // bitmap words for up to 4096 blocks per row
static_assert(kGroup == 2 || kGroup == 4, "group of 2 or 4 query blocks");

// Key row (within a 32-row score tile) fed to MFMA row m: bit layout
// m = a(2) hh(1) b(2)  ->  key = (a>>1)<<4 | hh<<3 | (a&1)<<2 | b.
__device__ __forceinline__ int sigma32(int m) {
    const int a = m >> 3, hh = (m >> 2) & 1, b = m & 3;
    return ((a >> 1) << 4) | (hh << 3) | ((a & 1) << 2) | b;
}

__device__ __forceinline__ uint64_t uniform_u64(uint64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// 16-byte chunk swizzles (CH chunks per row) of the K and V tiles in LDS.
template <int CH>
__device__ __forceinline__ int kswz(int kv) { return kv & (CH - 1); }
template <int CH>
__device__ __forceinline__ int vswz(int kv) { return (kv & 3) * (CH / 4); }

template <int D>
struct AttnShared {
    bf16 ks[2][kBlock * D];
    bf16 vs[2][kBlock * D];
    uint64_t qmask[kGroup][kMaxWords];
    uint64_t umask[kMaxWords];
};

template <int D, typename Tin>
__global__ __launch_bounds__(kAttnThreads) void sparse_attn_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
    Tin *__restrict__ o, int S, int heads, int Tt, int Ht, int Wt, int groups_per_bh,
    int ngroups, const int32_t *__restrict__ kv_nb, const int32_t *__restrict__ kv_inds,
    float scale_log2) {
    constexpr int KS = D / 16;          // k-steps of the score product (16 dims each)
    constexpr int DT = D / 32;          // 32-wide output d tiles
    constexpr int CH = D / 8;           // 16-byte chunks per row
    constexpr int ROWB = D * 2;         // bytes per K/V row in LDS
    constexpr int CHUNKS = kBlock * CH; // 16-byte chunks per K (or V) tile
    constexpr int CPT = CHUNKS / kAttnThreads;  // chunks per thread per tile (K and V each)
    static_assert(CPT >= 1, "tile too small for the workgroup");

    __shared__ __attribute__((aligned(1024))) AttnShared<D> sh;

    const int nb = S / kBlock;
    const int nwords = (nb + 63) >> 6;
    const int grp = xcd_contiguous(blockIdx.x, ngroups);
    const int bh = grp / groups_per_bh;
    const int gi = grp % groups_per_bh;
    const int h = bh % heads;
    const int b = bh / heads;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;

    // the G members of this group (-1 = no block in this slot)
    int member[kGroup];
    if (Tt > 0) {
        // kGroup 4: a 2 (time) x 1 x 2 (width) box; kGroup 2: 2 frames of one tile
        const int cw = kGroup == 4 ? (Wt + 1) >> 1 : Wt;
        const int a = gi / (Ht * cw), hh = (gi / cw) % Ht, c = gi % cw;
#pragma unroll
        for (int s = 0; s < kGroup; ++s) {
            const int t = 2 * a + (kGroup == 4 ? (s >> 1) : s);
            const int ww = kGroup == 4 ? 2 * c + (s & 1) : c;
            member[s] = (t < Tt && ww < Wt) ? (t * Ht + hh) * Wt + ww : -1;
        }
    } else {
#pragma unroll
        for (int s = 0; s < kGroup; ++s) {
            const int i = gi * kGroup + s;
            member[s] = i < nb ? i : -1;
        }
    }

    // ---- per-member bitmaps of listed blocks, and their union
    for (int e = tid; e < kGroup * kMaxWords; e += kAttnThreads) (&sh.qmask[0][0])[e] = 0ull;
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kGroup; ++s) {
        if (member[s] < 0) continue;
        const int64_t row = (int64_t)bh * nb + member[s];
        int n = kv_nb[row];
        n = n < 0 ? 0 : (n > nb ? nb : n);
        const int32_t *list = kv_inds + row * nb;
        for (int e = tid; e < n; e += kAttnThreads) {
            int j = list[e];
            j = j < 0 ? 0 : (j >= nb ? nb - 1 : j);
            atomicOr((unsigned long long *)&sh.qmask[s][j >> 6], 1ull << (j & 63));
        }
    }
    __syncthreads();
    for (int wd = tid; wd < nwords; wd += kAttnThreads)
    {
        uint64_t u = 0ull;
#pragma unroll
        for (int s = 0; s < kGroup; ++s) u |= sh.qmask[s][wd];
        sh.umask[wd] = u;
    }
    __syncthreads();

    // ---- this wave: member slot and 32-row half
    const int slot = w >> 1;
    const int myblk = member[slot];
    const int64_t tok = (int64_t)heads * D;
    const int64_t head0 = (int64_t)b * S * tok + (int64_t)h * D;
    const int qtok = (myblk < 0 ? 0 : myblk) * kBlock + (w & 1) * 32 + l32;

    // Q^T as B operands, pre-multiplied by scale * log2(e) so that the score
    // MFMAs produce log2-domain logits directly
    bf16x8 qf[KS];
    if (myblk >= 0) {
        const Tin *qr = q + head0 + (int64_t)qtok * tok + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 x = load8_bf16(qr + 16 * ks);
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[ks][e] = (bf16)((float)x[e] * scale_log2);
        }
    }
    // Retire the Q loads here: otherwise they are still counted as pending at
    // the loop header, and the score MFMAs of every tile would wait (in-order
    // vmcnt) for the K/V prefetch issued just before them.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    // ---- union cursor (wave-uniform, kept in scalar registers): ascending set bits of umask
    int cur_word = 0;
    uint64_t cur_bits = uniform_u64(sh.umask[0]);
    auto next_block = [&]() -> int {
        while (cur_bits == 0ull) {
            if (++cur_word >= nwords) return -1;
            cur_bits = uniform_u64(sh.umask[cur_word]);
        }
        const int bit = __builtin_ctzll(cur_bits);
        cur_bits &= cur_bits - 1;
        return (cur_word << 6) | bit;
    };
    // this wave's membership bits of word `mword` (scalar; reloaded when the walk moves on)
    int mword = -1;
    uint64_t mbits = 0ull;

    // ---- staging: K and V chunks of one tile in registers
    bf16x8 kst[CPT], vst[CPT];
    auto fetch = [&](int j) {
        const Tin *kb = k + head0 + (int64_t)j * kBlock * tok;
        const Tin *vb = v + head0 + (int64_t)j * kBlock * tok;
#pragma unroll
        for (int r = 0; r < CPT; ++r) {
            const int e = r * kAttnThreads + tid;
            const int kv = e / CH, c = e % CH;
            kst[r] = load8_bf16(kb + (int64_t)kv * tok + 8 * c);
            vst[r] = load8_bf16(vb + (int64_t)kv * tok + 8 * c);
        }
    };
    auto stash = [&](int stage) {
        char *kd = reinterpret_cast<char *>(sh.ks[stage]);
        char *vd = reinterpret_cast<char *>(sh.vs[stage]);
#pragma unroll
        for (int r = 0; r < CPT; ++r) {
            const int e = r * kAttnThreads + tid;
            const int kv = e / CH, c = e % CH;
            *reinterpret_cast<bf16x8 *>(kd + kv * ROWB + ((c ^ kswz<CH>(kv)) << 4)) = kst[r];
            *reinterpret_cast<bf16x8 *>(vd + kv * ROWB + ((c ^ vswz<CH>(kv)) << 4)) = vst[r];
        }
    };

    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[dt][j] = 0.0f;
    float m_ref = 0.0f;       // reference max of the row, log2 units (raised lazily)
    bool m_valid = false;     // set by the row's first tile
    float l_run = 0.0f;       // this lane's part of the row sum

    int cur = next_block();
    int nxt = -1;
    if (cur >= 0) {
        fetch(cur);
        stash(0);
        nxt = next_block();
        if (nxt >= 0) fetch(nxt);
    }
    __syncthreads();

    for (int it = 0; cur >= 0; ++it) {
        const int stage = it & 1;
        int nxt2 = -1;
        if (nxt >= 0) {
            stash(stage ^ 1);  // tile it+1 -> the other stage (free since the last barrier)
            nxt2 = next_block();
            if (nxt2 >= 0) fetch(nxt2);
        }
        if (myblk >= 0 && (cur >> 6) != mword) {
            mword = cur >> 6;
            mbits = uniform_u64(sh.qmask[slot][mword]);
        }
        const bool mine = myblk >= 0 && ((mbits >> (cur & 63)) & 1ull);
        if (mine) {
            const char *kb = reinterpret_cast<const char *>(sh.ks[stage]);
            const char *vb = reinterpret_cast<const char *>(sh.vs[stage]);
            // S^T - m = K Q^T (log2 units) for the two 32-key halves of the tile; the
            // accumulators start at -m so the MFMAs also subtract the reference max
            const float init = m_valid ? -m_ref : 0.0f;
            f32x16 sacc[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
                for (int j = 0; j < 16; ++j) sacc[mt][j] = init;
                const int kv = 32 * mt + sigma32(l32);
                const char *krow = kb + kv * ROWB;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int c = 2 * ks + hi;
                    const bf16x8 a =
                        *reinterpret_cast<const bf16x8 *>(krow + ((c ^ kswz<CH>(kv)) << 4));
                    sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc[mt], 0, 0, 0);
                }
            }
            // Lazy reference max: only when this lane's logits exceed the reference by
            // more than 16 (log2 units), or on the row's first tile, is the reference
            // raised to the row max and O, l rescaled (wave-uniform branch).
            float lm = fmaxf(sacc[0][0], sacc[1][0]);
#pragma unroll
            for (int j = 1; j < 16; ++j) lm = fmaxf(lm, fmaxf(sacc[0][j], sacc[1][j]));
            const bool need = !m_valid || lm > 16.0f;
            if (__builtin_amdgcn_ballot_w64(need) != 0ull) {
                const float rm = fmaxf(lm, __shfl_xor(lm, 32));  // row max (shifted units)
                const bool row_need = !m_valid || rm > 16.0f;     // same in lanes l, l^32
                const float delta = row_need ? rm : 0.0f;
                const float alpha = m_valid ? __builtin_amdgcn_exp2f(-delta) : 0.0f;
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) sacc[mt] -= delta;
                m_ref = (m_valid ? m_ref : 0.0f) + delta;
                m_valid = true;
            }
            bf16x8 pb[2][2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    pb[mt][j >> 3][j & 7] = (bf16)__builtin_amdgcn_exp2f(sacc[mt][j]);
            // row sum of the bf16 weights the P V product uses (dot with ones)
            {
                typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
                const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
                float part[2] = {0.0f, 0.0f};
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int p = 0; p < 2; ++p)
#pragma unroll
                        for (int e = 0; e < 8; e += 2) {
                            const bf16x2 pr = {pb[mt][p][e], pb[mt][p][e + 1]};
                            part[p] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, part[p], false);
                        }
                l_run += part[0] + part[1];
            }
            // O^T += V^T P^T: 4 k-steps of 16 keys (mt, p); the 8 transpose reads of
            // an output d-tile are issued together, ahead of its 4 MFMAs
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                bf16x8 va[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int mt = kk >> 1, p = kk & 1;
#pragma unroll
                    for (int r = 0; r < 2; ++r) {
                        const int g16 = lane >> 4, s = lane & 15;
                        const int kv = 32 * mt + 16 * p + 8 * (g16 >> 1) + 4 * r + (s >> 2);
                        const int d = 32 * dt + 16 * (g16 & 1) + 4 * (s & 3);
                        const int c = (d >> 3) ^ vswz<CH>(kv);
                        const char *addr = vb + kv * ROWB + (c << 4) + (d & 7) * 2;
                        const bf16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                            (NABLA_LDS bf16x4 *)(addr));
                        va[kk][4 * r + 0] = x[0];
                        va[kk][4 * r + 1] = x[1];
                        va[kk][4 * r + 2] = x[2];
                        va[kk][4 * r + 3] = x[3];
                    }
                }
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kk], pb[kk >> 1][kk & 1],
                                                                       oacc[dt], 0, 0, 0);
            }
        }
        __syncthreads();  // stage it+1 written; everyone done with stage it
        cur = nxt;
        nxt = nxt2;
    }

    if (myblk < 0) return;
    const float lsum = l_run + __shfl_xor(l_run, 32);
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;  // empty list -> O = 0
    Tin *orow = o + head0 + (int64_t)qtok * tok;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            Tin *dst = orow + 32 * dt + 8 * jj + 4 * hi;
            if constexpr (sizeof(Tin) == 2) {
                bf16x4 r;
#pragma unroll
                for (int u = 0; u < 4; ++u) r[u] = (bf16)(oacc[dt][4 * jj + u] * inv);
                *reinterpret_cast<bf16x4 *>(dst) = r;
            } else {
                *reinterpret_cast<float4 *>(dst) =
                    make_float4(oacc[dt][4 * jj] * inv, oacc[dt][4 * jj + 1] * inv,
                                oacc[dt][4 * jj + 2] * inv, oacc[dt][4 * jj + 3] * inv);
            }
        }
    }
}

template <int D, typename Tin>
static hipError_t launch_attn_t(const void *q, const void *k, const void *v, int B, int S,
                                int heads, int Tt, int Ht, int Wt, const int32_t *kv_nb,
                                const int32_t *kv_inds, float scale_log2, void *o,
                                hipStream_t stream) {
    const int nb = S / kBlock;
    const int gpb = Tt > 0 ? ((Tt + 1) / 2) * Ht * (kGroup == 4 ? (Wt + 1) / 2 : Wt)
                           : (nb + kGroup - 1) / kGroup;
    const int ngroups = B * heads * gpb;
    hipLaunchKernelGGL((sparse_attn_kernel<D, Tin>), dim3(ngroups), dim3(kAttnThreads), 0, stream,
                       (const Tin *)q, (const Tin *)k, (const Tin *)v, (Tin *)o, S, heads, Tt, Ht,
                       Wt, gpb, ngroups, kv_nb, kv_inds, scale_log2);
    return hipGetLastError();
}

hipError_t launch_sparse_attn(const void *q, const void *k, const void *v, bool bf16_in,
                              int B, int S, int heads, int D, int Tt, int Ht, int Wt,
                              const int32_t *kv_nb, const int32_t *kv_inds, float scale, void *o,
                              hipStream_t stream) {
    const float scale_log2 = scale * 1.4426950408889634f;
    if (D == 128)
        return bf16_in ? launch_attn_t<128, bf16>(q, k, v, B, S, heads, Tt, Ht, Wt, kv_nb,
                                                  kv_inds, scale_log2, o, stream)
                       : launch_attn_t<128, float>(q, k, v, B, S, heads, Tt, Ht, Wt, kv_nb,
                                                   kv_inds, scale_log2, o, stream);
    return bf16_in ? launch_attn_t<64, bf16>(q, k, v, B, S, heads, Tt, Ht, Wt, kv_nb, kv_inds,
                                             scale_log2, o, stream)
                   : launch_attn_t<64, float>(q, k, v, B, S, heads, Tt, Ht, Wt, kv_nb, kv_inds,
                                              scale_log2, o, stream);
}

}  // namespace nabla
