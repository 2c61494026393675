// sparse_attn_bwd.hip -- gradients of the NABLA block-sparse attention on gfx950.
//
// The forward (sparse_attn.hip) computes, for each query row r of block i,
// O_r = softmax(scale q_r K_J^T) V_J over the tokens J of the kv blocks listed for i
// (full 64 x 64 blocks: "nabla" page, NablaAttentionImpl.forward and nablaT_v2's
// BlockMask creation).  The pages train with this attention (NABLA summary page,
// Results: the training speed-up; flex attention's backward is the gradient of the
// same masked softmax).  With the forward's per-row log-sum-exp lse and a given dO:
//   P  = exp(scale q k^T - lse),   dP = dO V^T,   Delta = rowsum(dO * O)
//   dS = P (dP - Delta),   dq = scale dS K,   dk = scale dS^T Q,   dv = P^T dO.
//
// Kernels (bf16 tensors, fp32 accumulation):
//   bwd_delta_kernel          Delta per (b, h, token) from the stored O and dO.
//   bwd_tlist_*               transposed lists: for kv block j of (b, h), the query
//                             blocks whose lists hold j, ascending.
//   bwd_dq4_kernel            D = 128: one workgroup per query block walks its kv list:
//                             S^T = K Q^T, dP^T = V dO^T, dS^T, dq^T += K^T dS^T
//                             (v_mfma_f32_32x32x16_bf16, 32 rows and 32 keys per wave,
//                             2 waves per SIMD; the key halves' parts added at the end).
//   bwd_dq_kernel             the same at D = 64 (32 rows and all 64 keys per wave).
//   bwd_dkdv16_kernel         D = 128: one workgroup per kv block walks its query list:
//                             S = Q K^T, dP = dO V^T, dS, dv^T += dO^T P, dk^T += Q^T dS
//                             (v_mfma_f32_16x16x32_bf16, 16 keys per wave, 2 waves per SIMD).
//   bwd_dkdv_kernel           the same at D = 64 (32x32x16, 32 keys per wave).
// Both gradient kernels recompute S and dP, so every output row is written once by one
// workgroup in a fixed order: no atomics, and the results are deterministic.
//
// Padded layouts (a T x H x W latent grid whose H or W is not a multiple of 8: the last
// patch row / column is partial, the sibling "video_sparse_attn" page's variable block
// sizes): the padding positions are never keys, as in the forward.  dq sets dS to 0 at
// them on partial tiles; dk and dv are 0 there.  The instances without kPad carry none
// of that code.
//
// Layout tricks shared with the forward: a lane owns one column of each 32 x 32
// product; the rows fed to the first product are permuted (sigma32) so that its fp32
// results j = 8p .. 8p+7, packed to bf16, are directly the B operand of the second
// product over 16 consecutive rows; transposed operands come from ds_read_b64_tr_b16.
#include "attn_tile.h"
#include "nabla_launch.h"

namespace nabla {

namespace {

constexpr int kBwdThreads = 128;  // 2 waves: the two 32-row (or 32-key) halves of a block
constexpr float kLog2e = 1.4426950408889634f;

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// 16-byte chunk swizzle of the tiles in LDS.  Each tile is read two ways: as rows (16 bytes
// per lane, rfrag: the 16 lanes of a cycle take 16 rows with distinct row % 16) and
// transposed (8 bytes per lane, tfrag: the 32 lanes of a cycle take 4 rows R .. R + 3,
// R % 4 = 0, times chunks 4 t .. 4 t + 3, in two half chunks).  On the 64 four-byte banks
// both are free of conflicts when the swizzle is a bijection on row % 16 (rows) and sends
// the row bits that vary inside a transposed read to the chunk bits that do not:
//   CH = 16 (256-byte rows): bits 0-1 of the row to bits 2-3 of the chunk, bits 2-3 to 0-1;
//   CH = 8 (128-byte rows, two per bank line): row bit 1 to chunk bit 2, bits 2-3 to 0-1.
// (The forward's row swizzle, row % CH, makes the transposed reads 4-way conflicted.)
template <int CH>
__device__ __forceinline__ int bswz(int row) {
    static_assert(CH == 16 || CH == 8, "D = 128 or 64");
    if constexpr (CH == 16)
        return ((row & 3) << 2) | ((row >> 2) & 3);
    else
        return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Transposing read of a bf16 tile in LDS (rows of ROWB bytes, 16-byte chunks XOR-swizzled
// by bswz): the A operand [32 (d) x 16 (rows)] of k-step kk = 2 mt + p, output d tile dt,
// i.e. lane l gets tile[32 mt + 16 p + 8 (l / 32) + 0..7][32 dt + l % 32].
template <int D>
__device__ __forceinline__ bf16x8 tfrag(const char *tb, int lane, int dt, int kk) {
    constexpr int CH = D / 8, ROWB = 2 * D;
    const int g16 = lane >> 4, sl = lane & 15, mt = kk >> 1, p = kk & 1;
    bf16x8 a;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int row = 32 * mt + 16 * p + 8 * (g16 >> 1) + 4 * r + (sl >> 2);
        const int d = 32 * dt + 16 * (g16 & 1) + 4 * (sl & 3);
        const int c = (d >> 3) ^ bswz<CH>(row);
        const bf16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (NABLA_LDS bf16x4 *)(tb + row * ROWB + (c << 4) + (d & 7) * 2));
        a[4 * r + 0] = x[0];
        a[4 * r + 1] = x[1];
        a[4 * r + 2] = x[2];
        a[4 * r + 3] = x[3];
    }
    return a;
}

// Row fragment: lane l gets tile[row][16 ks + 8 (l / 32) + 0..7] (A operand of a product
// over d for row `row`).
template <int D>
__device__ __forceinline__ bf16x8 rfrag(const char *tb, int row, int hi, int ks) {
    constexpr int CH = D / 8, ROWB = 2 * D;
    const int c = 2 * ks + hi;
    return *reinterpret_cast<const bf16x8 *>(tb + row * ROWB + ((c ^ bswz<CH>(row)) << 4));
}

// Per-lane byte offsets (global side) of the 16-byte chunks this thread moves for one
// 64-row tile: chunk e = r * 128 + tid lands at byte 16 e of the LDS tile, i.e. row e / CH,
// position e % CH, so the lane fetches global chunk (e % CH) ^ bswz(row).
template <int D>
__device__ __forceinline__ void tile_offsets(int tid, int64_t tok, uint32_t (&off)[kBlock * D / 8 / kBwdThreads]) {
    constexpr int CH = D / 8;
#pragma unroll
    for (int r = 0; r < kBlock * CH / kBwdThreads; ++r) {
        const int e = r * kBwdThreads + tid;
        const int row = e / CH, cpos = e % CH;
        off[r] = (uint32_t)((row * tok + 8 * (cpos ^ bswz<CH>(row))) * 2);
    }
}

// Gradient accumulators live in AGPRs for the whole walk: their MFMAs are issued from
// inline asm with the accumulator bound to AGPRs ("+a"), while the score products stay
// compiler builtins in VGPRs (the build selects the VGPR form for MFMAs), which the softmax
// reads.  acc += a b (v_mfma_f32_32x32x16_bf16).
//
// The compiler's hazard recognizer does not look inside inline asm, so these asm blocks
// supply the wait states the CDNA3/CDNA4 ISA's table of required independent instructions
// asks for around XDL (matrix) ops; every case that can occur here:
//   * a and b written by a VALU instruction just before (dS and P packed to bf16, Q^T / K^T
//     fragments assembled in registers): VALU write -> MFMA read of SrcA/B needs 2 wait
//     states; `s_nop 4` gives 5.
//   * a and b read from LDS: the compiler itself waits (lgkmcnt) for the value, as for any
//     use of an asm input operand.
//   * acc zeroed by v_accvgpr_write before the walk: a VALU-class write read as SrcC; the
//     same 5 wait states cover it.
//   * consecutive mfma_acc on one accumulator: SrcC is exactly the previous op's vdst and the
//     ops have one opcode, the back-to-back case the hardware forwards (0 wait states);
//     chains on different accumulators have no dependence.
//   * the walk never writes an accumulator from VALU code while an MFMA reads it (no
//     write-after-read case): the accumulators are only read after acc_settle below.
__device__ __forceinline__ void mfma_acc(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
    asm("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Waits out the last MFMAs writing the accumulators before VALU instructions (or
// v_accvgpr_read) read them: an XDL op's vdst read by VALU needs its pass count + 2 wait
// states, at most 18 for the 16-pass 32 x 32 shapes; three `s_nop 7` give 24.  The asm names
// every accumulator as in and out, so no read of them can be scheduled above it.
template <int DT>
__device__ __forceinline__ void acc_settle(f32x16 (&acc)[DT]) {
    static_assert(DT == 2 || DT == 4, "2 or 4 d tiles");
    if constexpr (DT == 4)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]));
    else
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[0]), "+a"(acc[1]));
}

// Stores a [D x 32] fp32 product tile set (acc[dt]: rows d = 32 dt + ..., column = this
// lane's row) times `mul` as bf16 into row `dst` (the lane's row, D contiguous values).
template <int D>
__device__ __forceinline__ void store_rowT(bf16 *dst, const f32x16 (&acc)[D / 32], int hi, float mul) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            bf16x4 r;
#pragma unroll
            for (int u = 0; u < 4; ++u) r[u] = (bf16)(acc[dt][4 * jj + u] * mul);
            *reinterpret_cast<bf16x4 *>(dst + 32 * dt + 8 * jj + 4 * hi) = r;
        }
}

}  // namespace

// ---- Delta[bh][s] = sum_d dO[b, s, h, d] * O[b, s, h, d] (fp32, from the bf16 values).
// D / 8 lanes per (token, head) row, 8 elements each, reduced by lane shuffles.
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const bf16 *__restrict__ o,
                                                       const bf16 *__restrict__ dout,
                                                       float *__restrict__ delta, int S,
                                                       int heads, int64_t nrows) {
    constexpr int L = D / 8;
    const int64_t r = ((int64_t)blockIdx.x * 256 + threadIdx.x) / L;
    const int c = threadIdx.x % L;
    float acc = 0.0f;
    if (r < nrows) {
        const bf16x8 x = load8_bf16(o + r * D + 8 * c);
        const bf16x8 y = load8_bf16(dout + r * D + 8 * c);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)x[e], (float)y[e], acc);
    }
#pragma unroll
    for (int m = 1; m < L; m <<= 1) acc += __shfl_xor(acc, m);
    if (c == 0 && r < nrows) {
        const int64_t tok = r / heads;  // b * S + s
        const int h = (int)(r % heads);
        const int64_t b = tok / S, s = tok % S;
        delta[(b * heads + h) * S + s] = acc;
    }
}

// ---- transposed lists.  tmat[bh][j][i] = 1 iff block j is listed for query block i.
__global__ __launch_bounds__(256) void bwd_tlist_zero_kernel(uint4 *__restrict__ t, int64_t n16) {
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n16; e += (int64_t)gridDim.x * 256)
        t[e] = z;
}

// grid = B*heads*nb query rows
__global__ __launch_bounds__(256) void bwd_tlist_scatter_kernel(const int32_t *__restrict__ kv_nb,
                                                               const int32_t *__restrict__ kv_inds,
                                                               int nb, uint8_t *__restrict__ tmat) {
    const int64_t row = blockIdx.x;
    const int64_t bh = row / nb;
    const int i = (int)(row % nb);
    const int n = clamp_count(kv_nb[row], nb);
    for (int e = threadIdx.x; e < n; e += 256) {
        const int j = clamp_block(kv_inds[row * nb + e], nb);
        tmat[(bh * nb + j) * nb + i] = 1;
    }
}

// one wave per kv block (bh, j): q_inds[bh][j][0 .. q_nb) = the i with tmat[bh][j][i], ascending
__global__ __launch_bounds__(256) void bwd_tlist_compact_kernel(const uint8_t *__restrict__ tmat,
                                                               int nb, int64_t nrows,
                                                               int32_t *__restrict__ q_nb,
                                                               int32_t *__restrict__ q_inds) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= nrows) return;  // wave-uniform; no barrier in this kernel
    const int lane = threadIdx.x & 63;
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const uint8_t *t = tmat + row * nb;
    int base = 0;
    for (int c0 = 0; c0 < nb; c0 += 64) {
        const int i = c0 + lane;
        const bool bit = i < nb && t[i] != 0;
        const uint64_t bal = __ballot(bit);
        if (bit) q_inds[row * nb + base + __popcll(bal & below)] = i;
        base += __popcll(bal);
    }
    if (lane == 0) q_nb[row] = base;
}

// ---- dq.  One workgroup (2 waves) per query block i of (b, h); wave w owns rows 32 w ..
// 32 w + 31, lane (l32, hi) row 32 w + l32.  K and V tiles of the listed blocks go through
// a 2-stage LDS ring (direct global -> LDS loads, one tile ahead).
// Patch rows / columns of block j that are tokens (8 x 8 unless the grid is padded).
__device__ __forceinline__ void patch_extent(int j, int Ht, int Wt, int Hv, int Wv, int &vr,
                                             int &vc) {
    const int th = (j / Wt) % Ht, tw = j % Wt;
    vr = min(kTile, Hv - th * kTile);
    vc = min(kTile, Wv - tw * kTile);
}

template <int D, bool kPad>
__global__ __launch_bounds__(kBwdThreads) void bwd_dq_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ delta,
    bf16 *__restrict__ dq, int S, int heads, const int32_t *__restrict__ kv_nb,
    const int32_t *__restrict__ kv_inds, const int32_t *__restrict__ order, float scale,
    float scale_log2, int Ht, int Wt, int Hv, int Wv) {
    constexpr int KS = D / 16, DT = D / 32, CPT = kBlock * D / 8 / kBwdThreads;
    __shared__ __attribute__((aligned(1024))) bf16 ksh[2][kBlock * D];
    __shared__ __attribute__((aligned(1024))) bf16 vsh[2][kBlock * D];

    const int nb = S / kBlock;
    const int64_t row = order[blockIdx.x];  // longest lists first, within phases of heads
    const int bh = (int)(row / nb), i = (int)(row % nb);
    const int b = bh / heads, h = bh % heads;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hi = lane >> 5;
    const int64_t tok = (int64_t)heads * D;
    const int64_t head0 = (int64_t)b * S * tok + (int64_t)h * D;
    const int qtok = i * kBlock + 32 * w + l32;
    const int n = clamp_count(kv_nb[row], nb);
    const int32_t *list = kv_inds + row * nb;

    // Q^T (times scale * log2 e: the score products give log2-domain logits) and dO^T as
    // B operands: lane (l32, hi) holds d = 16 ks + 8 hi + 0..7 of its row
    bf16x8 qf[KS], df[KS];
    {
        const bf16 *qr = q + head0 + (int64_t)qtok * tok + 8 * hi;
        const bf16 *dr = dout + head0 + (int64_t)qtok * tok + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 x = load8_bf16(qr + 16 * ks);
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[ks][e] = (bf16)((float)x[e] * scale_log2);
            df[ks] = load8_bf16(dr + 16 * ks);
        }
    }
    const float lse2 = lse[(int64_t)bh * S + qtok] * kLog2e;
    const float dl = delta[(int64_t)bh * S + qtok];

    uint32_t off[CPT];
    tile_offsets<D>(tid, tok, off);
    const uint32_t ldk = __builtin_amdgcn_readfirstlane(lds_offset(ksh[0]) + w * 64 * 16);
    const uint32_t ldv = __builtin_amdgcn_readfirstlane(lds_offset(vsh[0]) + w * 64 * 16);
    auto issue = [&](int jj, int stage) {
        const int j = __builtin_amdgcn_readfirstlane(clamp_block(jj, nb));
        const bf16 *kb = k + head0 + (int64_t)j * kBlock * tok;
        const bf16 *vb = v + head0 + (int64_t)j * kBlock * tok;
#pragma unroll
        for (int r = 0; r < CPT; ++r) {
            const uint32_t sb = stage * (kBlock * D * 2) + r * kBwdThreads * 16;
            lds_direct16_sv(kb, off[r], ldk + sb);
            lds_direct16_sv(vb, off[r], ldv + sb);
        }
    };

    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = splat16(0.0f);

    if (n > 0) issue(list[0], 0);
    vm_wait<0>();
    __syncthreads();
    const int kv0 = sigma32(l32), kv1 = 32 + sigma32(l32);
    for (int u = 0; u < n; ++u) {
        const int st = u & 1;
        if (u + 1 < n) issue(list[u + 1], st ^ 1);
        const char *kb = reinterpret_cast<const char *>(ksh[st]);
        const char *vb = reinterpret_cast<const char *>(vsh[st]);
        // S^T - lse (log2 units) and dP^T for the two 32-key halves.  The K and V row
        // fragments are read KLA k-steps ahead of their MFMAs (a ring of KLA + 1 k-steps;
        // the sched_barrier fences keep the reads from sinking next to their uses).
        f32x16 sacc[2], pacc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            sacc[mt] = splat16(-lse2);
            pacc[mt] = splat16(-dl);
        }
        constexpr int KLA = 3;
        bf16x8 fr[KLA + 1][4];
        auto fread = [&](int ks) {
            fr[ks & KLA][0] = rfrag<D>(kb, kv0, hi, ks);
            fr[ks & KLA][1] = rfrag<D>(kb, kv1, hi, ks);
            fr[ks & KLA][2] = rfrag<D>(vb, kv0, hi, ks);
            fr[ks & KLA][3] = rfrag<D>(vb, kv1, hi, ks);
        };
#pragma unroll
        for (int ks = 0; ks < KLA; ++ks) fread(ks);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + KLA < KS) fread(ks + KLA);
            __builtin_amdgcn_sched_barrier(0);
            const bf16x8(&f)[4] = fr[ks & KLA];
            sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[0], qf[ks], sacc[0], 0, 0, 0);
            sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[1], qf[ks], sacc[1], 0, 0, 0);
            pacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[2], df[ks], pacc[0], 0, 0, 0);
            pacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[3], df[ks], pacc[1], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // the first d tile's K^T fragments, read under the VALU work below
        bf16x8 kt[2][4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) kt[0][kk] = tfrag<D>(kb, lane, 0, kk);
        // dS^T = P^T (dP^T - Delta), packed: registers 8p .. 8p+7 = 16 consecutive keys
        bf16x8 ds[2][2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                ds[mt][j >> 3][j & 7] = (bf16)(__builtin_amdgcn_exp2f(sacc[mt][j]) * pacc[mt][j]);
        if constexpr (kPad) {
            // a partial patch: its padding positions are not keys (register j of half mt
            // holds key 32 mt + 16 (j / 8) + 8 hi + j % 8 of the block)
            int vr, vc;
            patch_extent(clamp_block(list[u], nb), Ht, Wt, Hv, Wv, vr, vc);
            if (vr < kTile || vc < kTile) {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int key = 32 * mt + 16 * (j >> 3) + 8 * hi + (j & 7);
                        if (!((key >> 3) < vr && (key & 7) < vc)) ds[mt][j >> 3][j & 7] = (bf16)0.0f;
                    }
            }
        }
        // dQ^T += K^T dS^T; each next d tile's K^T fragments are read under the current
        // one's MFMAs
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            if (dt + 1 < DT) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) kt[(dt + 1) & 1][kk] = tfrag<D>(kb, lane, dt + 1, kk);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) mfma_acc(acc[dt], kt[dt & 1][kk], ds[kk >> 1][kk & 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        vm_wait<0>();
        __syncthreads();  // tile u + 1 has landed; everyone is done with tile u's stage
    }
    acc_settle(acc);
    store_rowT<D>(dq + head0 + (int64_t)qtok * tok, acc, hi, scale);
}

// ---- dq at D = 128 with the keys of each tile split over waves.  One workgroup of 4 waves per
// query block i: wave w takes rows 32 (w % 2) .. + 31 (lane (l32, hi): row 32 (w % 2) + l32) and
// keys 32 (w / 2) .. + 31 of every listed tile, and accumulates its own part of dQ^T; the two
// key halves' parts are added through LDS once per block, in a fixed order.  A wave holds half
// the score accumulators and fragments of the 2-wave kernel: about 230 registers, so two
// workgroups (two waves per SIMD) are resident on a CU, with the same LDS bytes per MFMA.  The
// dQ accumulators stay in VGPRs (plain MFMA builtins): under 256 registers nothing needs them
// pinned to AGPRs, and pinned they cost copies between the register classes in every tile.
constexpr int kDq4Threads = 256;

template <bool kPad>
__global__ __launch_bounds__(kDq4Threads, 2) void bwd_dq4_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ delta,
    bf16 *__restrict__ dq, int S, int heads, const int32_t *__restrict__ kv_nb,
    const int32_t *__restrict__ kv_inds, const int32_t *__restrict__ order, float scale,
    float scale_log2, int Ht, int Wt, int Hv, int Wv) {
    constexpr int D = 128, KS = D / 16, DT = D / 32, CH = D / 8;
    constexpr int CPT = kBlock * CH / kDq4Threads;
    __shared__ __attribute__((aligned(1024))) bf16 ksh[2][kBlock * D];
    __shared__ __attribute__((aligned(1024))) bf16 vsh[2][kBlock * D];

    const int nb = S / kBlock;
    const int64_t row = order[blockIdx.x];  // longest lists first, within phases of heads
    const int bh = (int)(row / nb), i = (int)(row % nb);
    const int b = bh / heads, h = bh % heads;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hi = lane >> 5;
    const int rh = w & 1, kh = w >> 1;  // row half, key half
    const int64_t tok = (int64_t)heads * D;
    const int64_t head0 = (int64_t)b * S * tok + (int64_t)h * D;
    const int qtok = i * kBlock + 32 * rh + l32;
    const int n = clamp_count(kv_nb[row], nb);
    const int32_t *list = kv_inds + row * nb;

    bf16x8 qf[KS], df[KS];
    {
        const bf16 *qr = q + head0 + (int64_t)qtok * tok + 8 * hi;
        const bf16 *dr = dout + head0 + (int64_t)qtok * tok + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 x = load8_bf16(qr + 16 * ks);
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[ks][e] = (bf16)((float)x[e] * scale_log2);
            df[ks] = load8_bf16(dr + 16 * ks);
        }
    }
    const float lse2 = lse[(int64_t)bh * S + qtok] * kLog2e;
    const float dl = delta[(int64_t)bh * S + qtok];

    uint32_t off[CPT];
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
        const int e = r * kDq4Threads + tid;
        const int rr = e / CH, cpos = e % CH;
        off[r] = (uint32_t)((rr * tok + 8 * (cpos ^ bswz<CH>(rr))) * 2);
    }
    const uint32_t ldk = __builtin_amdgcn_readfirstlane(lds_offset(ksh[0]) + w * 64 * 16);
    const uint32_t ldv = __builtin_amdgcn_readfirstlane(lds_offset(vsh[0]) + w * 64 * 16);
    auto issue = [&](int jj, int stage) {
        const int j = __builtin_amdgcn_readfirstlane(clamp_block(jj, nb));
        const bf16 *kb = k + head0 + (int64_t)j * kBlock * tok;
        const bf16 *vb = v + head0 + (int64_t)j * kBlock * tok;
#pragma unroll
        for (int r = 0; r < CPT; ++r) {
            const uint32_t sb = stage * (kBlock * D * 2) + r * kDq4Threads * 16;
            lds_direct16_sv(kb, off[r], ldk + sb);
            lds_direct16_sv(vb, off[r], ldv + sb);
        }
    };

    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = splat16(0.0f);

    if (n > 0) issue(list[0], 0);
    vm_wait<0>();
    __syncthreads();
    const int kvr = 32 * kh + sigma32(l32);  // this lane's key row in the S^T product
    for (int u = 0; u < n; ++u) {
        const int st = u & 1;
        if (u + 1 < n) issue(list[u + 1], st ^ 1);
        const char *kb = reinterpret_cast<const char *>(ksh[st]);
        const char *vb = reinterpret_cast<const char *>(vsh[st]);
        // S^T - lse and dP^T for this wave's 32 keys
        f32x16 sacc = splat16(-lse2), pacc = splat16(-dl);
        constexpr int KLA = 1;
        bf16x8 fr[KLA + 1][2];
        auto fread = [&](int ks) {
            fr[ks & KLA][0] = rfrag<D>(kb, kvr, hi, ks);
            fr[ks & KLA][1] = rfrag<D>(vb, kvr, hi, ks);
        };
#pragma unroll
        for (int ks = 0; ks < KLA; ++ks) fread(ks);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + KLA < KS) fread(ks + KLA);
            __builtin_amdgcn_sched_barrier(0);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[ks & KLA][0], qf[ks], sacc, 0, 0, 0);
            pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[ks & KLA][1], df[ks], pacc, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 kt[2][2];
#pragma unroll
        for (int p = 0; p < 2; ++p) kt[0][p] = tfrag<D>(kb, lane, 0, 2 * kh + p);
        // dS^T = P^T (dP^T - Delta), packed: registers 8p .. 8p+7 = 16 consecutive keys
        bf16x8 ds[2];
#pragma unroll
        for (int j = 0; j < 16; ++j)
            ds[j >> 3][j & 7] = (bf16)(__builtin_amdgcn_exp2f(sacc[j]) * pacc[j]);
        if constexpr (kPad) {
            // a partial patch: its padding positions are not keys (register j holds key
            // 32 kh + 16 (j / 8) + 8 hi + j % 8 of the block)
            int vr, vc;
            patch_extent(clamp_block(list[u], nb), Ht, Wt, Hv, Wv, vr, vc);
            if (vr < kTile || vc < kTile) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = 32 * kh + 16 * (j >> 3) + 8 * hi + (j & 7);
                    if (!((key >> 3) < vr && (key & 7) < vc)) ds[j >> 3][j & 7] = (bf16)0.0f;
                }
            }
        }
        // dQ^T += K^T dS^T over this wave's keys (k-steps 2 kh, 2 kh + 1)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            if (dt + 1 < DT) {
#pragma unroll
                for (int p = 0; p < 2; ++p) kt[(dt + 1) & 1][p] = tfrag<D>(kb, lane, dt + 1, 2 * kh + p);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int p = 0; p < 2; ++p)
                acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[dt & 1][p], ds[p], acc[dt], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        vm_wait<0>();
        __syncthreads();  // tile u + 1 has landed; everyone is done with tile u's stage
    }
    // the key half 1 waves hand their parts to the key half 0 waves through LDS (the ring is
    // free: the walk ended with a barrier and no load is in flight)
    float *part = reinterpret_cast<float *>(&ksh[0][0]) + (size_t)rh * (DT * 16 * 64);
    if (kh == 1) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) part[(dt * 16 + r) * 64 + lane] = acc[dt][r];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[dt][r] += part[(dt * 16 + r) * 64 + lane];
        store_rowT<D>(dq + head0 + (int64_t)qtok * tok, acc, hi, scale);
    }
}

// ---- dk, dv.  One workgroup (2 waves) per kv block j of (b, h); wave w owns keys 32 w ..
// 32 w + 31, lane (l32, hi) key 32 w + l32.  Q and dO tiles of the query blocks that list
// j go through a 2-stage LDS ring, with their rows' lse (log2 units) and Delta.
template <int D, bool kPad>
__global__ __launch_bounds__(kBwdThreads) void bwd_dkdv_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ delta,
    bf16 *__restrict__ dk, bf16 *__restrict__ dv, int S, int heads,
    const int32_t *__restrict__ q_nb, const int32_t *__restrict__ q_inds,
    const int32_t *__restrict__ order, float scale, float scale_log2, int Ht, int Wt, int Hv,
    int Wv) {
    constexpr int KS = D / 16, DT = D / 32, CPT = kBlock * D / 8 / kBwdThreads;
    __shared__ __attribute__((aligned(1024))) bf16 qsh[2][kBlock * D];
    __shared__ __attribute__((aligned(1024))) bf16 dsh[2][kBlock * D];
    __shared__ __attribute__((aligned(16))) float lsh[2][kBlock];  // lse (log2 units)
    __shared__ __attribute__((aligned(16))) float esh[2][kBlock];  // Delta

    const int nb = S / kBlock;
    const int64_t row = order[blockIdx.x];  // longest lists first, within phases of heads
    const int bh = (int)(row / nb), j = (int)(row % nb);
    const int b = bh / heads, h = bh % heads;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hi = lane >> 5;
    const int64_t tok = (int64_t)heads * D;
    const int64_t head0 = (int64_t)b * S * tok + (int64_t)h * D;
    const int ktok = j * kBlock + 32 * w + l32;
    const int n = clamp_count(q_nb[row], nb);
    const int32_t *list = q_inds + row * nb;

    // K^T (times scale * log2 e) and V^T as B operands: lane (l32, hi) holds d = 16 ks +
    // 8 hi + 0..7 of its key
    bf16x8 kf[KS], vf[KS];
    {
        const bf16 *kr = k + head0 + (int64_t)ktok * tok + 8 * hi;
        const bf16 *vr = v + head0 + (int64_t)ktok * tok + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 x = load8_bf16(kr + 16 * ks);
#pragma unroll
            for (int e = 0; e < 8; ++e) kf[ks][e] = (bf16)((float)x[e] * scale_log2);
            vf[ks] = load8_bf16(vr + 16 * ks);
        }
    }

    uint32_t off[CPT];
    tile_offsets<D>(tid, tok, off);
    const uint32_t ldq = __builtin_amdgcn_readfirstlane(lds_offset(qsh[0]) + w * 64 * 16);
    const uint32_t ldd = __builtin_amdgcn_readfirstlane(lds_offset(dsh[0]) + w * 64 * 16);
    float stash = 0.0f;  // thread t < 64: lse of row t of the next tile; t >= 64: its Delta
    auto issue = [&](int ii, int stage) {
        const int i = __builtin_amdgcn_readfirstlane(clamp_block(ii, nb));
        const bf16 *qb = q + head0 + (int64_t)i * kBlock * tok;
        const bf16 *db = dout + head0 + (int64_t)i * kBlock * tok;
#pragma unroll
        for (int r = 0; r < CPT; ++r) {
            const uint32_t sb = stage * (kBlock * D * 2) + r * kBwdThreads * 16;
            lds_direct16_sv(qb, off[r], ldq + sb);
            lds_direct16_sv(db, off[r], ldd + sb);
        }
        const int64_t rr = (int64_t)bh * S + (int64_t)i * kBlock + (tid & 63);
        stash = tid < 64 ? lse[rr] * kLog2e : delta[rr];
    };
    auto land = [&](int stage) {  // after vm_wait: the row statistics into LDS
        if (tid < 64)
            lsh[stage][tid] = stash;
        else
            esh[stage][tid - 64] = stash;
    };

    f32x16 dka[DT], dva[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        dka[dt] = splat16(0.0f);
        dva[dt] = splat16(0.0f);
    }

    if (n > 0) {
        issue(list[0], 0);
        vm_wait<0>();
        land(0);
    }
    __syncthreads();
    const int qr0 = sigma32(l32), qr1 = 32 + sigma32(l32);
    for (int u = 0; u < n; ++u) {
        const int st = u & 1;
        if (u + 1 < n) issue(list[u + 1], st ^ 1);
        const char *qb = reinterpret_cast<const char *>(qsh[st]);
        const char *db = reinterpret_cast<const char *>(dsh[st]);
        // S - lse (log2 units) and dP - Delta: rows = the tile's queries in sigma order,
        // columns = keys.  The accumulators start at minus the row statistics (register
        // 8p + e of half mt holds query 32 mt + 16 p + 8 hi + e), so the products give the
        // exponent of P and the factor of dS directly.
        f32x16 sacc[2], pacc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int q0 = 32 * mt + 16 * p + 8 * hi;
                const float4 l0 = *reinterpret_cast<const float4 *>(&lsh[st][q0]);
                const float4 l1 = *reinterpret_cast<const float4 *>(&lsh[st][q0 + 4]);
                const float4 e0 = *reinterpret_cast<const float4 *>(&esh[st][q0]);
                const float4 e1 = *reinterpret_cast<const float4 *>(&esh[st][q0 + 4]);
                const float lq[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
                const float eq[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sacc[mt][8 * p + e] = -lq[e];
                    pacc[mt][8 * p + e] = -eq[e];
                }
            }
        // Q and dO row fragments read KLA k-steps ahead of their MFMAs (as in dq)
        constexpr int KLA = 3;
        bf16x8 fr[KLA + 1][4];
        auto fread = [&](int ks) {
            fr[ks & KLA][0] = rfrag<D>(qb, qr0, hi, ks);
            fr[ks & KLA][1] = rfrag<D>(qb, qr1, hi, ks);
            fr[ks & KLA][2] = rfrag<D>(db, qr0, hi, ks);
            fr[ks & KLA][3] = rfrag<D>(db, qr1, hi, ks);
        };
#pragma unroll
        for (int ks = 0; ks < KLA; ++ks) fread(ks);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + KLA < KS) fread(ks + KLA);
            __builtin_amdgcn_sched_barrier(0);
            const bf16x8(&f)[4] = fr[ks & KLA];
            sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[0], kf[ks], sacc[0], 0, 0, 0);
            sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[1], kf[ks], sacc[1], 0, 0, 0);
            pacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[2], vf[ks], pacc[0], 0, 0, 0);
            pacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[3], vf[ks], pacc[1], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // the first d tile's dO^T and Q^T fragments, read under the VALU work below
        bf16x8 gt[2][4], qt[2][4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            gt[0][kk] = tfrag<D>(db, lane, 0, kk);
            qt[0][kk] = tfrag<D>(qb, lane, 0, kk);
        }
        // P and dS = P (dP - Delta), packed (register 8p + e of half mt: query
        // 32 mt + 16 p + 8 hi + e)
        bf16x8 pp[2][2], dd[2][2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float pr = __builtin_amdgcn_exp2f(sacc[mt][8 * p + e]);
                    pp[mt][p][e] = (bf16)pr;
                    dd[mt][p][e] = (bf16)(pr * pacc[mt][8 * p + e]);
                }
        // dV^T += dO^T P and dK^T += Q^T dS; each next d tile's fragments are read under
        // the current one's MFMAs
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            if (dt + 1 < DT) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    gt[(dt + 1) & 1][kk] = tfrag<D>(db, lane, dt + 1, kk);
                    qt[(dt + 1) & 1][kk] = tfrag<D>(qb, lane, dt + 1, kk);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                mfma_acc(dva[dt], gt[dt & 1][kk], pp[kk >> 1][kk & 1]);
                mfma_acc(dka[dt], qt[dt & 1][kk], dd[kk >> 1][kk & 1]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        vm_wait<0>();
        if (u + 1 < n) land(st ^ 1);
        __syncthreads();  // tile u + 1 has landed; everyone is done with tile u's stage
    }
    acc_settle(dka);
    acc_settle(dva);
    float kmul = scale, vmul = 1.0f;
    if constexpr (kPad) {
        // this lane's key (32 w + l32 of block j) at a padding position: dk = dv = 0
        int vr, vc;
        patch_extent(j, Ht, Wt, Hv, Wv, vr, vc);
        const int key = 32 * w + l32;
        if (!((key >> 3) < vr && (key & 7) < vc)) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                dka[dt] = splat16(0.0f);
                dva[dt] = splat16(0.0f);
            }
            kmul = 0.0f;
            vmul = 0.0f;
        }
    }
    store_rowT<D>(dk + head0 + (int64_t)ktok * tok, dka, hi, kmul);
    store_rowT<D>(dv + head0 + (int64_t)ktok * tok, dva, hi, vmul);
}

// ---- dk, dv at D = 128 with 16 keys per wave.  One workgroup of 4 waves per kv block j of
// (b, h); wave w owns keys 16 w .. 16 w + 15, lane (jl, g) = (l % 16, l / 16) key 16 w + jl.
// The products run on v_mfma_f32_16x16x32_bf16, whose lane layout (checked on the GPU against
// a CPU product) is: A [16 x 32]: lane i + 16 g holds row i, k = 8 g .. 8 g + 7; B [32 x 16]:
// lane n + 16 g holds k = 8 g .. 8 g + 7 of column n; D [16 x 16]: lane n + 16 g holds rows
// 4 g .. 4 g + 3 of column n.  A wave then needs about 200 registers (dK^T and dV^T for 16
// keys, K and V as B operands), so two workgroups, 8 waves, two per SIMD, are resident on a
// CU where the 32-key kernel runs one wave per SIMD and leaves the SIMD idle whenever that
// wave waits.  The arithmetic per (query, key) is the 32-key kernel's.
constexpr int kDkdv16Threads = 256;

// Query of A-operand row m (0..63) of the S and dP products.  Output register r of lane
// (n, g) in query m-tile mt is then query 32 (mt / 2) + 8 g + 4 (mt % 2) + r: m-tiles 2 kq and
// 2 kq + 1 give each lane the 8 consecutive queries 32 kq + 8 g + 0..7 that the B operand of
// the products over queries needs, with no data movement.
__device__ __forceinline__ int pi16(int m) {
    const int mt = m >> 4, g = (m >> 2) & 3, r = m & 3;
    return 32 * (mt >> 1) + 8 * g + 4 * (mt & 1) + r;
}
// 16-byte chunk swizzle of this kernel's Q and dO tiles (256-byte rows).  Its row reads take
// the 16 rows pi16(16 mt + 0..15), which differ in row bits 0, 1, 3 and 4; its transposed
// reads take rows R + 8 g + 0..3 (bits 0, 1 within a lane group g, bits 3, 4 across groups)
// times two chunks 2c, 2c + 1.  Row bit 0 goes to chunk bits 0 and 1, bit 1 to bit 2, bit 3
// to bit 3 and bit 4 to bits 0 and 3.  Both patterns then cover the 64 four-byte banks once
// per cycle whether a cycle serves consecutive lanes (16 for 16-byte reads, 32 for 8-byte
// reads) or lanes l and l + 32 together (a CPU model checks all four cases).  The swizzle
// does not depend on row bits 2 and 5, so a lane's addresses for m-tiles (row reads) and for
// k-steps and halves (transposed reads) differ by constants.
__device__ __forceinline__ int sw16(int row) {
    return ((row & 1) ? 3 : 0) ^ (((row >> 1) & 1) << 2) ^ (((row >> 3) & 1) << 3) ^
           (((row >> 4) & 1) ? 9 : 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <bool kPad>
__global__ __launch_bounds__(kDkdv16Threads, 2) void bwd_dkdv16_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ delta,
    bf16 *__restrict__ dk, bf16 *__restrict__ dv, int S, int heads,
    const int32_t *__restrict__ q_nb, const int32_t *__restrict__ q_inds,
    const int32_t *__restrict__ order, float scale, float scale_log2, int Ht, int Wt, int Hv,
    int Wv) {
    constexpr int D = 128, CH = D / 8, KS = D / 32, MD = D / 16;
    constexpr int CPT = kBlock * CH / kDkdv16Threads;  // 16-byte chunks per thread and tile
    constexpr int ROWB = 2 * D;
    __shared__ __attribute__((aligned(1024))) bf16 qsh[2][kBlock * D];
    __shared__ __attribute__((aligned(1024))) bf16 dsh[2][kBlock * D];
    __shared__ __attribute__((aligned(16))) float lsh[2][kBlock];  // -lse (log2 units)
    __shared__ __attribute__((aligned(16))) float esh[2][kBlock];  // -Delta

    const int nb = S / kBlock;
    const int64_t row = order[blockIdx.x];  // longest lists first, within phases of heads
    const int bh = (int)(row / nb), j = (int)(row % nb);
    const int b = bh / heads, h = bh % heads;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, jl = lane & 15, g = lane >> 4;
    const int64_t tok = (int64_t)heads * D;
    const int64_t head0 = (int64_t)b * S * tok + (int64_t)h * D;
    const int ktok = j * kBlock + 16 * w + jl;
    const int n = clamp_count(q_nb[row], nb);
    const int32_t *list = q_inds + row * nb;

    // K (times scale * log2 e) and V as B operands: lane (jl, g) holds d = 32 ks + 8 g + 0..7
    bf16x8 kf[KS], vf[KS];
    {
        const bf16 *kr = k + head0 + (int64_t)ktok * tok + 8 * g;
        const bf16 *vr = v + head0 + (int64_t)ktok * tok + 8 * g;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 x = load8_bf16(kr + 32 * ks);
#pragma unroll
            for (int e = 0; e < 8; ++e) kf[ks][e] = (bf16)((float)x[e] * scale_log2);
            vf[ks] = load8_bf16(vr + 32 * ks);
        }
    }

    // chunk e = r * 256 + tid of a tile lands at LDS byte 16 e (row e / CH, position e % CH)
    // and holds global chunk (e % CH) ^ sw16(row)
    uint32_t off[CPT];
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
        const int e = r * kDkdv16Threads + tid;
        const int rr = e / CH, cpos = e % CH;
        off[r] = (uint32_t)((rr * tok + 8 * (cpos ^ sw16(rr))) * 2);
    }
    const uint32_t ldq = __builtin_amdgcn_readfirstlane(lds_offset(qsh[0]) + w * 64 * 16);
    const uint32_t ldd = __builtin_amdgcn_readfirstlane(lds_offset(dsh[0]) + w * 64 * 16);
    float stash = 0.0f;  // thread t < 64: -lse of row t of the next tile; 64 <= t < 128: -Delta
    auto issue = [&](int ii, int stage) {
        const int i = __builtin_amdgcn_readfirstlane(clamp_block(ii, nb));
        const bf16 *qb = q + head0 + (int64_t)i * kBlock * tok;
        const bf16 *db = dout + head0 + (int64_t)i * kBlock * tok;
#pragma unroll
        for (int r = 0; r < CPT; ++r) {
            const uint32_t sb = stage * (kBlock * D * 2) + r * kDkdv16Threads * 16;
            lds_direct16_sv(qb, off[r], ldq + sb);
            lds_direct16_sv(db, off[r], ldd + sb);
        }
        if (tid < 128) {
            const int64_t rr = (int64_t)bh * S + (int64_t)i * kBlock + (tid & 63);
            stash = -(tid < 64 ? lse[rr] * kLog2e : delta[rr]);
        }
    };
    auto land = [&](int stage) {  // after vm_wait: the row statistics into LDS
        if (tid < 64)
            lsh[stage][tid] = stash;
        else if (tid < 128)
            esh[stage][tid - 64] = stash;
    };

    f32x4 dka[MD], dva[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md) {
        dka[md] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        dva[md] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // This lane's LDS byte offsets within a tile.  Row reads: row pi16(16 mt + jl) =
    // rr0 + 32 (mt / 2) + 4 (mt % 2), chunk (4 ks + g) ^ sw16(rr0).  Transposed reads: row
    // rt0 + 32 kq + 4 hh, chunk (2 md + (jl % 4) / 2) ^ sw16(rt0), byte 8 (jl % 2) in it.
    const int rr0 = pi16(jl), rt0 = 8 * g + (jl >> 2);
    uint32_t offr[KS], offt[MD];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        offr[ks] = (uint32_t)(rr0 * ROWB + (((4 * ks + g) ^ sw16(rr0)) << 4));
#pragma unroll
    for (int md = 0; md < MD; ++md)
        offt[md] = (uint32_t)(rt0 * ROWB + (((2 * md + ((jl & 3) >> 1)) ^ sw16(rt0)) << 4) +
                              8 * (jl & 1));
    const int q0l = 8 * g;  // queries 32 (mt / 2) + 8 g + 4 (mt % 2) + 0..3 of S's registers

    // one tile in LDS stage ST (a constant, so that every LDS address is a lane offset plus
    // an immediate)
    auto tile = [&](auto stc, int u) {
        constexpr int ST = decltype(stc)::value;
        if (u + 1 < n) issue(list[u + 1], ST ^ 1);
        const char *qb = reinterpret_cast<const char *>(qsh[ST]);
        const char *db = reinterpret_cast<const char *>(dsh[ST]);
        // S - lse (log2 units) and dP - Delta for this wave's keys: the accumulators start at
        // minus the statistics of their queries
        f32x4 sacc[4], pacc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int q0 = q0l + 32 * (mt >> 1) + 4 * (mt & 1);
            const float4 l4 = *reinterpret_cast<const float4 *>(&lsh[ST][q0]);
            const float4 e4 = *reinterpret_cast<const float4 *>(&esh[ST][q0]);
            sacc[mt] = f32x4{l4.x, l4.y, l4.z, l4.w};
            pacc[mt] = f32x4{e4.x, e4.y, e4.z, e4.w};
        }
        // the row fragments of k-step ks + 1 are read under the MFMAs of k-step ks
        bf16x8 fq[2][4], fd[2][4];
        auto rread = [&](int ks) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int ro = (32 * (mt >> 1) + 4 * (mt & 1)) * ROWB;
                fq[ks & 1][mt] = *reinterpret_cast<const bf16x8 *>(qb + ro + offr[ks]);
                fd[ks & 1][mt] = *reinterpret_cast<const bf16x8 *>(db + ro + offr[ks]);
            }
        };
        rread(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 1 < KS) rread(ks + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                sacc[mt] = mfma16(fq[ks & 1][mt], kf[ks], sacc[mt]);
                pacc[mt] = mfma16(fd[ks & 1][mt], vf[ks], pacc[mt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // P and dS = P (dP - Delta), packed as the B operands of the two k-steps over the
        // tile's queries (k-step kq: queries 32 kq + 8 g + 0..7 = m-tiles 2 kq, 2 kq + 1)
        bf16x8 pp[2], dd[2];
#pragma unroll
        for (int kq = 0; kq < 2; ++kq)
#pragma unroll
            for (int hm = 0; hm < 2; ++hm)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float pr = __builtin_amdgcn_exp2f(sacc[2 * kq + hm][r]);
                    pp[kq][4 * hm + r] = (bf16)pr;
                    dd[kq][4 * hm + r] = (bf16)(pr * pacc[2 * kq + hm][r]);
                }
        // dV^T += dO^T P and dK^T += Q^T dS: the A operands are transposing reads, lane
        // (jl, g) getting column d = 16 md + jl of rows 32 kq + 8 g + 0..7
        // the transposed fragments of d tile md + 1 are read under the MFMAs of d tile md
        bf16x8 at_d[2][2], at_q[2][2];
        auto tread = [&](int md) {
#pragma unroll
            for (int kq = 0; kq < 2; ++kq)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int ro = (32 * kq + 4 * hh) * ROWB;
                    const bf16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (NABLA_LDS bf16x4 *)(db + ro + offt[md]));
                    const bf16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (NABLA_LDS bf16x4 *)(qb + ro + offt[md]));
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        at_d[md & 1][kq][4 * hh + e] = x[e];
                        at_q[md & 1][kq][4 * hh + e] = y[e];
                    }
                }
        };
        tread(0);
#pragma unroll
        for (int md = 0; md < MD; ++md) {
            if (md + 1 < MD) tread(md + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kq = 0; kq < 2; ++kq) {
                dva[md] = mfma16(at_d[md & 1][kq], pp[kq], dva[md]);
                dka[md] = mfma16(at_q[md & 1][kq], dd[kq], dka[md]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        vm_wait<0>();
        if (u + 1 < n) land(ST ^ 1);
        __syncthreads();  // tile u + 1 has landed; everyone is done with tile u's stage
    };

    if (n > 0) {
        issue(list[0], 0);
        vm_wait<0>();
        land(0);
    }
    __syncthreads();
    for (int u = 0; u < n; u += 2) {
        tile(std::integral_constant<int, 0>{}, u);
        if (u + 1 < n) tile(std::integral_constant<int, 1>{}, u + 1);
    }
    float kmul = scale, vmul = 1.0f;
    if constexpr (kPad) {
        // this lane's key (16 w + jl of block j) at a padding position: dk = dv = 0
        int vr, vc;
        patch_extent(j, Ht, Wt, Hv, Wv, vr, vc);
        const int key = 16 * w + jl;
        if (!((key >> 3) < vr && (key & 7) < vc)) {
#pragma unroll
            for (int md = 0; md < MD; ++md) {
                dka[md] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                dva[md] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
            kmul = 0.0f;
            vmul = 0.0f;
        }
    }
    // lane (jl, g) holds d = 16 md + 4 g + 0..3 of its key: 8-byte runs of the key's row
    bf16 *dkr = dk + head0 + (int64_t)ktok * tok + 4 * g;
    bf16 *dvr = dv + head0 + (int64_t)ktok * tok + 4 * g;
#pragma unroll
    for (int md = 0; md < MD; ++md) {
        bf16x4 xk, xv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            xk[r] = (bf16)(dka[md][r] * kmul);
            xv[r] = (bf16)(dva[md][r] * vmul);
        }
        *reinterpret_cast<bf16x4 *>(dkr + 16 * md) = xk;
        *reinterpret_cast<bf16x4 *>(dvr + 16 * md) = xv;
    }
}

// ---- host side

// Workspace: [Delta: B*heads*S fp32 | q_nb: B*heads*nb | q_inds: B*heads*nb*nb int32 |
// tmat: B*heads*nb*nb bytes | dq order, dk/dv order: B*heads*nb int32 each], each part
// 256-byte aligned.
size_t sparse_attn_bwd_workspace_bytes(int B, int S, int heads) {
    const size_t bh = (size_t)B * heads, nb = (size_t)S / kBlock;
    return round256(bh * S * 4) + round256(bh * nb * 4) + round256(bh * nb * nb * 4) +
           round256(bh * nb * nb) + 2 * round256(bh * nb * 4);
}

template <int D, bool kPad>
static hipError_t launch_bwd_t(const bf16 *q, const bf16 *k, const bf16 *v, const bf16 *o,
                               const bf16 *dout, const float *lse, int B, int S, int heads,
                               const int32_t *kv_nb, const int32_t *kv_inds, float scale, bf16 *dq,
                               bf16 *dk, bf16 *dv, int Ht, int Wt, int Hv, int Wv, void *ws,
                               hipStream_t stream) {
    const int nb = S / kBlock;
    const size_t BH = (size_t)B * heads;
    char *p = static_cast<char *>(ws);
    float *delta = reinterpret_cast<float *>(p);
    p += round256(BH * S * 4);
    int32_t *q_nb = reinterpret_cast<int32_t *>(p);
    p += round256(BH * nb * 4);
    int32_t *q_inds = reinterpret_cast<int32_t *>(p);
    p += round256(BH * nb * nb * 4);
    uint8_t *tmat = reinterpret_cast<uint8_t *>(p);
    const int64_t tbytes = (int64_t)round256(BH * nb * nb);
    p += tbytes;
    int32_t *order_q = reinterpret_cast<int32_t *>(p);
    p += round256(BH * nb * 4);
    int32_t *order_k = reinterpret_cast<int32_t *>(p);

    const int64_t nrows = (int64_t)B * S * heads;
    const int64_t dgrid = (nrows * (D / 8) + 255) / 256;
    hipLaunchKernelGGL(bwd_delta_kernel<D>, dim3((unsigned)dgrid), dim3(256), 0, stream, o, dout,
                       delta, S, heads, nrows);
    const int64_t n16 = tbytes / 16;
    const int64_t zgrid = (n16 + 255) / 256;
    hipLaunchKernelGGL(bwd_tlist_zero_kernel, dim3((unsigned)(zgrid < 8192 ? zgrid : 8192)),
                       dim3(256), 0, stream, reinterpret_cast<uint4 *>(tmat), n16);
    const unsigned rows = (unsigned)(BH * nb);
    hipLaunchKernelGGL(bwd_tlist_scatter_kernel, dim3(rows), dim3(256), 0, stream, kv_nb, kv_inds,
                       nb, tmat);
    hipLaunchKernelGGL(bwd_tlist_compact_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, tmat,
                       nb, (int64_t)rows, q_nb, q_inds);
    // Launch orders: longest lists first within phases of as few heads as give one round of
    // the resident workgroups (one head at 720p), so that the long rows do not start last
    // and the K/V (or Q/dO) tiles read together stay in the caches (A/B at 720p: phases of
    // 1, 2, 3 and 5 heads 24.8, 25.6, 26.7 and 27.5 ms).
    const int resident = resident_workgroups<bwd_dq_kernel<D, kPad>>(kBwdThreads);
    if (resident <= 0) return hipErrorInvalidDevice;
    int hpp = (resident + nb - 1) / nb;
    hpp = hpp < 1 ? 1 : (hpp > (int)BH ? (int)BH : hpp);
    hipError_t e = launch_longest_first(kv_nb, (int)rows, hpp * nb, nb, order_q, stream);
    if (e != hipSuccess) return e;
    e = launch_longest_first(q_nb, (int)rows, hpp * nb, nb, order_k, stream);
    if (e != hipSuccess) return e;
    const float scale_log2 = scale * kLog2e;
    if constexpr (D == 128)
        hipLaunchKernelGGL((bwd_dq4_kernel<kPad>), dim3(rows), dim3(kDq4Threads), 0, stream, q, k,
                           v, dout, lse, delta, dq, S, heads, kv_nb, kv_inds, order_q, scale,
                           scale_log2, Ht, Wt, Hv, Wv);
    else
        hipLaunchKernelGGL((bwd_dq_kernel<D, kPad>), dim3(rows), dim3(kBwdThreads), 0, stream, q,
                           k, v, dout, lse, delta, dq, S, heads, kv_nb, kv_inds, order_q, scale,
                           scale_log2, Ht, Wt, Hv, Wv);
    if constexpr (D == 128)
        hipLaunchKernelGGL((bwd_dkdv16_kernel<kPad>), dim3(rows), dim3(kDkdv16Threads), 0, stream,
                           q, k, v, dout, lse, delta, dk, dv, S, heads, q_nb, q_inds, order_k,
                           scale, scale_log2, Ht, Wt, Hv, Wv);
    else
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, kPad>), dim3(rows), dim3(kBwdThreads), 0, stream, q,
                           k, v, dout, lse, delta, dk, dv, S, heads, q_nb, q_inds, order_k, scale,
                           scale_log2, Ht, Wt, Hv, Wv);
    return hipGetLastError();
}

hipError_t launch_sparse_attn_bwd(const void *q, const void *k, const void *v, const void *o,
                                  const void *dout, const float *lse, int B, int S, int heads,
                                  int D, const int32_t *kv_nb, const int32_t *kv_inds,
                                  float scale, void *dq, void *dk, void *dv, int Ht, int Wt,
                                  int Hv, int Wv, void *ws, hipStream_t stream) {
    const auto c = [](const void *x) { return static_cast<const bf16 *>(x); };
    const auto m = [](void *x) { return static_cast<bf16 *>(x); };
    const bool pad = Hv > 0;
    if (D == 128) {
        if (pad)
            return launch_bwd_t<128, true>(c(q), c(k), c(v), c(o), c(dout), lse, B, S, heads,
                                           kv_nb, kv_inds, scale, m(dq), m(dk), m(dv), Ht, Wt,
                                           Hv, Wv, ws, stream);
        return launch_bwd_t<128, false>(c(q), c(k), c(v), c(o), c(dout), lse, B, S, heads, kv_nb,
                                        kv_inds, scale, m(dq), m(dk), m(dv), 0, 0, 0, 0, ws,
                                        stream);
    }
    if (pad)
        return launch_bwd_t<64, true>(c(q), c(k), c(v), c(o), c(dout), lse, B, S, heads, kv_nb,
                                      kv_inds, scale, m(dq), m(dk), m(dv), Ht, Wt, Hv, Wv, ws,
                                      stream);
    return launch_bwd_t<64, false>(c(q), c(k), c(v), c(o), c(dout), lse, B, S, heads, kv_nb,
                                   kv_inds, scale, m(dq), m(dk), m(dv), 0, 0, 0, 0, ws, stream);
}

}  // namespace nabla
