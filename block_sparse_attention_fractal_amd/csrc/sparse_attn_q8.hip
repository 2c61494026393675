// sparse_attn_q8.hip -- the quantized block-sparse attention forward on gfx950.
//
// The attention of the quantized variant (the sibling "sla" backend page, SageSLA
// forward: INT8 Q K^T, FP8 P V) over the kv lists of the NABLA estimator, on the codes
// written by quant.hip:
//   z_c  = scale * qs_i * ks_j * <q8, k8_c>       (INT8 product, exact int32)
//   P    = e4m3(c * 2^(log2e z_c - m))           (FP8 weights, c 2^(...) <= 448)
//   o[d] = vs[d] * sum_c P_c v8_cd / sum_c P_c    (FP8 product, fp32 accumulation)
// for each query row over the keys of its listed 64 x 64 blocks.
//
// Design (CDNA4 / gfx950), the bf16 kernel's walk with both products at twice the rate:
//   * The schedule, the groups of 4 neighbouring query blocks (a 2 (time) x 1 x 2
//     (width) box) and the walk over the union of their lists are those of the bf16
//     kernel: one K tile and one V^T tile per union block are fetched once per group
//     and shared through a 4-stage LDS ring; waves skip the tiles their block does not
//     list; persistent workgroups take groups longest first within phases of a few
//     heads.
//   * Scores S^T = K Q^T with v_mfma_i32_32x32x32_i8 (int32, exact): a lane owns one
//     query row.  K rows are fed in an order that leaves lane (n, hi) holding the 32
//     keys 32 hi .. 32 hi + 31 of its row in register order, which is exactly the B
//     operand of v_mfma_f32_32x32x64_f8f6f4 for O^T = V^T P^T over all 64 keys of the
//     tile in one k-step.  The V^T A operand is 32 consecutive bytes of a V^T row.
//   * Both tiles are stored in LDS in MFMA-operand order: every fragment read is a
//     64-lane ds_read_b128 of 1 KiB of consecutive bytes (no bank conflicts); the
//     global -> LDS loads (global_load_lds_dwordx4) gather the 16-byte chunks into
//     that order.
//   * Every wave runs one tile behind in its softmax: at each step it issues the score
//     MFMAs of the new tile and, while they run, does the softmax and P V of the tile
//     it listed at the step before, so the VALU work overlaps its own MFMAs (and the
//     other wave's on the SIMD).
//   * Softmax in fp32, log2 domain, with a lazy reference max: the reference m is
//     raised to the row max only when a tile's max exceeds it by more than 2 (and on
//     the row's first tile), so the weights 2^(s - m) stay <= 4 and c = 112 keeps the
//     e4m3 codes <= 448; the rescale of O is rare.
//   * The row sum is an FP8 MFMA of the same packed weights with a V^T block whose
//     first row is ones: the sum of exactly the weights P V uses, with no VALU.
#include "attn_tile.h"
#include "nabla_launch.h"

namespace nabla {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int kQStages = 4;
constexpr float kQLazy = 2.0f;                 // log2 units the weights may exceed the reference
constexpr float kQLog2C = 6.807354922057604f;  // log2(112): 112 * 2^2 = 448, the largest e4m3
// The INT8 score products start from this bias: the int32 result acc + 0x4B400000, read as
// fp32, is exactly 1.5 * 2^23 + acc for |acc| < 2^22 (|acc| <= 127^2 D < 2^21 here), so one
// fma turns it into the logit, with no int -> float conversion.
constexpr int kQBias = 0x4B400000;
constexpr float kQBiasF = 12582912.0f;  // 1.5 * 2^23
// A padding key's score: below every biased score, so it never sets the tile maximum.
constexpr int kQMasked = (int)0x80000000u;

template <int D>
struct AttnQ8Shared {
    int8_t ks[kQStages][kBlock * D];   // K tiles, MFMA-operand order
    uint8_t vs[kQStages][D * kBlock];  // V^T tiles (e4m3 codes), MFMA-operand order
    int8_t qs[kAttnWaves][32 * D];     // each wave's 32 query rows, MFMA-operand order
    uint64_t qmask[kGroup][kMaxWords];
    uint16_t ulist[kMaxWords * 64];    // the union of the members' lists, ascending
    uint8_t umem[kMaxWords * 64];      // bit s: member s lists that block
    int ucount;
    int slot;
};

__device__ __forceinline__ i32x16 splat16i(int x) {
    i32x16 r;
#pragma unroll
    for (int j = 0; j < 16; ++j) r[j] = x;
    return r;
}

__device__ __forceinline__ int imax16(const i32x16 &s) {
    int x = max(s[0], s[1]);
#pragma unroll
    for (int j = 2; j < 16; ++j) x = max(x, s[j]);
    return x;
}


// kPad: the layout is a padded grid (Hv x Wv latents, partial patches); padding keys are
// never keys.  The instance without it carries none of that code.
template <int D, bool kPad>
__global__ __launch_bounds__(kAttnThreads) void sparse_attn_q8_kernel(
    const int8_t *__restrict__ q8, const float *__restrict__ qsc, const int8_t *__restrict__ k8,
    const float *__restrict__ ksc, const uint8_t *__restrict__ v8,
    const float *__restrict__ vsc, bf16 *__restrict__ o, int S, int heads, int Tt, int Ht,
    int Wt, int Hv, int Wv, NatGrid ng, int groups_per_bh, int ngroups,
    const int32_t *__restrict__ kv_nb,
    const int32_t *__restrict__ kv_inds, float scale_log2, const int32_t *__restrict__ order,
    int32_t *__restrict__ counter) {
    constexpr int KS = D / 32;                 // k-steps of the INT8 score product
    constexpr int DT = D / 32;                 // 32-wide output d tiles
    constexpr int TILEB = kBlock * D;          // bytes of a K or V^T tile
    constexpr int TCH = TILEB / 16;            // 16-byte chunks per tile
    constexpr int LOADS = 2 * TCH / kAttnThreads;  // chunks per lane per tile (K and V^T)
    static_assert(LOADS >= 1 && (2 * TCH) % kAttnThreads == 0, "tile / workgroup size");
    static_assert(TCH % 64 == 0, "a wave's chunks lie in one tile");

    __shared__ __attribute__((aligned(1024))) AttnQ8Shared<D> sh;

    const int nb = S / kBlock;
    const int nwords = (nb + 63) >> 6;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int wu = __builtin_amdgcn_readfirstlane(w);  // the wave index as a scalar

    // Global byte offset, within its 8 KiB (D = 128) tile, of each chunk this lane loads.
    // Chunk e = r * threads + tid: e < TCH is K position e (fragment (mt, ks), lane l:
    // key sigma(mt, l % 32), dims 32 ks + 16 (l / 32) ..); otherwise V^T position
    // p = e - TCH (fragment (dt, hc), lane l: row d = 32 dt + l % 32, keys 32 (l / 32)
    // + 16 hc ..).  sigma(mt, m = 8a + 4h + b) = 32 h + 16 mt + 4 a + b.
    uint32_t goff[LOADS];
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
        const int e = r * kAttnThreads + tid;
        if (e < TCH) {
            const int mt = e / (KS * 64), ks = (e / 64) % KS, l = e & 63, m = l & 31;
            const int key = 32 * ((m >> 2) & 1) + 16 * mt + 4 * (m >> 3) + (m & 3);
            goff[r] = (uint32_t)(key * D + 16 * (2 * ks + (l >> 5)));
        } else {
            const int p = e - TCH;
            const int dt = p / 128, hc = (p / 64) & 1, l = p & 63;
            goff[r] = (uint32_t)((32 * dt + (l & 31)) * kBlock + 32 * (l >> 5) + 16 * hc);
        }
    }
    const uint32_t lds_k = __builtin_amdgcn_readfirstlane(lds_offset(sh.ks[0]));
    const uint32_t lds_v = __builtin_amdgcn_readfirstlane(lds_offset(sh.vs[0]));
    // A operand of the row-sum product: row 0 of the V^T block is e4m3 1.0 (0x38), the rest 0
    const int one8 = l32 == 0 ? 0x38383838 : 0;
    const i32x8 ones = {one8, one8, one8, one8, one8, one8, one8, one8};

    for (;;) {
    if (tid == 0) sh.slot = atomicAdd(counter, 1);
    __syncthreads();
    // the same in every lane: read as a scalar, so that the exit test is a scalar branch
    const int pos = __builtin_amdgcn_readfirstlane(sh.slot);
    if (pos >= ngroups) break;
    const int grp = order[pos];
    const int bh = grp / groups_per_bh;
    const int gi = grp % groups_per_bh;
    const int h = bh % heads;
    const int b = bh / heads;

    int member[kGroup];
#pragma unroll
    for (int s = 0; s < kGroup; ++s) member[s] = group_member(gi, s, Tt, Ht, Wt, nb);

    // ---- per-member bitmaps of listed blocks, and their union
    for (int e = tid; e < kGroup * kMaxWords; e += kAttnThreads) (&sh.qmask[0][0])[e] = 0ull;
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kGroup; ++s) {
        if (member[s] < 0) continue;
        const int64_t row = (int64_t)bh * nb + member[s];
        const int n = clamp_count(kv_nb[row], nb);
        const int32_t *list = kv_inds + row * nb;
        for (int e = tid; e < n; e += kAttnThreads) {
            const int j = clamp_block(list[e], nb);
            atomicOr((unsigned long long *)&sh.qmask[s][j >> 6], 1ull << (j & 63));
        }
    }
    __syncthreads();
    if (w == 0) {
        uint64_t u = 0ull;
        if (lane < nwords) {
#pragma unroll
            for (int s = 0; s < kGroup; ++s) u |= sh.qmask[s][lane];
        }
        const int cnt = __popcll(u);
        int incl = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int x = __shfl_up(incl, d);
            if (lane >= d) incl += x;
        }
        int p = incl - cnt;
        while (u != 0ull) {
            const int bit = __builtin_ctzll(u);
            u &= u - 1;
            int mem = 0;
#pragma unroll
            for (int s = 0; s < kGroup; ++s) mem |= (int)((sh.qmask[s][lane] >> bit) & 1ull) << s;
            sh.ulist[p] = (uint16_t)(lane * 64 + bit);
            sh.umem[p] = (uint8_t)mem;
            ++p;
        }
        if (lane == 63) sh.ucount = incl;
    }
    __syncthreads();
    const int U = sh.ucount;

    // ---- this wave: member slot (opposite corners of the box share a SIMD) and 32-row half
    const int slot = w < 4 ? (w >> 1) : 3 - ((w - 4) >> 1);
    const int myblk = member[slot];
    const int64_t qrow = (int64_t)bh * nb + (myblk < 0 ? 0 : myblk);
    const int qtok = (myblk < 0 ? 0 : myblk) * kBlock + (w & 1) * 32 + l32;
    // Q^T as B operands, kept in this wave's LDS slice: lane (n, hi), k-step ks holds dims
    // 32 ks + 16 hi .. + 15 of row n, at ((ks * 64) + lane) * 16
    char *qlds = reinterpret_cast<char *>(sh.qs[w]);
    float qscale = 0.0f;
    if (myblk >= 0) {
        const int8_t *qr = q8 + (qrow * kBlock + (w & 1) * 32 + l32) * D + 16 * hi;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            *reinterpret_cast<i32x4 *>(qlds + (ks * 64 + lane) * 16) =
                *reinterpret_cast<const i32x4 *>(qr + 32 * ks);
        qscale = qsc[qrow] * scale_log2;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): retire the Q loads before the walk

    const int8_t *k8_bh = k8 + (int64_t)bh * nb * TILEB;
    const uint8_t *v8_bh = v8 + (int64_t)bh * nb * TILEB;
    auto issue = [&](int jj, int stage) {
        const int j = __builtin_amdgcn_readfirstlane(jj);
        const int8_t *kb = k8_bh + (int64_t)j * TILEB;
        const uint8_t *vb = v8_bh + (int64_t)j * TILEB;
#pragma unroll
        for (int r = 0; r < LOADS; ++r) {
            const int e0 = r * kAttnThreads + wu * 64;  // wave-uniform
            if (e0 < TCH)
                lds_direct16_sv(kb, goff[r], lds_k + stage * TILEB + 16 * e0);
            else
                lds_direct16_sv(vb, goff[r], lds_v + stage * TILEB + 16 * (e0 - TCH));
        }
    };
    auto settle = [&](bool newest_in_flight) {
        if (newest_in_flight)
            vm_wait<LOADS>();
        else
            vm_wait<0>();
    };

    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = splat16(0.0f);
    f32x16 lacc = splat16(0.0f);  // row sums (row 0 of the product: lanes 0..31, register 0)
    float m_ref = 0.0f;           // reference max of the row, log2 units
    bool m_valid = false;

    i32x8 pb = {0, 0, 0, 0, 0, 0, 0, 0};     // packed weights (every byte rewritten per tile)
    const i32x16 bias16 = splat16i(kQBias);  // accumulator start of the score products
    bool pend = false;      // a listed tile's scores wait for their softmax and P V
    int pend_stage = 0;
    float pend_unit = 0.0f;
    int pend_j = 0;  // the pending tile's block (padded layouts: its patch extent)

    // K fragments of the tile in `stage`: (mt, ks) is one contiguous 1 KiB read
    auto kread = [&](int stage, i32x4 (&kf)[2][KS]) {
        const char *kb = reinterpret_cast<const char *>(sh.ks[stage]);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kf[mt][ks] = *reinterpret_cast<const i32x4 *>(kb + ((mt * KS + ks) * 64 + lane) * 16);
    };
    // V^T fragments of d tiles dt0 .. dt0 + DT/2 - 1 of the tile in `stage`: each d tile is
    // two contiguous 1 KiB reads
    constexpr int DH = DT / 2;
    auto vread = [&](int stage, int dt0, i32x8 (&va)[DH]) {
        const char *vb = reinterpret_cast<const char *>(sh.vs[stage]);
#pragma unroll
        for (int u = 0; u < DH; ++u) {
            const int dt = dt0 + u;
            const i32x4 a0 = *reinterpret_cast<const i32x4 *>(vb + ((dt * 2) * 64 + lane) * 16);
            const i32x4 a1 = *reinterpret_cast<const i32x4 *>(vb + ((dt * 2 + 1) * 64 + lane) * 16);
            va[u] = (i32x8){a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        }
    };
    // scores S^T = K Q^T of one tile (biased int32, exact; see kQBias)
    auto qk = [&](const i32x4 (&kf)[2][KS], i32x16 (&sacc)[2]) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const i32x4 qf = *reinterpret_cast<const i32x4 *>(qlds + (ks * 64 + lane) * 16);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                sacc[mt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[mt][ks], qf,
                                                                 ks == 0 ? bias16 : sacc[mt],
                                                                 0, 0, 0);
        }
    };
    // scores -> packed e4m3 weights pb (B operand of P V: byte t of lane (n, hi) is key
    // 32 hi + t); O and the row sum rescaled when the reference moves
    auto softmax = [&](const i32x16 (&sacc)[2], float unit) {
        const int imax = max(imax16(sacc[0]), imax16(sacc[1]));
        const float tmax = (__int_as_float(imax) - kQBiasF) * unit;
        const float rm = fmaxf(tmax, __shfl_xor(tmax, 32));  // the row's tile max
        if (__builtin_amdgcn_ballot_w64(!m_valid || rm > m_ref + kQLazy) != 0ull) {
            const bool need = !m_valid || rm > m_ref + kQLazy;  // same in lanes l, l ^ 32
            const float mnew = need ? rm : m_ref;
            const float alpha = m_valid ? __builtin_amdgcn_exp2f(m_ref - mnew) : 0.0f;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
            lacc *= alpha;
            m_ref = mnew;
            m_valid = true;
        }
        // logit = (as_float(biased) - 1.5 * 2^23) * unit + log2(112) - m in one fma
        const float off = __builtin_fmaf(-kQBiasF, unit, kQLog2C - m_ref);
#pragma unroll
        for (int q4 = 0; q4 < 8; ++q4) {
            const int mt = q4 >> 2, j0 = 4 * (q4 & 3);
            float f[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                f[i] = __builtin_amdgcn_exp2f(
                    __builtin_fmaf(__int_as_float(sacc[mt][j0 + i]), unit, off));
            int pk = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], pb[q4], false);
            pb[q4] = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], pk, true);
        }
    };
    // O^T += V^T P^T for d tiles dt0 .. dt0 + DT/2 - 1
    auto pv = [&](int dt0, const i32x8 (&va)[DH], const i32x8 &w8) {
#pragma unroll
        for (int u = 0; u < DH; ++u)
            oacc[dt0 + u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va[u], w8, oacc[dt0 + u],
                                                                           0, 0, 0, 0, 0, 0);
    };
    // the pending tile (scores in sold): softmax, then P V and the row sums; the first half
    // of the V^T fragments is read before the softmax, the second half after it
    auto finish = [&](i32x16 (&sold)[2]) {
        i32x8 va[DH];
        vread(pend_stage, 0, va);
        // a partial patch of a padded grid: its padding positions are not keys (lane
        // (n, hi) holds key 32 hi + 16 mt + j in register j of half mt, and byte t of the
        // packed weights is key 32 hi + t): their scores drop out of the tile maximum, and
        // their weights are cleared after packing (a 0 block scale could turn a forced
        // -inf logit into NaN)
        int vr = kTile, vc = kTile;
        if constexpr (kPad) {
            const int th = (pend_j / Wt) % Ht, tw = pend_j % Wt;
            vr = min(kTile, Hv - th * kTile);
            vc = min(kTile, Wv - tw * kTile);
            if (vr < kTile || vc < kTile) {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int jj = 0; jj < 16; ++jj) {
                        const int key = 32 * hi + 16 * mt + jj;
                        if (!((key >> 3) < vr && (key & 7) < vc)) sold[mt][jj] = kQMasked;
                    }
            }
        }
        softmax(sold, pend_unit);
        if constexpr (kPad) {
            if (vr < kTile || vc < kTile) {
#pragma unroll
                for (int q4 = 0; q4 < 8; ++q4) {
                    uint32_t keep = 0u;
#pragma unroll
                    for (int b4 = 0; b4 < 4; ++b4) {
                        const int key = 32 * hi + 4 * q4 + b4;
                        if ((key >> 3) < vr && (key & 7) < vc) keep |= 0xFFu << (8 * b4);
                    }
                    pb[q4] = (int)((uint32_t)pb[q4] & keep);
                }
            }
        }
        pv(0, va, pb);
        vread(pend_stage, DH, va);
        pv(DH, va, pb);
        lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pb, lacc, 0, 0, 0, 0, 0, 0);
    };
    // ---- the walk over union tiles u_0, u_1, ...; u_k lives in LDS stage k % 4.
    // Step k: start loading u_{k+2}; issue the score MFMAs of u_k (if this wave's block
    // lists it); while they run, the softmax and P V of the wave's pending tile (the one
    // it listed at step k-1, still in its stage); make sure u_{k+1} has landed; barrier.
    // The ring holds u_{k-1} .. u_{k+2}, so the pending tile's V^T is still in LDS.
    if (U > 0) {
        issue(sh.ulist[0], 0);
        if (U > 1) issue(sh.ulist[1], 1);
        settle(U > 1);
    }
    __syncthreads();

    int pf_blk = U > 2 ? sh.ulist[2] : -1;
    int pf_mem = U > 0 ? sh.umem[0] : 0;
    int pf_j = U > 0 ? sh.ulist[0] : 0;
    // one step; the scores of u_k go to snew, the pending tile's are in sold
    auto step = [&](int kk, int stage, i32x16 (&snew)[2], i32x16 (&sold)[2]) {
        const int n2 = __builtin_amdgcn_readfirstlane(pf_blk);  // u_{k+2}
        const int memk = __builtin_amdgcn_readfirstlane(pf_mem);
        const int jk = __builtin_amdgcn_readfirstlane(pf_j);     // u_k
        pf_blk = kk + 3 < U ? sh.ulist[kk + 3] : -1;
        pf_mem = kk + 1 < U ? sh.umem[kk + 1] : 0;
        pf_j = kk + 1 < U ? sh.ulist[kk + 1] : 0;
        const int stage2 = (stage + 2) & (kQStages - 1);
        if (n2 >= 0) issue(n2, stage2);
        const bool mine = myblk >= 0 && ((memk >> slot) & 1);
        if (mine) {
            i32x4 kf[2][KS];
            kread(stage, kf);
            qk(kf, snew);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (pend) finish(sold);
        pend = mine;
        pend_stage = stage;
        pend_unit = qscale * ksc[(int64_t)bh * nb + jk];
        pend_j = jk;
        settle(n2 >= 0);
        __syncthreads();  // u_{k+1} has landed; everyone is done with u_{k-1}'s stage
    };
    // unrolled by two so that the two score buffers swap roles without copies
    i32x16 sa[2], sb[2];
    int kk = 0, stage = 0;
    for (; kk + 1 < U; kk += 2, stage = (stage + 2) & (kQStages - 1)) {
        step(kk, stage, sa, sb);
        step(kk + 1, (stage + 1) & (kQStages - 1), sb, sa);
    }
    bool last_in_a = false;  // the pending scores (if any) after the walk: in sa or sb
    if (kk < U) {
        step(kk, stage, sa, sb);
        last_in_a = true;
    }
    if (pend) {  // the last listed tile
        if (last_in_a)
            finish(sa);
        else
            finish(sb);
    }

    if (myblk >= 0) {
        const float lsum = __shfl(lacc[0], l32);  // row 0 of the sum product, lane n
        const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;  // empty list -> O = 0
        // the row's token in o's layout (natural order when ng.W > 0)
        const int64_t otok = block_row_token(qtok / kBlock, qtok % kBlock, ng);
        bf16 *orow = o + ((int64_t)b * S + otok) * ((int64_t)heads * D) + (int64_t)h * D;
        const float *vsr = vsc + (int64_t)bh * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d = 32 * dt + 8 * jj + 4 * hi;
                const float4 sv = *reinterpret_cast<const float4 *>(vsr + d);
                bf16x4 r;
                r[0] = (bf16)(oacc[dt][4 * jj + 0] * inv * sv.x);
                r[1] = (bf16)(oacc[dt][4 * jj + 1] * inv * sv.y);
                r[2] = (bf16)(oacc[dt][4 * jj + 2] * inv * sv.z);
                r[3] = (bf16)(oacc[dt][4 * jj + 3] * inv * sv.w);
                *reinterpret_cast<bf16x4 *>(orow + d) = r;
            }
        }
    }
    __syncthreads();  // the next group reuses the LDS
    }  // persistent loop
}

size_t sparse_attn_q8_workspace_bytes(int B, int S, int heads, int Tt, int Ht, int Wt) {
    return attn_schedule_bytes(B, S, heads, Tt, Ht, Wt);
}

template <int D>
static hipError_t launch_q8_t(const int8_t *q8, const float *qs, const int8_t *k8,
                              const float *ks, const uint8_t *v8, const float *vs, int B, int S,
                              int heads, int Tt, int Ht, int Wt, int Hv, int Wv, bool natural,
                              const int32_t *kv_nb, const int32_t *kv_inds, float scale_log2,
                              void *o, void *ws, hipStream_t stream) {
    const NatGrid ng = nat_grid(natural && Hv == 0 ? kTile * Wt : 0);
    const int resident = resident_workgroups<sparse_attn_q8_kernel<D, false>>(kAttnThreads);
    if (resident <= 0) return hipErrorInvalidDevice;
    const AttnSchedule sc =
        launch_attn_plan(kv_nb, kv_inds, B, S, heads, Tt, Ht, Wt, resident, ws, stream);
    if (Hv > 0)
        hipLaunchKernelGGL((sparse_attn_q8_kernel<D, true>), dim3(sc.grid), dim3(kAttnThreads), 0,
                           stream, q8, qs, k8, ks, v8, vs, static_cast<bf16 *>(o), S, heads, Tt,
                           Ht, Wt, Hv, Wv, ng, sc.groups_per_bh, sc.ngroups, kv_nb, kv_inds,
                           scale_log2, sc.order, sc.counter);
    else
        hipLaunchKernelGGL((sparse_attn_q8_kernel<D, false>), dim3(sc.grid), dim3(kAttnThreads),
                           0, stream, q8, qs, k8, ks, v8, vs, static_cast<bf16 *>(o), S, heads,
                           Tt, Ht, Wt, 0, 0, ng, sc.groups_per_bh, sc.ngroups, kv_nb, kv_inds,
                           scale_log2, sc.order, sc.counter);
    return hipGetLastError();
}

hipError_t launch_sparse_attn_q8(const int8_t *q8, const float *qs, const int8_t *k8,
                                 const float *ks, const uint8_t *v8, const float *vs, int B,
                                 int S, int heads, int D, int Tt, int Ht, int Wt,
                                 const int32_t *kv_nb, const int32_t *kv_inds, float scale,
                                 int Hv, int Wv, bool natural, void *o, void *ws,
                                 hipStream_t stream) {
    const float scale_log2 = scale * 1.4426950408889634f;
    if (D == 128)
        return launch_q8_t<128>(q8, qs, k8, ks, v8, vs, B, S, heads, Tt, Ht, Wt, Hv, Wv, natural,
                                kv_nb, kv_inds, scale_log2, o, ws, stream);
    return launch_q8_t<64>(q8, qs, k8, ks, v8, vs, B, S, heads, Tt, Ht, Wt, Hv, Wv, natural,
                           kv_nb, kv_inds, scale_log2, o, ws, stream);
}

}  // namespace nabla
