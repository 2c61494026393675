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
//   * Tiles go into a 4-stage LDS ring (XOR-swizzled 16-byte chunks), two tiles
//     ahead of the one computed.  bf16 inputs are loaded straight into LDS
//     (global_load_lds_dwordx4); fp32 inputs go through registers, rounded to
//     bf16.  One barrier per tile hands the landed tile to every wave.
//   * Persistent workgroups (one per CU) take groups from a counter, a few
//     heads at a time and longest first within them (see the schedule below).
//   * Waves w and w + 4 share a SIMD.  Waves 4-7 run one P V behind waves 0-3,
//     so that the two waves of a SIMD are in different phases of a tile.
//   * Online softmax in fp32, log2 domain: Q is pre-multiplied by
//     scale * log2(e), the score accumulators start at minus the row's
//     reference max, so exp2 reads the MFMA output directly.  The reference is
//     only raised when a tile exceeds it by more than 16 (and on the row's
//     first tile), so the O rescale is rare.  The row sum is a bf16 dot
//     product of the packed weights with ones (the same weights P V uses).
#include "attn_tile.h"
#include "nabla_launch.h"

namespace nabla {






__device__ __forceinline__ float max16(const f32x16 &s) {
    float x = fmaxf(s[0], s[1]);
#pragma unroll
    for (int j = 2; j < 16; ++j) x = fmaxf(x, s[j]);
    return x;
}

// Weights p = exp2(logit) of one 32-key half packed to bf16 (pb[p]: registers 8p ..
// 8p+7, the P V B operand of 16 consecutive keys); returns their sum, taken as a bf16
// dot product with ones so that the row sum uses exactly the weights P V uses.
__device__ __forceinline__ float expand(const f32x16 &s, bf16x8 (&pb)[2]) {
    typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int j = 0; j < 16; ++j) pb[j >> 3][j & 7] = (bf16)__builtin_amdgcn_exp2f(s[j]);
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
    float part[2] = {0.0f, 0.0f};
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const bf16x2 pr = {pb[pp][e], pb[pp][e + 1]};
            part[pp] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, part[pp], false);
        }
    return part[0] + part[1];
}


constexpr int kStages = 4;  // LDS ring: tiles k-1 (delayed P V), k, k+1, k+2 (landing)

template <int D>
struct AttnShared {
    bf16 ks[kStages][kBlock * D];
    bf16 vs[kStages][kBlock * D];
    uint64_t qmask[kGroup][kMaxWords];
    uint16_t ulist[kMaxWords * 64];  // the union of the members' lists, ascending
    uint8_t umem[kMaxWords * 64];    // bit s: member s lists that block
    int ucount;
    int slot;  // the schedule position this workgroup works on
};

// ---- schedule.  The cost of a group is the number of tiles in the union of its
// members' lists (the iterations of its walk).  Persistent workgroups take the next
// group from a counter.  The order is by phases of a few consecutive (batch, head)
// pairs, and within a phase the longest groups first (LPT).  Dynamic taking keeps every
// CU busy to the end whatever the per-head density; a phase big enough to pack well but
// far smaller than the whole launch keeps the K/V tiles that the running groups read to
// a few heads, which the memory-side cache holds (measured at 720p: 3.7 % less time
// than one longest-first order over all heads; one head per phase packs badly).

// grid = ceil(ngroups / 4), 256 lanes: wave w of workgroup x takes group 4x + w and ORs its
// members' lists into a bitmap of its own in LDS (no barrier); cost[g] = |union of the lists of
// group g|.  Workgroup 0 resets the counter.
__global__ __launch_bounds__(256) void attn_plan_cost_kernel(
    const int32_t *__restrict__ kv_nb, const int32_t *__restrict__ kv_inds, int nb, int Tt,
    int Ht, int Wt, int groups_per_bh, int ngroups, int32_t *__restrict__ cost,
    int32_t *__restrict__ counter) {
    __shared__ uint64_t bits[4][kMaxWords];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = blockIdx.x * 4 + w;
    if (blockIdx.x == 0 && threadIdx.x == 0) *counter = 0;
    if (g >= ngroups) return;  // wave-uniform; nothing below synchronizes waves
    const int bh = g / groups_per_bh, gi = g % groups_per_bh;
    uint64_t *bw = bits[w];
#pragma unroll
    for (int e = lane; e < kMaxWords; e += 64) bw[e] = 0ull;
    __builtin_amdgcn_wave_barrier();
    int n[kGroup];
    const int32_t *list[kGroup];
#pragma unroll
    for (int s = 0; s < kGroup; ++s) {
        const int m = group_member(gi, s, Tt, Ht, Wt, nb);
        const int64_t row = (int64_t)bh * nb + (m < 0 ? 0 : m);
        n[s] = m < 0 ? 0 : clamp_count(kv_nb[row], nb);
        list[s] = kv_inds + row * nb;
    }
    int nmax = 0;
#pragma unroll
    for (int s = 0; s < kGroup; ++s) nmax = max(nmax, n[s]);
    // 256 entries of every member per pass: all their loads issued before the first atomic
    constexpr int PL = 4;  // loads per lane and member
    for (int e0 = 0; e0 < nmax; e0 += 64 * PL) {
        int jj[kGroup][PL];
#pragma unroll
        for (int s = 0; s < kGroup; ++s)
#pragma unroll
            for (int u = 0; u < PL; ++u) {
                const int e = e0 + 64 * u + lane;
                jj[s][u] = e < n[s] ? list[s][e] : -1;
            }
#pragma unroll
        for (int s = 0; s < kGroup; ++s)
#pragma unroll
            for (int u = 0; u < PL; ++u)
                if (e0 + 64 * u + lane < n[s]) {
                    const int j = clamp_block(jj[s][u], nb);
                    atomicOr((unsigned long long *)&bw[j >> 6], 1ull << (j & 63));
                }
    }
    __builtin_amdgcn_wave_barrier();
    int cnt = 0;
#pragma unroll
    for (int wd = lane; wd < kMaxWords; wd += 64) cnt += __popcll(bw[wd]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off);
    if (lane == 0) cost[g] = cnt;
}

// One workgroup of 1024 lanes per phase.  Phase p holds the groups g of [p * per_phase,
// (p + 1) * per_phase), the last phase also the remainder up to ngroups; workgroup p
// writes them to the same positions of order[] by descending cost (counting sort; the
// order among equal costs is arbitrary and does not affect any result).
__global__ __launch_bounds__(1024) void attn_plan_order_kernel(const int32_t *__restrict__ cost,
                                                              int ngroups, int per_phase, int nb,
                                                              int32_t *__restrict__ order) {
    __shared__ int start[kMaxWords * 64 + 1];  // one bin per possible cost 0 .. nb
    __shared__ int part[2][1024];
    const int tid = threadIdx.x;
    const int g0 = blockIdx.x * per_phase;
    const int n = blockIdx.x + 1 == gridDim.x ? ngroups - g0 : per_phase;
    const int32_t *c = cost + g0;
    int32_t *out = order + g0;
    const int nbins = nb + 1;
    for (int b = tid; b < nbins; b += 1024) start[b] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += 1024) atomicAdd(&start[clamp_count(c[i], nb)], 1);
    __syncthreads();
    // thread t owns descending positions [t*chunk, (t+1)*chunk), position p = bin nb - p
    const int chunk = (nbins + 1023) / 1024;
    int sum = 0;
    for (int p = tid * chunk; p < (tid + 1) * chunk && p < nbins; ++p) sum += start[nb - p];
    part[0][tid] = sum;
    __syncthreads();
    int src = 0;
    for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan of the per-thread sums
        const int x = part[src][tid] + (tid >= off ? part[src][tid - off] : 0);
        part[src ^ 1][tid] = x;
        src ^= 1;
        __syncthreads();
    }
    int run = part[src][tid] - sum;  // exclusive
    for (int p = tid * chunk; p < (tid + 1) * chunk && p < nbins; ++p) {
        const int b = nb - p, n = start[b];
        start[b] = run;
        run += n;
    }
    __syncthreads();
    for (int i = tid; i < n; i += 1024) out[atomicAdd(&start[clamp_count(c[i], nb)], 1)] = g0 + i;
}

// kPad: the layout is a padded grid (Hv x Wv latents, partial patches); padding keys are
// masked.  The instance without it carries none of that code.
// kNat: q, k, v and o are in natural order (a grid of whole patches, rows of ng.W tokens);
// every row is read and written where the fractal permute would have moved it, so the
// arithmetic, and the result, are those of the fractal layout.  lse stays in fractal order.
template <int D, typename Tin, bool kPad, bool kNat>
__global__ __launch_bounds__(kAttnThreads) void sparse_attn_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
    Tin *__restrict__ o, int S, int heads, int Tt, int Ht, int Wt, int Hv, int Wv, NatGrid ng,
    int groups_per_bh,
    int ngroups, const int32_t *__restrict__ kv_nb, const int32_t *__restrict__ kv_inds,
    float scale_log2, const int32_t *__restrict__ order, int32_t *__restrict__ counter,
    float *__restrict__ lse) {
    constexpr int KS = D / 16;          // k-steps of the score product (16 dims each)
    constexpr int DT = D / 32;          // 32-wide output d tiles
    constexpr int CH = D / 8;           // 16-byte chunks per row
    constexpr int ROWB = D * 2;         // bytes per K/V row in LDS
    constexpr int CHUNKS = kBlock * CH; // 16-byte chunks per K (or V) tile
    constexpr int CPT = CHUNKS / kAttnThreads;  // chunks per thread per tile (K and V each)
    static_assert(CPT >= 1, "tile too small for the workgroup");
    static_assert(!(kPad && kNat), "the natural layout holds whole patches only");

    __shared__ __attribute__((aligned(1024))) AttnShared<D> sh;

    const int nb = S / kBlock;
    const int nwords = (nb + 63) >> 6;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;

    // persistent: take schedule positions until none is left (every wave of the
    // workgroup sees the same position, so all leave together)
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
    // union list: wave 0, lane = 64-block word (at most 64 words); an exclusive scan
    // of the words' popcounts places each lane's blocks
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
            const int o = __shfl_up(incl, d);
            if (lane >= d) incl += o;
        }
        int pos = incl - cnt;
        while (u != 0ull) {
            const int bit = __builtin_ctzll(u);
            u &= u - 1;
            int mem = 0;
#pragma unroll
            for (int s = 0; s < kGroup; ++s) mem |= (int)((sh.qmask[s][lane] >> bit) & 1ull) << s;
            sh.ulist[pos] = (uint16_t)(lane * 64 + bit);
            sh.umem[pos] = (uint8_t)mem;
            ++pos;
        }
        if (lane == 63) sh.ucount = incl;
    }
    __syncthreads();
    const int U = sh.ucount;  // tiles in the walk

    // ---- this wave: member slot and 32-row half
    // Waves w and w + 4 share a SIMD.  They take members of opposite corners of the
    // 2 x 1 x 2 box (slots 0 and 3, or 1 and 2), whose lists overlap least, so that
    // the two SIMD pairs of a step carry similar work.
    const int slot = w < 4 ? (w >> 1) : 3 - ((w - 4) >> 1);
    const int myblk = member[slot];
    const int64_t tok = (int64_t)heads * D;
    const int64_t head0 = (int64_t)b * S * tok + (int64_t)h * D;
    const int qtok = (myblk < 0 ? 0 : myblk) * kBlock + (w & 1) * 32 + l32;
    // the row's token in the layout of q and o
    const int64_t qrow = kNat ? (int64_t)nat_block_base(myblk < 0 ? 0 : myblk, ng) +
                                    nat_row_off((w & 1) * 32 + l32, ng.W)
                              : (int64_t)qtok;

    // Q^T as B operands, pre-multiplied by scale * log2(e) so that the score
    // MFMAs produce log2-domain logits directly
    bf16x8 qf[KS];
    if (myblk >= 0) {
        const Tin *qr = q + head0 + qrow * tok + 8 * hi;
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

    // ---- tile loads.  bf16: straight into LDS (lds_direct16), chunk e = r*threads + tid
    // of the tile lands at byte 16e of the stage, i.e. row e / CH, swizzled position
    // e % CH, so the lane fetches global chunk (e % CH) ^ swizzle(row).  fp32: through
    // registers (rounded to bf16), stored to the stage after the tile's compute.
    constexpr bool kDirect = sizeof(Tin) == 2;
    bf16x8 kst[kDirect ? 1 : CPT], vst[kDirect ? 1 : CPT];
    // per-lane byte offsets of the chunks within a tile (global side, swizzled)
    uint32_t koff[CPT], voff[CPT];
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
        const int e = r * kAttnThreads + tid;
        const int kv = e / CH, cpos = e % CH;
        const int64_t kvrow = kNat ? nat_row_off(kv, ng.W) : kv;
        koff[r] = (uint32_t)((kvrow * tok + 8 * (cpos ^ kswz<CH>(kv))) * sizeof(Tin));
        voff[r] = (uint32_t)((kvrow * tok + 8 * (cpos ^ vswz<CH>(kv))) * sizeof(Tin));
    }
    const uint32_t lds_k0 = __builtin_amdgcn_readfirstlane(lds_offset(sh.ks[0]) + w * 64 * 16);
    const uint32_t lds_v0 = __builtin_amdgcn_readfirstlane(lds_offset(sh.vs[0]) + w * 64 * 16);
    auto issue = [&](int jj, int stage) {
        const int j = __builtin_amdgcn_readfirstlane(jj);  // wave-uniform block index
        const int64_t jrow = kNat ? (int64_t)nat_block_base(j, ng) : (int64_t)j * kBlock;
        const Tin *kb = k + head0 + jrow * tok;
        const Tin *vb = v + head0 + jrow * tok;
#pragma unroll
        for (int r = 0; r < CPT; ++r) {
            if constexpr (kDirect) {
                const uint32_t sb = stage * (kBlock * D * 2) + r * kAttnThreads * 16;
                lds_direct16_sv(kb, koff[r], lds_k0 + sb);
                lds_direct16_sv(vb, voff[r], lds_v0 + sb);
            } else {
                const int e = r * kAttnThreads + tid;
                const int kv = e / CH, cpos = e % CH;
                const int64_t kvrow = kNat ? nat_row_off(kv, ng.W) : kv;
                kst[r] = load8_bf16(kb + kvrow * tok + 8 * cpos);
                vst[r] = load8_bf16(vb + kvrow * tok + 8 * cpos);
            }
        }
    };
    auto land = [&](int stage) {  // fp32 path: registers -> stage
        if constexpr (!kDirect) {
            char *kd = reinterpret_cast<char *>(sh.ks[stage]);
            char *vd = reinterpret_cast<char *>(sh.vs[stage]);
#pragma unroll
            for (int r = 0; r < CPT; ++r) {
                const int e = r * kAttnThreads + tid;
                const int kv = e / CH, c = e % CH;
                *reinterpret_cast<bf16x8 *>(kd + kv * ROWB + ((c ^ kswz<CH>(kv)) << 4)) = kst[r];
                *reinterpret_cast<bf16x8 *>(vd + kv * ROWB + ((c ^ vswz<CH>(kv)) << 4)) = vst[r];
            }
        }
    };
    // bf16: wait until only the loads issued for the newest tile (if any) are in flight
    auto settle = [&](bool newest_in_flight) {
        if constexpr (kDirect) {
            if (newest_in_flight)
                vm_wait<2 * CPT>();
            else
                vm_wait<0>();
        }
    };

    // V^T fragments of output d tile dt (A operands of the 4 P V k-steps kk = 2mt + p):
    // lane group g16 = lane / 16, s = lane % 16 points at V[key 32mt + 16p + 8(g16/2) +
    // 4r + s/4][d 32dt + 16(g16%2) + 4(s%4)], so the transpose read returns
    // V^T[32dt + l32][8 consecutive keys]
    auto vfrags_dt = [&](const char *vb, int dt, bf16x8 (&va)[4]) {
        const int g16 = lane >> 4, sl = lane & 15;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int mt = kk >> 1, p = kk & 1;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int kv = 32 * mt + 16 * p + 8 * (g16 >> 1) + 4 * r + (sl >> 2);
                const int d = 32 * dt + 16 * (g16 & 1) + 4 * (sl & 3);
                const int c = (d >> 3) ^ vswz<CH>(kv);
                const bf16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (NABLA_LDS bf16x4 *)(vb + kv * ROWB + (c << 4) + (d & 7) * 2));
                va[kk][4 * r + 0] = x[0];
                va[kk][4 * r + 1] = x[1];
                va[kk][4 * r + 2] = x[2];
                va[kk][4 * r + 3] = x[3];
            }
        }
    };

    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[dt][j] = 0.0f;
    float m_ref = 0.0f;       // reference max of the row, log2 units (raised lazily)
    f32x16 minit = splat16(0.0f);  // -m_ref in every element: the score accumulators' start
    bool m_valid = false;     // set by the row's first tile
    float l_run = 0.0f;       // this lane's part of the row sum

    // scores and softmax of the tile in `stage` -> packed weights pb (and O, l rescaled
    // when the reference max moves)
    auto score_softmax = [&](int stage, bf16x8 (&pb)[2][2], int vr, int vc) {
            const char *kb = reinterpret_cast<const char *>(sh.ks[stage]);
            // The LDS reads are issued well ahead of the MFMAs that use them (the
            // sched_barrier fences keep the compiler from sinking them next to their
            // uses): the K fragments of k-step ks + 3 under the score MFMAs of ks (a
            // ring of four k-steps), the first d tile's V^T fragments under the last
            // score MFMAs, and each next d tile's under the P V MFMAs of the current one.
            constexpr int KLA = 3;  // k-steps of K fragments in flight ahead of the MFMAs
            const int kv0 = sigma32(l32), kv1 = 32 + sigma32(l32);
            const char *krow0 = kb + kv0 * ROWB, *krow1 = kb + kv1 * ROWB;
            bf16x8 kf[KLA + 1][2];
            auto kread = [&](int ks) {
                const int c = 2 * ks + hi;
                kf[ks & KLA][0] =
                    *reinterpret_cast<const bf16x8 *>(krow0 + ((c ^ kswz<CH>(kv0)) << 4));
                kf[ks & KLA][1] =
                    *reinterpret_cast<const bf16x8 *>(krow1 + ((c ^ kswz<CH>(kv1)) << 4));
            };
#pragma unroll
            for (int ks = 0; ks < KLA; ++ks) kread(ks);
            // S^T - m = K Q^T (log2 units) for the two 32-key halves (two MFMA chains):
            // the first k-step reads its accumulator input from the -m block, so the
            // MFMAs also subtract the reference max
            f32x16 sacc[2];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + KLA < KS) kread(ks + KLA);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        kf[ks & KLA][mt], qf[ks], ks == 0 ? minit : sacc[mt], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_sched_barrier(0);
            // a partial patch of a padded grid (vr rows x vc columns of tokens): its padding
            // positions are not keys (register j of half mt holds key 32 mt + 16 (j / 8) +
            // 8 hi + j % 8)
            if (kPad && (vr < kTile || vc < kTile)) {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int key = 32 * mt + 16 * (j >> 3) + 8 * hi + (j & 7);
                        if (!((key >> 3) < vr && (key & 7) < vc)) sacc[mt][j] = -INFINITY;
                    }
            }
            float part = expand(sacc[0], pb[0]) + expand(sacc[1], pb[1]);
            // Lazy reference max.  The weights are formed against the current
            // reference; only when this lane's 32 weights of the tile sum to more
            // than 2^16 (a logit far above the reference; also inf), or on the row's
            // first tile, is the reference raised to the row max, O and l rescaled
            // and the weights formed again (wave-uniform branch, rare).
            if (__builtin_amdgcn_ballot_w64(!m_valid || !(part <= 65536.0f)) != 0ull) {
                const float lm = fmaxf(max16(sacc[0]), max16(sacc[1]));
                const float rm = fmaxf(lm, __shfl_xor(lm, 32));   // row max (shifted units)
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
                minit = splat16(-m_ref);
                part = expand(sacc[0], pb[0]) + expand(sacc[1], pb[1]);
            }
            l_run += part;
    };
    // O^T += V^T P^T for the tile in `stage`: 4 k-steps of 16 keys (mt, p) per output
    // d tile; each next d tile's V^T fragments are read under the current one's MFMAs
    auto pv_tile = [&](int stage, const bf16x8 (&pb)[2][2]) {
            const char *vb = reinterpret_cast<const char *>(sh.vs[stage]);
            bf16x8 va[2][4];
            vfrags_dt(vb, 0, va[0]);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                if (dt + 1 < DT) vfrags_dt(vb, dt + 1, va[(dt + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        va[dt & 1][kk], pb[kk >> 1][kk & 1], oacc[dt], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
    };
    bf16x8 pb_prev[2][2];      // packed weights of the previous tile (waves 4-7)
    bool prev_listed = false;  // waves 4-7: the previous tile's P V is still to do
    int prev_stage = 0;

    // ---- the walk over union tiles u_0, u_1, ...; u_k lives in LDS stage k % 4.
    // Step k: start loading u_{k+2} (its stage held u_{k-2}, whose last use, the
    // delayed P V, was in step k-1), compute, make sure u_{k+1} has landed, barrier.
    if (U > 0) {
        issue(sh.ulist[0], 0);
        land(0);
        if (U > 1) {
            issue(sh.ulist[1], 1);
            land(1);
        }
        settle(U > 1);
    }
    __syncthreads();

    // block of u_{k+2} and member bits of u_k, read one step ahead
    int pf_blk = U > 2 ? sh.ulist[2] : -1;
    int pf_mem = U > 0 ? sh.umem[0] : 0;
    for (int kk = 0, stage = 0; kk < U; ++kk, stage = (stage + 1) & (kStages - 1)) {
        const int n2 = __builtin_amdgcn_readfirstlane(pf_blk);  // u_{k+2}
        const int memk = __builtin_amdgcn_readfirstlane(pf_mem);
        pf_blk = kk + 3 < U ? sh.ulist[kk + 3] : -1;
        pf_mem = kk + 1 < U ? sh.umem[kk + 1] : 0;
        const int stage2 = (stage + 2) & (kStages - 1);
        if (n2 >= 0) issue(n2, stage2);
        const bool mine = myblk >= 0 && ((memk >> slot) & 1);
        // Waves w and w + 4 share a SIMD.  Waves 0-3 do tile k's scores, softmax and
        // P V in step k; waves 4-7 do tile k-1's P V first and then tile k's scores
        // and softmax, keeping the packed weights to the next step.  The two waves of
        // a SIMD are thus half a tile apart: one's softmax (VALU) runs under the
        // other's MFMAs instead of both waves doing the same phase at once.
        const bool delayed = w >= 4;
        if (delayed && prev_listed) pv_tile(prev_stage, pb_prev);
        if (mine) {
            int vr = kTile, vc = kTile;  // token rows / columns of the tile's patch
            if (kPad) {
                const int blk = __builtin_amdgcn_readfirstlane((int)sh.ulist[kk]);
                const int th = (blk / Wt) % Ht, tw = blk % Wt;
                vr = min(kTile, Hv - th * kTile);
                vc = min(kTile, Wv - tw * kTile);
            }
            bf16x8 pb[2][2];
            score_softmax(stage, pb, vr, vc);
            if (delayed) {
#pragma unroll
                for (int x = 0; x < 2; ++x)
#pragma unroll
                    for (int y = 0; y < 2; ++y) pb_prev[x][y] = pb[x][y];
            } else {
                pv_tile(stage, pb);
            }
        }
        prev_listed = delayed && mine;
        prev_stage = stage;
        if (n2 >= 0) land(stage2);
        settle(n2 >= 0);
        __syncthreads();  // u_{k+1} has landed; everyone is done with u_{k-1}'s stage
    }
    // the last tile's delayed P V (its stage is not reused before the next group)
    if (prev_listed) pv_tile(prev_stage, pb_prev);

    if (myblk >= 0) {
    const float lsum = l_run + __shfl_xor(l_run, 32);
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;  // empty list -> O = 0
    // natural-log log-sum-exp of the row's scaled scores: (m_ref + log2 l) * ln 2, with the
    // row sum of the weights P V used; -inf for an empty list
    if (lse != nullptr && hi == 0)
        lse[(int64_t)bh * S + qtok] =
            lsum > 0.0f ? (m_ref + log2f(lsum)) * 0.6931471805599453f : -INFINITY;
    Tin *orow = o + head0 + qrow * tok;
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
    }  // myblk >= 0
    __syncthreads();  // the next group reuses the LDS
    }  // persistent loop
}

// ---- host side

int attn_groups_per_bh(int S, int Tt, int Ht, int Wt) {
    const int nb = S / kBlock;
    return Tt > 0 ? ((Tt + 1) / 2) * Ht * (kGroup == 4 ? (Wt + 1) / 2 : Wt)
                  : (nb + kGroup - 1) / kGroup;
}

static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Schedule: [counter | cost[ngroups] | order[ngroups]], each part 256-byte aligned.
size_t attn_schedule_bytes(int B, int S, int heads, int Tt, int Ht, int Wt) {
    const size_t ngroups = (size_t)B * heads * attn_groups_per_bh(S, Tt, Ht, Wt);
    return 256 + 2 * round256(ngroups * sizeof(int32_t));
}

size_t sparse_attn_workspace_bytes(int B, int S, int heads, int Tt, int Ht, int Wt) {
    return attn_schedule_bytes(B, S, heads, Tt, Ht, Wt);
}

hipError_t launch_longest_first(const int32_t *cost, int n, int per_phase, int maxcost,
                                int32_t *order, hipStream_t stream) {
    const int nphases = n / per_phase > 0 ? n / per_phase : 1;
    hipLaunchKernelGGL(attn_plan_order_kernel, dim3(nphases), dim3(1024), 0, stream, cost, n,
                       per_phase < n ? per_phase : n, maxcost, order);
    return hipGetLastError();
}

AttnSchedule launch_attn_plan(const int32_t *kv_nb, const int32_t *kv_inds, int B, int S,
                              int heads, int Tt, int Ht, int Wt, int resident, void *ws,
                              hipStream_t stream) {
    AttnSchedule sc;
    const int nb = S / kBlock;
    sc.groups_per_bh = attn_groups_per_bh(S, Tt, Ht, Wt);
    sc.ngroups = B * heads * sc.groups_per_bh;
    char *wsb = static_cast<char *>(ws);
    sc.counter = reinterpret_cast<int32_t *>(wsb);
    int32_t *cost = reinterpret_cast<int32_t *>(wsb + 256);
    sc.order = reinterpret_cast<int32_t *>(wsb + 256 + round256((size_t)sc.ngroups * 4));
    hipLaunchKernelGGL(attn_plan_cost_kernel, dim3((sc.ngroups + 3) / 4), dim3(256), 0, stream,
                       kv_nb, kv_inds, nb, Tt, Ht, Wt, sc.groups_per_bh, sc.ngroups, cost,
                       sc.counter);
    // Heads per phase: enough groups that the phase, and above all the last one, keeps
    // every CU busy with room for longest-first packing (three groups per resident
    // workgroup), and at least two heads.
    const int gpb = sc.groups_per_bh;
    const int bh_total = B * heads;
    int hpp = (3 * resident + gpb - 1) / gpb;
    hpp = hpp < 2 ? 2 : (hpp > bh_total ? bh_total : hpp);
    const int nphases = bh_total / hpp;  // the remainder joins the last phase
    const int per_phase = hpp * gpb;
    hipLaunchKernelGGL(attn_plan_order_kernel, dim3(nphases), dim3(1024), 0, stream, cost,
                       sc.ngroups, per_phase, nb, sc.order);
    sc.grid = sc.ngroups < resident ? sc.ngroups : resident;
    return sc;
}

template <int D, typename Tin, bool kPad, bool kNat>
static hipError_t launch_attn_t(const void *q, const void *k, const void *v, int B, int S,
                                int heads, int Tt, int Ht, int Wt, int Hv, int Wv,
                                const int32_t *kv_nb,
                                const int32_t *kv_inds, float scale_log2, void *o, float *lse,
                                void *ws, hipStream_t stream) {
    const auto kernel = sparse_attn_kernel<D, Tin, kPad, kNat>;
    const int resident =
        resident_workgroups<sparse_attn_kernel<D, Tin, kPad, kNat>>(kAttnThreads);
    const NatGrid ng = nat_grid(kNat ? kTile * Wt : 0);
    if (resident <= 0) return hipErrorInvalidDevice;
    const AttnSchedule sc =
        launch_attn_plan(kv_nb, kv_inds, B, S, heads, Tt, Ht, Wt, resident, ws, stream);
    hipLaunchKernelGGL(kernel, dim3(sc.grid), dim3(kAttnThreads), 0, stream, (const Tin *)q,
                       (const Tin *)k, (const Tin *)v, (Tin *)o, S, heads, Tt, Ht, Wt, Hv, Wv, ng,
                       sc.groups_per_bh, sc.ngroups, kv_nb, kv_inds, scale_log2, sc.order,
                       sc.counter, lse);
    return hipGetLastError();
}

hipError_t launch_sparse_attn(const void *q, const void *k, const void *v, bool bf16_in,
                              int B, int S, int heads, int D, int Tt, int Ht, int Wt, int H,
                              int W, bool natural, const int32_t *kv_nb,
                              const int32_t *kv_inds, float scale, void *o, float *lse, void *ws,
                              hipStream_t stream) {
    const float scale_log2 = scale * 1.4426950408889634f;
    const bool pad = H > 0 && (H % kTile != 0 || W % kTile != 0);
#define NABLA_ATTN_T(DD, T, P, N, HV, WV) \
    launch_attn_t<DD, T, P, N>(q, k, v, B, S, heads, Tt, Ht, Wt, HV, WV, kv_nb, kv_inds, \
                               scale_log2, o, lse, ws, stream)
#define NABLA_ATTN(DD, T)                                        \
    return pad       ? NABLA_ATTN_T(DD, T, true, false, H, W)    \
           : natural ? NABLA_ATTN_T(DD, T, false, true, 0, 0)    \
                     : NABLA_ATTN_T(DD, T, false, false, 0, 0)
    if (D == 128) {
        if (bf16_in) NABLA_ATTN(128, bf16);
        NABLA_ATTN(128, float);
    }
    if (bf16_in) NABLA_ATTN(64, bf16);
    NABLA_ATTN(64, float);
#undef NABLA_ATTN
#undef NABLA_ATTN_T
}

}  // namespace nabla
