// block_mask.hip -- the NABLA block-mask estimator on gfx950.
//
// Follows the "nabla" page (FastVideo), nablaT_v2: map estimation (64-token
// mean pooling of q and k, qa @ ka^T / sqrt(D), row softmax), map binarization
// (ascending sort, cumulative sum, keep where the cumulative value reaches
// 1 - thr, back to block order), the STA union and the BlockMask lists
// (kv_nb = kept count, kv_inds = kept indices first); and the NABLA summary
// page, Technical Summary > Methodology ("Adaptive Mask Construction",
// "Hybrid Integration with STA").
//
// Precision: fp32 with a fixed order of every rounding step, so the integer
// outputs are reproducible bit for bit:
//   pool   sequential fp32 sum over the 64 tokens of a block, then * 2^-6;
//   score  acc = fma(qa[d], ka[d], acc), d = 0..D-1 from +0, then / fl32(sqrt D);
//          -0 becomes +0;
//   exp    Cody-Waite reduction n = rint(x log2 e), r = x - n ln2 (two-part
//          constant), degree-7 Taylor polynomial in Horner form with fma, times
//          2^n; 0 below x = -64;
//   soft   Z = sum of floor(e_j 2^48) (exact integer), rounded to fp32 via
//          double, times 2^-48; p_j = e_j / Z; P_j = floor(p_j 2^48);
//   order  ascending by (s_j, j); the cumulative mass is an exact integer sum,
//          so the first kept position does not depend on summation order.
// The row's arg-max block is always kept.
//
// The score chain runs on the fp32 matrix cores (v_mfma_f32_4x4x1_16b_f32 in the fused
// selection kernel, v_mfma_f32_32x32x2_f32 in scores_kernel): each MFMA step is one
// correctly rounded fma, applied in step order (measured on gfx950 against fmaf chains,
// subnormals included), so the chain over d ascending is exactly the one above.
//
// Kernels
//   pool_kernel         HBM-bound: each workgroup reads the 64 token rows of one block of
//                       q and k (16-byte coalesced loads) and writes heads*D fp32 means.
//   select_rows_kernel  rows of up to 512 blocks (and the top-k variant): one wave owns
//                       whole rows; q pooled here where it can be, k means staged in LDS
//                       per 4 dimensions, scores on the matrix cores, then per row: max,
//                       exp, Z, a histogram-refined search for the cut key over the 64-bit
//                       keys (orderable(s) << 12 | j) with exact integer masses, the STA
//                       union and a ballot compaction of the kept indices.
//   scores_kernel +     rows of 513-2048 blocks: the scores as a tiled product into a
//   select_rows_w4 /    workspace buffer, then the same selection, four waves per SIMD:
//   select_pair         one row per wave up to 1024 blocks, one row per pair of waves
//                       beyond (the waves meet in LDS around each row-wide quantity).
//   select_kernel       rows of more than 2048 blocks: a workgroup of eight waves per row.
#include "nabla_device.h"
#include "nabla_launch.h"

namespace nabla {

// ---------------------------------------------------------------- pool
// grid (nb, B): block i of q is pooled into qa [B*heads][nb][D] and block i of k into
// ka [B*heads][D/4][nb][4] (the layout the selection kernels read), or, KROW, into
// ka [B*heads][nb][D] like q (for scores_kernel: whole 512-byte rows per head, where the
// column layout's scattered 16-byte writes cost about a tenth of the kernel's time).  One
// workgroup does both, so that the whole grid is resident at once (no partial second round
// of workgroups).
// H, W > 0: the latent grid of a padded fractal layout (Wt = ceil(W/8) patches per row
// of patches): a block averages its tokens only, summed in order and divided by their
// count min(8, H - 8 ht) * min(8, W - 8 wt).  H = W = 0: whole 64-token blocks.
// ng.W > 0: q and k are in natural order (whole patches, rows of ng.W tokens); block i's
// rows are read where the fractal permute would have taken them from, in the same order.
// first = 1: k only (the fused selection kernel pools q itself).
// PAD: the instance for padded grids (H > 0); the other one has no per-row checks.
template <typename Tin, bool PAD, bool KROW>
__global__ __launch_bounds__(256) void pool_kernel(const Tin *__restrict__ q,
                                                   const Tin *__restrict__ k,
                                                   float *__restrict__ qa,
                                                   float *__restrict__ ka, int S, int heads,
                                                   int D, int H, int W, NatGrid ng, int first) {
    constexpr int EPC = 16 / sizeof(Tin);  // elements per 16-byte chunk
    const int nb = S / kBlock;
    const int i = blockIdx.x, b = blockIdx.y;
    const int row_elems = heads * D;
    const int nchunks = row_elems / EPC;
    int vrows = kTile, vcols = kTile;
    if (PAD && H > 0) {
        const int Ht = (H + kTile - 1) / kTile, Wt = (W + kTile - 1) / kTile;
        const int th = (i / Wt) % Ht, tw = i % Wt;
        vrows = min(kTile, H - th * kTile);
        vcols = min(kTile, W - tw * kTile);
    }
    const bool whole = !PAD || (vrows == kTile && vcols == kTile);
    const int cnt = vrows * vcols;
    for (int item = threadIdx.x + first * nchunks; item < 2 * nchunks; item += 256) {
    const int z = item >= nchunks;  // 0: q, 1: k
    const int ch = item - z * nchunks;
    const Tin *x = z ? k : q;
    float *xa = z ? ka : qa;
    const bool nat = ng.W > 0;
    const int rstep = nat ? ng.W : kTile;  // tokens between rows of a patch
    const int64_t blk0 = nat ? nat_block_base(i, ng) : (int64_t)i * kBlock;
    const Tin *base = x + ((int64_t)b * S + blk0) * row_elems;
    {
        float acc[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[e] = 0.0f;
        const Tin *p = base + ch * EPC;
        // 16 rows in flight per lane, then add them in token order
        for (int r0 = 0; r0 < kBlock; r0 += 16) {
            uint4 raw[16];
#pragma unroll
            for (int u = 0; u < 16; ++u)
                raw[u] = *reinterpret_cast<const uint4 *>(
                    p + (int64_t)(((r0 + u) >> 3) * rstep + ((r0 + u) & 7)) * row_elems);
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int r = r0 + u;
                if (!whole && !((r >> 3) < vrows && (r & 7) < vcols)) continue;  // padding
                if constexpr (sizeof(Tin) == 2) {
                    const uint32_t wd[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[2 * e] = acc[2 * e] + __uint_as_float(wd[e] << 16);
                        acc[2 * e + 1] = acc[2 * e + 1] + __uint_as_float(wd[e] & 0xffff0000u);
                    }
                } else {
                    acc[0] = acc[0] + __uint_as_float(raw[u].x);
                    acc[1] = acc[1] + __uint_as_float(raw[u].y);
                    acc[2] = acc[2] + __uint_as_float(raw[u].z);
                    acc[3] = acc[3] + __uint_as_float(raw[u].w);
                }
            }
        }
        const int el = ch * EPC;
        const int h = el / D, d = el - h * D;
        const int64_t bhh = (int64_t)b * heads + h;
#pragma unroll
        for (int e = 0; e < EPC; e += 4) {
            // q (and k with KROW): row-major [bh][nb][D]; k: [bh][D/4][nb] float4s, so that
            // the selection's score loop reads the k means of consecutive blocks from
            // consecutive addresses
            float *out = (z && !KROW) ? xa + ((bhh * (D / 4) + (d + e) / 4) * nb + i) * 4
                                      : xa + (bhh * nb + i) * D + d + e;
            // mean: * 2^-6 on whole blocks (exact, equal to / 64), else / token count
            float m[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                m[u] = whole ? acc[e + u] * 0.015625f : acc[e + u] / (float)cnt;
            *reinterpret_cast<float4 *>(out) = make_float4(m[0], m[1], m[2], m[3]);
        }
    }
    }
}

// ---------------------------------------------------------------- select helpers
// Branch-free: the polynomial runs on max(x, -64) and the result is selected, so that a
// wave evaluates it once with no divergent paths (x >= -64 takes exactly the same steps).
__device__ __forceinline__ float nabla_exp(float x_in) {
    const float x = fmaxf(x_in, -64.0f);
    const float log2e = 1.44269504088896341f;
    const float ln2_hi = 0.693145751953125f;
    const float ln2_lo = 1.42860682030941723e-6f;
    const float n = __builtin_rintf(x * log2e);
    float r = __builtin_fmaf(-n, ln2_hi, x);
    r = __builtin_fmaf(-n, ln2_lo, r);
    float p = 1.98412698412698413e-4f;
    p = __builtin_fmaf(p, r, 1.38888888888888889e-3f);
    p = __builtin_fmaf(p, r, 8.33333333333333333e-3f);
    p = __builtin_fmaf(p, r, 4.16666666666666667e-2f);
    p = __builtin_fmaf(p, r, 1.66666666666666667e-1f);
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    const float two_n = __int_as_float(((int)n + 127) << 23);
    return x_in >= -64.0f ? p * two_n : 0.0f;
}

// Monotone map of finite floats to unsigned ints (callers pass no -0).
__device__ __forceinline__ uint32_t f32_orderable(float s) {
    const uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_from_orderable(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// floor(v * 2^48) for 0 <= v <= 1, exactly and without branches: t = v * 2^16 is exact,
// its integer part h = trunc(t) <= 2^16 and its fraction f = t - h are exact (h is zero or
// at least t / 2), and f * 2^32 < 2^32 is exact, so floor(v * 2^48) = h * 2^32 +
// trunc(f * 2^32): h is the high word, trunc(f * 2^32) the low word.  Denormals and 0 give 0.
// (Equal, for every float in [0, 1], to the shift of the 24-bit significand by its exponent.)
__device__ __forceinline__ int64_t fix48(float v) {
    const float t = v * 65536.0f;
    const uint32_t h = (uint32_t)t;
    const float f = t - (float)h;
    const uint32_t l = (uint32_t)(f * 4294967296.0f);
    return (int64_t)(((uint64_t)h << 32) | l);
}

template <int NW>
struct SelectShared {
    int64_t hmass[1024];
    uint64_t hkey[1024];
    int hcnt[1024];
    uint64_t red_min[NW], red_max[NW];
    int64_t red_sum[NW];
    int64_t wsum[NW];
    int sel_bin, sel_cnt;
    int64_t sel_below;
    uint64_t sel_key;
};

// ---- wave-wide reductions and scans on DPP.  Each step is one VALU operation whose
// source is another lane of the wave: row_shr:k (within 16-lane rows), then row_bcast15
// (lane 15 of a row into the next row; rows 1 and 3 written) and row_bcast31 (lane 31 into
// rows 2 and 3).  Six steps give an inclusive scan over all 64 lanes; lane 63 then holds the
// whole-wave result, read back with v_readlane.  No LDS round trip.  Lanes without a
// source lane (the first k of a row, and the rows a broadcast does not write) keep `old`.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWS, 0xF, false);
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

__device__ __forceinline__ uint64_t u64_of(uint32_t lo, uint32_t hi) {
    return ((uint64_t)hi << 32) | lo;
}
// one scan step of a 64-bit value: v op= (the value at the DPP source lane, or `idle`
// where there is none)
template <int CTRL, int ROWS, typename Op>
__device__ __forceinline__ uint64_t dpp_step_u64(uint64_t v, uint64_t idle, Op op) {
    const uint32_t lo = dpp_u32<CTRL, ROWS>((uint32_t)idle, (uint32_t)v);
    const uint32_t hi = dpp_u32<CTRL, ROWS>((uint32_t)(idle >> 32), (uint32_t)(v >> 32));
    return op(v, u64_of(lo, hi));
}
template <typename Op>
__device__ __forceinline__ uint64_t wave_scan_u64(uint64_t v, uint64_t idle, Op op) {
    v = dpp_step_u64<kRowShr1, 0xF>(v, idle, op);
    v = dpp_step_u64<kRowShr2, 0xF>(v, idle, op);
    v = dpp_step_u64<kRowShr4, 0xF>(v, idle, op);
    v = dpp_step_u64<kRowShr8, 0xF>(v, idle, op);
    v = dpp_step_u64<kRowBcast15, 0xA>(v, idle, op);
    v = dpp_step_u64<kRowBcast31, 0xC>(v, idle, op);
    return v;
}
__device__ __forceinline__ uint64_t lane63_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
    return u64_of(lo, hi);
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
    // identity ~0: lanes without a source compare against the largest value
    return lane63_u64(wave_scan_u64(v, ~0ull, [](uint64_t a, uint64_t b) { return b < a ? b : a; }));
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    return lane63_u64(wave_scan_u64(v, 0ull, [](uint64_t a, uint64_t b) { return b > a ? b : a; }));
}
// inclusive prefix sum over the lanes (exact integer sums)
__device__ __forceinline__ int64_t wave_incl_scan_i64(int64_t v, int /*lane*/) {
    return (int64_t)wave_scan_u64((uint64_t)v, 0ull, [](uint64_t a, uint64_t b) { return a + b; });
}
__device__ __forceinline__ int64_t wave_sum_i64(int64_t v) {
    return (int64_t)lane63_u64((uint64_t)wave_incl_scan_i64(v, 0));
}

// ---------------------------------------------------------------- select (rows <= 2048)
// One wave owns RW whole rows: lane l holds the scores of columns j = 64c + l (c < CPT)
// of each of them, so the selection of a row is wave-local work with no barrier.
//
// Scores: the k means are read as float4s of consecutive blocks (coalesced, shared by
// the waves of the workgroup through L1); the q means of the wave's rows sit in LDS
// and are read as broadcasts.  Every score is the same sequential fma chain over d as
// above.
//
// Cut: the smallest key T whose inclusive prefix mass reaches cut.  One histogram pass
// over kSelBins bins of the score range [smin, smax] finds the bin holding it (the bin
// index is a monotone function of the score, so all keys of earlier bins are smaller
// and their exact mass is the prefix before the bin); the keys of that bin are then
// ranked exactly (at most 64 of them: one per lane), or, when more share the bin (ties,
// flat rows), the bin's key range is refined by further histogram passes first.
constexpr int kSelBins = 256;

struct SelectWaveScratch {
    int64_t hm[kSelBins];  // bin masses
    int hc[kSelBins];      // bin counts (rows of more than 1024 blocks)
    uint64_t lkey[64];     // keys of the cut bin
    int64_t lmass[64];
};

// fp32 max / min over the wave on DPP (lanes without a source keep their own value);
// exact whatever the order
template <bool MAX>
__device__ __forceinline__ float wave_ext_f32(float v) {
    auto step = [&](uint32_t t) {
        const float o = __uint_as_float(t);
        v = MAX ? fmaxf(v, o) : fminf(v, o);
    };
    step(dpp_u32<kRowShr1, 0xF>(__float_as_uint(v), __float_as_uint(v)));
    step(dpp_u32<kRowShr2, 0xF>(__float_as_uint(v), __float_as_uint(v)));
    step(dpp_u32<kRowShr4, 0xF>(__float_as_uint(v), __float_as_uint(v)));
    step(dpp_u32<kRowShr8, 0xF>(__float_as_uint(v), __float_as_uint(v)));
    step(dpp_u32<kRowBcast15, 0xA>(__float_as_uint(v), __float_as_uint(v)));
    step(dpp_u32<kRowBcast31, 0xC>(__float_as_uint(v), __float_as_uint(v)));
    return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 63));
}
__device__ __forceinline__ float wave_max_f32(float v) { return wave_ext_f32<true>(v); }
__device__ __forceinline__ float wave_min_f32(float v) { return wave_ext_f32<false>(v); }
// the value of lane `src` (wave-uniform) in every lane
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, src);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), src);
    return u64_of(lo, hi);
}

// TOPK: the top-k variant ("sla" page, get_block_map): scores without the 1/sqrt(D)
// scale, every block weighs one unit instead of its softmax weight, and `cut` is
// nb - k + 1, so the cut keeps exactly the k largest keys (none when k = 0).
// KST (rows of 129 blocks or more, 4+ column groups): the k means of one float4 column
// (4 dims of every block) are staged in LDS once per workgroup, double-buffered and loaded
// straight from memory into LDS, and the four waves read them from there; shorter rows read
// them from global memory through L1.
// PH: 0 = scores and selection in this kernel; 2 = selection only, the scores read from the
// score buffer sbuf [bh][nb][nb] that scores_kernel wrote (no q means, k means or staging).
//
// q != null (bf16, whole blocks; configurations whose lanes cover a row in 16-byte chunks):
// each wave pools its own RW query blocks from q (in place of reading qa), with the same
// arithmetic as pool_kernel (a sequential fp32 sum over the 64 tokens in token order, then
// * 2^-6): 64 / RW lanes per block, each summing D * RW / 64 dimensions.  The q reads then
// overlap the selection work of the other resident waves, and the pooling pass reads k only.
// S, heads, ng: q's layout (as pool_kernel).
template <int D, int CPT, int RW, bool TOPK, int PH>
__device__ __forceinline__ void select_rows_body(const float *__restrict__ qa,
                                                 const float *__restrict__ ka, int nb,
                                                 const uint8_t *__restrict__ sta, float sqrt_d,
                                                 int64_t cut, int32_t *__restrict__ kv_nb,
                                                 int32_t *__restrict__ kv_inds,
                                                 const bf16 *__restrict__ q, int S, int heads,
                                                 NatGrid ng, float *__restrict__ sbuf) {
    constexpr int NWV = 4;
    static_assert(PH == 0 || PH == 2, "fused (0) or selection from the score buffer (2)");
    constexpr bool SC = PH != 2;  // this launch computes the scores
    constexpr bool KST = SC && CPT >= 4;
    constexpr int KCOL = KST ? 64 * CPT : 1;  // float4s of one staged column (>= 256)
    constexpr int KRND = (KCOL + 255) / 256;   // staging rounds of 256 float4s (KCOL rounded up)
    __shared__ __attribute__((aligned(16))) float qs[NWV][SC ? RW : 1][SC ? D : 4];
    __shared__ SelectWaveScratch scr[NWV];
    __shared__ __attribute__((aligned(1024))) float4 kst[2][KST ? KRND * 256 : 1];
    const int bh = blockIdx.y, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int row0 = (blockIdx.x * NWV + wv) * RW;
    // with KST every wave takes part in the staging (loads and barriers) of the scores
    if (!KST && row0 >= nb) return;
    SelectWaveScratch &W = scr[wv];
    const uint64_t lanes_below = lane == 0 ? 0ull : (~0ull >> (64 - lane));

    constexpr int LPB = 64 / RW, DPL = D / LPB;  // lanes per query block, dims per lane
    constexpr int NCH = DPL / 8;                  // 16-byte chunks per lane and row
    // ---- scores (before the division by sqrt(D)) on the fp32 matrix cores.
    // v_mfma_f32_4x4x1_16b_f32 runs 16 blocks b = lane / 4 of D[4][4] += A[4][1] B[1][4]:
    // lane 4b + i supplies A_b[i], lane 4b + j supplies B_b[j], and register r of lane 4b + j
    // receives D_b[r][j], each step one fused multiply-add (measured on gfx950: bit-identical
    // to fmaf chained in step order, subnormals included).  With A = the q mean of row
    // (lane & 3) at dimension d and B = the k mean of block 64c + lane at d, for d ascending,
    // register r of chain (q, c) in lane l is the fp32 fma chain of row 4q + r against block
    // 64c + l: the score of the readings, at twice the unpacked vector fma rate and off the
    // vector ALU.  Waves of RW = 2 rows (the top-k variant's rows of more than 1024 blocks)
    // would leave half of each quad unused at twice the accumulator registers; they keep the
    // vector fma chain.
    constexpr bool MF = RW % 4 == 0;
    constexpr int NQ = MF ? RW / 4 : 1;
    f32x4 acc[NQ][MF ? CPT : 1];
    float vacc[MF ? 1 : RW][MF ? 1 : CPT];
#pragma unroll
    for (int qd = 0; qd < NQ; ++qd)
#pragma unroll
        for (int c = 0; c < (MF ? CPT : 1); ++c) acc[qd][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int r = 0; r < (MF ? 1 : RW); ++r)
#pragma unroll
        for (int c = 0; c < (MF ? 1 : CPT); ++c) vacc[r][c] = 0.0f;
    if constexpr (SC) {  // ---- q means, then the scores
    bool pooled = false;
    if constexpr (DPL % 8 == 0) {
        if (q != nullptr) {
            pooled = true;
            const int g = lane / LPB, li = lane - g * LPB, i = row0 + g;
            const int b = bh / heads, h = bh - b * heads;
            float acc[DPL];
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[e] = 0.0f;
            if (i < nb) {
                const bool nat = ng.W > 0;
                const int rstep = nat ? ng.W : kTile;  // tokens between rows of a patch
                const int64_t blk0 = nat ? nat_block_base(i, ng) : (int64_t)i * kBlock;
                const int64_t tok = (int64_t)heads * D;
                const bf16 *base = q + ((int64_t)b * S + blk0) * tok + (int64_t)h * D + 8 * li;
                constexpr int FL = 16 / NCH;  // rows in flight
                for (int r0 = 0; r0 < kBlock; r0 += FL) {
                    uint4 raw[FL][NCH];
#pragma unroll
                    for (int u = 0; u < FL; ++u)
#pragma unroll
                        for (int ch = 0; ch < NCH; ++ch)
                            raw[u][ch] = *reinterpret_cast<const uint4 *>(
                                base + (int64_t)(((r0 + u) >> 3) * rstep + ((r0 + u) & 7)) * tok +
                                8 * LPB * ch);
#pragma unroll
                    for (int u = 0; u < FL; ++u)
#pragma unroll
                        for (int ch = 0; ch < NCH; ++ch) {
                            const uint32_t wd[4] = {raw[u][ch].x, raw[u][ch].y, raw[u][ch].z,
                                                    raw[u][ch].w};
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                float &a0 = acc[8 * ch + 2 * e], &a1 = acc[8 * ch + 2 * e + 1];
                                a0 = a0 + __uint_as_float(wd[e] << 16);
                                a1 = a1 + __uint_as_float(wd[e] & 0xffff0000u);
                            }
                        }
                }
            }
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
                for (int e = 0; e < 8; ++e) qs[wv][g][8 * LPB * ch + 8 * li + e] = acc[8 * ch + e] * 0.015625f;
        }
    }
    if (!pooled)
        for (int e = lane; e < RW * D; e += 64) {
            const int r = e / D, d = e - r * D;
            qs[wv][r][d] = row0 + r < nb ? qa[((int64_t)bh * nb + row0 + r) * D + d] : 0.0f;
        }
    __builtin_amdgcn_wave_barrier();

    const float4 *kb = reinterpret_cast<const float4 *>(ka) + (int64_t)bh * (D / 4) * nb;
    // column d4 of the k means into buffer `buf`: float4 e = 256 r + tid lands at kst[buf][e]
    // (a wave's 64 lanes fill one contiguous KiB); lanes past the last block load the last
    // block's value again, so every wave issues the same number of loads (the staged values
    // past nb feed only columns that are not blocks)
    const uint32_t kst0 = __builtin_amdgcn_readfirstlane(lds_offset(&kst[0][0]) + wv * 1024);
    auto stage_col = [&](int d4, int buf) {
        if constexpr (KST) {
            const float4 *src = kb + (int64_t)d4 * nb;
#pragma unroll
            for (int r = 0; r < KRND; ++r) {
                const int e = r * 256 + (int)threadIdx.x;
                lds_direct16_sv(src, (uint32_t)(e < nb ? e : nb - 1) * 16u,
                                kst0 + (uint32_t)(buf * KRND * 4096 + r * 4096));
            }
        }
    };
    stage_col(0, 0);
#pragma unroll 1
    for (int d4 = 0; d4 < D / 4; ++d4) {
        float4 k4[CPT];
        if constexpr (KST) {
            vm_wait<0>();      // this wave's part of column d4 has landed
            __syncthreads();   // all of it has; every wave is done with column d4 - 1
            if (d4 + 1 < D / 4) stage_col(d4 + 1, (d4 + 1) & 1);
#pragma unroll
            for (int c = 0; c < CPT; ++c) k4[c] = kst[d4 & 1][64 * c + lane];
        } else {
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                const int j = 64 * c + lane;
                k4[c] = j < nb ? kb[(int64_t)d4 * nb + j] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        if constexpr (MF) {
#pragma unroll
            for (int qd = 0; qd < NQ; ++qd) {
                const float4 q4 =
                    *reinterpret_cast<const float4 *>(&qs[wv][4 * qd + (lane & 3)][4 * d4]);
#pragma unroll
                for (int c = 0; c < CPT; ++c)
                    acc[qd][c] = __builtin_amdgcn_mfma_f32_4x4x1f32(q4.x, k4[c].x, acc[qd][c], 0, 0, 0);
#pragma unroll
                for (int c = 0; c < CPT; ++c)
                    acc[qd][c] = __builtin_amdgcn_mfma_f32_4x4x1f32(q4.y, k4[c].y, acc[qd][c], 0, 0, 0);
#pragma unroll
                for (int c = 0; c < CPT; ++c)
                    acc[qd][c] = __builtin_amdgcn_mfma_f32_4x4x1f32(q4.z, k4[c].z, acc[qd][c], 0, 0, 0);
#pragma unroll
                for (int c = 0; c < CPT; ++c)
                    acc[qd][c] = __builtin_amdgcn_mfma_f32_4x4x1f32(q4.w, k4[c].w, acc[qd][c], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const float4 q4 = *reinterpret_cast<const float4 *>(&qs[wv][r][4 * d4]);
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    vacc[r][c] = __builtin_fmaf(q4.x, k4[c].x, vacc[r][c]);
                    vacc[r][c] = __builtin_fmaf(q4.y, k4[c].y, vacc[r][c]);
                    vacc[r][c] = __builtin_fmaf(q4.z, k4[c].z, vacc[r][c]);
                    vacc[r][c] = __builtin_fmaf(q4.w, k4[c].w, vacc[r][c]);
                }
            }
        }
    }
    }  // SC
    if (KST && row0 >= nb) return;  // no barrier below: waves are independent

    // ---- per row: softmax on the 2^-48 grid, cut key, STA union, compaction
#pragma unroll 1
    for (int r = 0; r < RW; ++r) {
        const int i = row0 + r;
        if (i >= nb) break;  // wave-uniform
        const int64_t row = (int64_t)bh * nb + i;
        float s[CPT];
        bool valid[CPT];
        float smax = -INFINITY, smin = INFINITY;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            valid[c] = 64 * c + lane < nb;
            if constexpr (PH == 2) {
                s[c] = valid[c] ? sbuf[row * nb + 64 * c + lane] : 0.0f;
            } else {
                float a = 0.0f;
#pragma unroll
                for (int rr = 0; rr < RW; ++rr)
                    if (rr == r) {
                        if constexpr (MF)
                            a = acc[rr >> 2][c][rr & 3];
                        else
                            a = vacc[rr][c];
                    }
                s[c] = (TOPK ? a : a / sqrt_d) + 0.0f;
            }
            if (valid[c]) {
                smax = fmaxf(smax, s[c]);
                smin = fminf(smin, s[c]);
            }
        }
        smax = wave_max_f32(smax);
        smin = wave_min_f32(smin);
        auto key_of = [&](int c) -> uint64_t {
            return ((uint64_t)f32_orderable(s[c]) << 12) | (uint64_t)(64 * c + lane);
        };

        // LEAN (rows of up to 1024 blocks): the weights are formed once and kept, and the cut
        // bin's members are counted with ballots.  Longer rows, already past 256 registers,
        // form the weights twice (for Z and for P) and count with LDS atomics instead.
        constexpr bool LEAN = CPT <= 16;
        int64_t P[CPT];
        if constexpr (TOPK) {
#pragma unroll
            for (int c = 0; c < CPT; ++c) P[c] = valid[c] ? 1 : 0;
        } else if constexpr (!LEAN) {
            int64_t esum = 0;
#pragma unroll
            for (int c = 0; c < CPT; ++c) esum += fix48(valid[c] ? nabla_exp(s[c] - smax) : 0.0f);
            esum = wave_sum_i64(esum);
            const float Z = (float)(double)esum * 0x1p-48f;
#pragma unroll
            for (int c = 0; c < CPT; ++c) P[c] = fix48(valid[c] ? nabla_exp(s[c] - smax) / Z : 0.0f);
        } else {
            float e[CPT];
            int64_t esum = 0;
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                e[c] = nabla_exp(valid[c] ? s[c] - smax : -INFINITY);  // 0 off the row
                esum += fix48(e[c]);
            }
            esum = wave_sum_i64(esum);
            const float Z = (float)(double)esum * 0x1p-48f;
#pragma unroll
            for (int c = 0; c < CPT; ++c) P[c] = fix48(e[c] / Z);  // e = 0 off the row
        }

        // One histogram pass over the members (inr) into kSelBins bins (bin_of); returns
        // the bin holding the cut (-1 if the members' mass stays below it) with the mass
        // before it, its count and, bit c of fbits, whether column group c of this lane is
        // in it (the count taken with ballots of those bits once the bin is known).
        static_assert(CPT <= 32, "one bit per column group");
        auto hist_pass = [&](auto inr, auto bin_of, int64_t below, int64_t &bbelow, int &bcnt,
                             uint32_t &fbits) {
#pragma unroll
            for (int q = 0; q < kSelBins / 64; ++q) {
                W.hm[lane * (kSelBins / 64) + q] = 0;
                if (!LEAN) W.hc[lane * (kSelBins / 64) + q] = 0;
            }
            __builtin_amdgcn_wave_barrier();
            // every lane adds for every column (non-members add 0 to bin 0): no divergent paths
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                const bool in = inr(c);
                const int bn = in ? bin_of(c) : 0;
                atomicAdd((unsigned long long *)&W.hm[bn], (unsigned long long)(in ? P[c] : 0));
                if (!LEAN) atomicAdd(&W.hc[bn], in ? 1 : 0);
            }
            __builtin_amdgcn_wave_barrier();
            int64_t m[kSelBins / 64];
            int64_t tot = 0;
#pragma unroll
            for (int q = 0; q < kSelBins / 64; ++q) {
                m[q] = W.hm[lane * (kSelBins / 64) + q];
                tot += m[q];
            }
            int64_t run = below + wave_incl_scan_i64(tot, lane) - tot;
            int found = -1;
            int64_t fb = 0;
#pragma unroll
            for (int q = 0; q < kSelBins / 64; ++q) {
                if (found < 0 && run < cut && run + m[q] >= cut) {
                    found = lane * (kSelBins / 64) + q;
                    fb = run;
                }
                run += m[q];
            }
            const uint64_t bal = __ballot(found >= 0);
            if (bal == 0ull) return -1;
            const int src = __builtin_ctzll(bal);
            bbelow = (int64_t)shfl_u64((uint64_t)fb, src);
            const int fbin = __builtin_amdgcn_readlane(found, src);
            fbits = 0;
#pragma unroll
            for (int c = 0; c < CPT; ++c) fbits |= (inr(c) && bin_of(c) == fbin ? 1u : 0u) << c;
            if constexpr (LEAN) {
                int n = 0;
#pragma unroll
                for (int c = 0; c < CPT; ++c) n += __popcll(__ballot((fbits >> c) & 1u));
                bcnt = n;
            } else {
                bcnt = W.hc[fbin];
            }
            return fbin;
        };
        // Exact rank of at most 64 members: the smallest key whose prefix reaches the cut.
        auto rank_list = [&](auto inr, int64_t below) -> uint64_t {
            int n = 0;
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                const bool in = inr(c);
                const uint64_t bal = __ballot(in);
                if (in) {
                    const int pos = n + __popcll(bal & lanes_below);
                    W.lkey[pos] = key_of(c);
                    W.lmass[pos] = P[c];
                }
                n += __popcll(bal);
            }
            __builtin_amdgcn_wave_barrier();
            uint64_t best = ~0ull;
            if (lane < n) {
                const uint64_t k0 = W.lkey[lane];
                int64_t pre = W.lmass[lane];
#pragma unroll 8
                for (int m = 0; m < n; ++m) pre += W.lkey[m] < k0 ? W.lmass[m] : 0;
                if (below + pre >= cut) best = k0;
            }
            return wave_min_u64(best);
        };

        uint64_t T = 0;  // cut <= 0: every block is kept
        if (cut > 0) {
            const float range = smax - smin;
            const float scale = range > 1e-30f ? (float)kSelBins / range : 0.0f;
            // bins of the score range (0 off the row).  One row per wave: computed once and kept
            // as bytes; several rows per wave (the fused kernel, registers held by the score
            // accumulators): recomputed where needed
            static_assert(kSelBins <= 256, "bins are kept in bytes");
            constexpr bool KEEPB = RW == 1;
            uint32_t bpk[KEEPB ? (CPT + 3) / 4 : 1];
            auto bin_of_score = [&](int c) -> uint32_t {
                const int bi = (int)((s[c] - smin) * scale);
                return valid[c] ? (uint32_t)(bi > kSelBins - 1 ? kSelBins - 1 : bi) : 0u;
            };
            if constexpr (KEEPB) {
#pragma unroll
                for (int u = 0; u < (CPT + 3) / 4; ++u) bpk[u] = 0;
#pragma unroll
                for (int c = 0; c < CPT; ++c) bpk[c >> 2] |= bin_of_score(c) << (8 * (c & 3));
            }
            auto bin_f = [&](int c) -> int {
                if constexpr (KEEPB)
                    return (int)((bpk[c >> 2] >> (8 * (c & 3))) & 0xffu);
                else
                    return (int)bin_of_score(c);
            };
            int64_t below = 0;
            int cnt = 0;
            uint32_t inb = 0;  // bit c: column group c of this lane is in the cut bin
            const int b = hist_pass([&](int c) { return valid[c]; }, bin_f, 0, below, cnt, inb);
            if (b < 0 && TOPK) {  // k = 0: no block is selected
                T = ~0ull;
            } else if (b < 0) {  // total mass below the cut: only the arg-max (largest key) stays
                uint64_t km = 0;
#pragma unroll
                for (int c = 0; c < CPT; ++c)
                    if (valid[c]) km = key_of(c) > km ? key_of(c) : km;
                T = wave_max_u64(km);
            } else if (cnt <= 64) {
                T = rank_list([&](int c) { return ((inb >> c) & 1u) != 0; }, below);
            } else {
                // many keys share the bin: narrow its key range by histogram passes
                uint64_t lo = ~0ull, hi = 0;
#pragma unroll
                for (int c = 0; c < CPT; ++c)
                    if ((inb >> c) & 1u) {
                        const uint64_t kk = key_of(c);
                        lo = kk < lo ? kk : lo;
                        hi = kk > hi ? kk : hi;
                    }
                lo = wave_min_u64(lo);
                hi = wave_max_u64(hi);
                for (;;) {
                    const uint64_t span = hi - lo;
                    const int shift = span < (uint64_t)kSelBins ? 0 : 64 - __clzll((long long)span) - 8;
                    auto inr = [&](int c) {
                        const uint64_t kk = key_of(c);
                        return valid[c] && kk >= lo && kk <= hi;
                    };
                    int64_t b2below = 0;
                    int c2 = 0;
                    uint32_t inb2 = 0;
                    const int b2 = hist_pass(inr, [&](int c) { return (int)((key_of(c) - lo) >> shift); },
                                             below, b2below, c2, inb2);
                    // b2 >= 0: the range holds the cut by construction
                    const uint64_t nlo = lo + ((uint64_t)b2 << shift);
                    const uint64_t nhi0 = nlo + ((1ull << shift) - 1);
                    const uint64_t nhi = nhi0 < hi ? nhi0 : hi;
                    if (c2 <= 64 || shift == 0 || b2 < 0) {
                        T = rank_list([&](int c) {
                            const uint64_t kk = key_of(c);
                            return valid[c] && kk >= nlo && kk <= nhi;
                        }, b2below);
                        break;
                    }
                    lo = nlo;
                    hi = nhi;
                    below = b2below;
                }
            }
        }

        // kept = key >= T, or the STA window; kv_inds ascending (j = 64c + lane)
        int base = 0;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int j = 64 * c + lane;
            const bool kept =
                valid[c] && (key_of(c) >= T || (sta != nullptr && sta[(int64_t)i * nb + j] != 0));
            const uint64_t bal = __ballot(kept);
            if (kept) kv_inds[row * nb + base + __popcll(bal & lanes_below)] = j;
            base += __popcll(bal);
        }
        if (lane == 0) kv_nb[row] = base;
        __builtin_amdgcn_wave_barrier();
    }
}

#define NABLA_SELECT_ARGS                                                                      \
    const float *__restrict__ qa, const float *__restrict__ ka, int nb,                        \
        const uint8_t *__restrict__ sta, float sqrt_d, int64_t cut,                            \
        int32_t *__restrict__ kv_nb, int32_t *__restrict__ kv_inds, const bf16 *__restrict__ q, \
        int S, int heads, NatGrid ng, float *__restrict__ sbuf
template <int D, int CPT, int RW, bool TOPK = false, int PH = 0>
__global__ __launch_bounds__(256) void select_rows_kernel(NABLA_SELECT_ARGS) {
    select_rows_body<D, CPT, RW, TOPK, PH>(qa, ka, nb, sta, sqrt_d, cut, kv_nb, kv_inds, q, S,
                                           heads, ng, sbuf);
}
// The selection launch of the two-launch path for rows of up to 16 column groups, held to
// 128 registers so that four waves per SIMD are resident.
template <int D, int CPT>
__global__ __launch_bounds__(256, 4) void select_rows_w4_kernel(NABLA_SELECT_ARGS) {
    select_rows_body<D, CPT, 1, false, 2>(qa, ka, nb, sta, sqrt_d, cut, kv_nb, kv_inds, q, S,
                                          heads, ng, sbuf);
}
#undef NABLA_SELECT_ARGS

// ---- rows of 1025-2048 blocks (30 or 32 column groups) from the score buffer, split over WV
// waves of one workgroup.  Wave v holds column groups CH v .. CH v + CH - 1; with WV = 2 and
// CH = 15 or 16 (as select_rows_w4_kernel holds a whole row of up to 1024 blocks) a wave fits
// in 128 registers and four waves per SIMD are resident, where a wave holding the whole row
// needs about 236 registers and runs two per SIMD.  The waves meet in LDS around every
// quantity of the whole row (extremes, Z, the histogram, the cut bin's members, the kept
// counts), with a workgroup barrier in between; each decision is taken from the same shared
// values in every wave, so all run the same path and the same barriers.  The arithmetic is
// select_rows_body's, and so are the lists.
template <int WV>
struct SelectPairShared {
    int64_t hm[kSelBins];  // the row's histogram masses
    uint64_t lkey[64];     // keys and masses of the cut bin's members
    int64_t lmass[64];
    float fmax[WV], fmin[WV];
    int64_t isum[WV];
    uint64_t kext[WV][2];  // per wave: lowest and highest member key (or the arg-max key)
    int cnt[WV];           // per wave: members of the cut bin
    int kcnt[WV];          // per wave: kept blocks
};

// Values the waves read back from LDS (or combine from it) are the same in every lane of a wave:
// readfirstlane makes them scalar, so that every branch on them, and the barriers inside such
// branches, is a uniform scalar branch.
__device__ __forceinline__ int uni_i32(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t uni_u64(uint64_t v) {
    return u64_of((uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v),
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32)));
}
__device__ __forceinline__ float uni_f32(float v) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

template <int CH, int WV>
__global__ __launch_bounds__(64 * WV, 4) void select_pair_kernel(
    int nb, const uint8_t *__restrict__ sta, int64_t cut, int32_t *__restrict__ kv_nb,
    int32_t *__restrict__ kv_inds, const float *__restrict__ sbuf) {
    static_assert(CH <= 32 && kSelBins == 256, "bit masks per column group; 4 bins per lane");
    __shared__ SelectPairShared<WV> sp;
    // sums over the waves of per-wave values in LDS: all, or those of the waves before this one
    auto all_of = [&](const int *a) {
        int t = 0;
#pragma unroll
        for (int w = 0; w < WV; ++w) t += a[w];
        return t;
    };
    auto before = [&](const int *a, int v) {
        int t = 0;
#pragma unroll
        for (int w = 0; w < WV; ++w) t += w < v ? a[w] : 0;
        return t;
    };
    const int i = blockIdx.x, bh = blockIdx.y;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t row = (int64_t)bh * nb + i;
    const uint64_t lanes_below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    auto col = [&](int c) { return 64 * (CH * wv + c) + lane; };

    float s[CH];
    bool valid[CH];
    float smax = -INFINITY, smin = INFINITY;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        valid[c] = col(c) < nb;
        s[c] = valid[c] ? sbuf[row * nb + col(c)] : 0.0f;
        if (valid[c]) {
            smax = fmaxf(smax, s[c]);
            smin = fminf(smin, s[c]);
        }
    }
    smax = wave_max_f32(smax);
    smin = wave_min_f32(smin);
    if (lane == 0) {
        sp.fmax[wv] = smax;
        sp.fmin[wv] = smin;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < WV; ++w) {
        smax = fmaxf(smax, sp.fmax[w]);
        smin = fminf(smin, sp.fmin[w]);
    }
    smax = uni_f32(smax);
    smin = uni_f32(smin);
    auto key_of = [&](int c) -> uint64_t {
        return ((uint64_t)f32_orderable(s[c]) << 12) | (uint64_t)col(c);
    };

    // weights on the 2^-48 grid: Z from the exact integer sum over both halves
    int64_t P[CH];
    {
        float e[CH];
        int64_t es = 0;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            e[c] = nabla_exp(valid[c] ? s[c] - smax : -INFINITY);  // 0 off the row
            es += fix48(e[c]);
        }
        es = wave_sum_i64(es);
        if (lane == 0) sp.isum[wv] = es;
        __syncthreads();
        es = 0;
#pragma unroll
        for (int w = 0; w < WV; ++w) es += sp.isum[w];
        es = (int64_t)uni_u64((uint64_t)es);
        const float Z = (float)(double)es * 0x1p-48f;
#pragma unroll
        for (int c = 0; c < CH; ++c) P[c] = fix48(e[c] / Z);
    }

    // One histogram pass over the members (inr) of both waves into the shared bins (bin_of):
    // the bin holding the cut (-1 if the members' mass stays below it), the mass before it, the
    // members of that bin in both waves, and this wave's member bits.
    auto hist_pass = [&](auto inr, auto bin_of, int64_t below, int64_t &bbelow, int &bcnt,
                         uint32_t &fbits) -> int {
        for (int t = threadIdx.x; t < kSelBins; t += 64 * WV) sp.hm[t] = 0;
        __syncthreads();
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const bool in = inr(c);
            const int bn = in ? bin_of(c) : 0;
            atomicAdd((unsigned long long *)&sp.hm[bn], (unsigned long long)(in ? P[c] : 0));
        }
        __syncthreads();
        // every wave scans all bins (lane l: bins 4l .. 4l + 3) and finds the same bin
        int64_t m[kSelBins / 64];
        int64_t tot = 0;
#pragma unroll
        for (int q = 0; q < kSelBins / 64; ++q) {
            m[q] = sp.hm[lane * (kSelBins / 64) + q];
            tot += m[q];
        }
        int64_t run = below + wave_incl_scan_i64(tot, lane) - tot;
        int found = -1;
        int64_t fb = 0;
#pragma unroll
        for (int q = 0; q < kSelBins / 64; ++q) {
            if (found < 0 && run < cut && run + m[q] >= cut) {
                found = lane * (kSelBins / 64) + q;
                fb = run;
            }
            run += m[q];
        }
        const uint64_t bal = __ballot(found >= 0);
        if (bal == 0ull) return -1;  // the same in both waves
        const int src = __builtin_ctzll(bal);
        bbelow = (int64_t)shfl_u64((uint64_t)fb, src);
        const int fbin = __builtin_amdgcn_readlane(found, src);
        fbits = 0;
#pragma unroll
        for (int c = 0; c < CH; ++c) fbits |= (inr(c) && bin_of(c) == fbin ? 1u : 0u) << c;
        int n = 0;
#pragma unroll
        for (int c = 0; c < CH; ++c) n += __popcll(__ballot((fbits >> c) & 1u));
        if (lane == 0) sp.cnt[wv] = n;
        __syncthreads();
        bcnt = uni_i32(all_of(sp.cnt));
        return fbin;
    };
    // Exact rank of the at most 64 members (bits mb) of the last pass's bin: wave 0's first,
    // then wave 1's; the smallest key whose prefix reaches the cut.
    auto rank_list = [&](uint32_t mb, int64_t below) -> uint64_t {
        int n = uni_i32(before(sp.cnt, wv));
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const bool in = (mb >> c) & 1u;
            const uint64_t bal = __ballot(in);
            if (in) {
                const int pos = n + __popcll(bal & lanes_below);
                sp.lkey[pos] = key_of(c);
                sp.lmass[pos] = P[c];
            }
            n += __popcll(bal);
        }
        __syncthreads();
        const int total = uni_i32(all_of(sp.cnt));
        uint64_t best = ~0ull;
        if (lane < total) {
            const uint64_t k0 = sp.lkey[lane];
            int64_t pre = sp.lmass[lane];
#pragma unroll 8
            for (int m2 = 0; m2 < total; ++m2) pre += sp.lkey[m2] < k0 ? sp.lmass[m2] : 0;
            if (below + pre >= cut) best = k0;
        }
        return wave_min_u64(best);
    };

    uint64_t T = 0;  // cut <= 0: every block is kept
    if (cut > 0) {
        const float range = smax - smin;
        const float scale = range > 1e-30f ? (float)kSelBins / range : 0.0f;
        uint32_t bpk[(CH + 3) / 4];  // the bins, as bytes (0 off the row)
#pragma unroll
        for (int u = 0; u < (CH + 3) / 4; ++u) bpk[u] = 0;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int bi = (int)((s[c] - smin) * scale);
            const uint32_t bc = valid[c] ? (uint32_t)(bi > kSelBins - 1 ? kSelBins - 1 : bi) : 0u;
            bpk[c >> 2] |= bc << (8 * (c & 3));
        }
        auto bin_f = [&](int c) -> int { return (int)((bpk[c >> 2] >> (8 * (c & 3))) & 0xffu); };
        int64_t below = 0;
        int cnt = 0;
        uint32_t inb = 0;
        const int b = hist_pass([&](int c) { return valid[c]; }, bin_f, 0, below, cnt, inb);
        if (b < 0) {  // total mass below the cut: only the arg-max (largest key) stays
            uint64_t km = 0;
#pragma unroll
            for (int c = 0; c < CH; ++c)
                if (valid[c]) km = key_of(c) > km ? key_of(c) : km;
            km = wave_max_u64(km);
            if (lane == 0) sp.kext[wv][1] = km;
            __syncthreads();
#pragma unroll
            for (int w = 0; w < WV; ++w) T = sp.kext[w][1] > T ? sp.kext[w][1] : T;
            T = uni_u64(T);
        } else if (cnt <= 64) {
            T = rank_list(inb, below);
        } else {
            // many keys share the bin: narrow its key range by histogram passes
            uint64_t lo = ~0ull, hi = 0;
#pragma unroll
            for (int c = 0; c < CH; ++c)
                if ((inb >> c) & 1u) {
                    const uint64_t kk = key_of(c);
                    lo = kk < lo ? kk : lo;
                    hi = kk > hi ? kk : hi;
                }
            lo = wave_min_u64(lo);
            hi = wave_max_u64(hi);
            if (lane == 0) {
                sp.kext[wv][0] = lo;
                sp.kext[wv][1] = hi;
            }
            __syncthreads();
#pragma unroll
            for (int w = 0; w < WV; ++w) {
                lo = sp.kext[w][0] < lo ? sp.kext[w][0] : lo;
                hi = sp.kext[w][1] > hi ? sp.kext[w][1] : hi;
            }
            lo = uni_u64(lo);
            hi = uni_u64(hi);
            for (;;) {
                const uint64_t span = hi - lo;
                const int shift = span < (uint64_t)kSelBins ? 0 : 64 - __clzll((long long)span) - 8;
                int64_t b2below = 0;
                int c2 = 0;
                uint32_t inb2 = 0;
                const int b2 = hist_pass(
                    [&](int c) {
                        const uint64_t kk = key_of(c);
                        return valid[c] && kk >= lo && kk <= hi;
                    },
                    [&](int c) { return (int)((key_of(c) - lo) >> shift); }, below, b2below, c2,
                    inb2);
                if (b2 < 0) {  // not reached: the range holds the cut by construction
                    T = lo;
                    break;
                }
                if (c2 <= 64 || shift == 0) {
                    T = rank_list(inb2, b2below);
                    break;
                }
                const uint64_t nlo = lo + ((uint64_t)b2 << shift);
                const uint64_t nhi0 = nlo + ((1ull << shift) - 1);
                lo = nlo;
                hi = nhi0 < hi ? nhi0 : hi;
                below = b2below;
            }
        }
    }

    // kept = key >= T, or the STA window; kv_inds ascending: wave 0's columns, then wave 1's
    uint32_t kbits = 0;
    int n = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const bool kept =
            valid[c] && (key_of(c) >= T || (sta != nullptr && sta[(int64_t)i * nb + col(c)] != 0));
        kbits |= (kept ? 1u : 0u) << c;
        n += __popcll(__ballot(kept));
    }
    if (lane == 0) sp.kcnt[wv] = n;
    __syncthreads();
    int base = uni_i32(before(sp.kcnt, wv));
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const bool kept = (kbits >> c) & 1u;
        const uint64_t bal = __ballot(kept);
        if (kept) kv_inds[row * nb + base + __popcll(bal & lanes_below)] = col(c);
        base += __popcll(bal);
    }
    if (threadIdx.x == 0) kv_nb[row] = all_of(sp.kcnt);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---- block scores as a tiled product (the two-launch path, rows of 513-2048 blocks).
// S[bh][i][j] = fl32(dot(qa_i, ka_j)) / fl32(sqrt D), -0 stored as +0, for one 64 x 64 block of
// one (b, head) per workgroup; qa and ka both row-major [bh][nb][D].  d runs in chunks of 32: a
// chunk of the block's 64 q means and 64 k means is staged in LDS, d-major (row pitch 65 floats,
// conflict-free operand reads), while
// the next chunk's global loads are already in flight in registers; each of the four waves
// computes a 32 x 32 tile with v_mfma_f32_32x32x2_f32, two dimensions per step, d ascending.
// Lane l supplies A = qa[row l % 32][d + l / 32] and B = ka[block l % 32][d + l / 32];
// register r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.  A chain of
// these steps gives bits identical to fmaf chained in d order (measured on gfx950,
// subnormals included), so each score is the readings' fp32 fma chain over d.  The small LDS
// footprint (16.6 KiB) leaves room for eight workgroups per CU to cover each other's loads.
// grid: nt * nt * BH workgroups in one dimension (nt = ceil(nb / 64)).  Workgroups go to the
// eight XCDs in turn by id; when the count divides by eight, id n takes tile
// (n mod 8) * count / 8 + n / 8 in (bh, row tile, column tile) order, so that each XCD works on
// one eighth of the (b, head) pairs and their pooled q and k stay in its own L2.
template <int D>
__global__ __launch_bounds__(256, 8) void scores_kernel(const float *__restrict__ qa,
                                                     const float *__restrict__ ka, int nb,
                                                     float sqrt_d, float *__restrict__ sbuf) {
    constexpr int P = 65, KC = 32, NCK = D / KC;  // pitch; dimensions per chunk; chunks
    constexpr int C4 = KC / 4;                    // float4s per row and chunk
    constexpr int NL = 64 * C4 / 256;             // float4 loads per lane, operand and chunk
    __shared__ float As[KC][P], Bs[KC][P];
    const int nt = (nb + 63) / 64, count = (int)gridDim.x;
    int n = (int)blockIdx.x;
    if (count % 8 == 0) n = (n % 8) * (count / 8) + n / 8;
    const int bh = n / (nt * nt), tt = n - bh * nt * nt;
    const int i0 = (tt / nt) * 64, j0 = (tt % nt) * 64;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const float *qb = qa + (int64_t)bh * nb * D;  // [nb][D]
    const float *kb = ka + (int64_t)bh * nb * D;  // [nb][D] (the pooling pass's row-major k means)
    // chunk loads: 64 rows x C4 float4s of each operand, NL per lane each, d fastest (coalesced)
    float4 xa[NL], xb[NL];
    auto load = [&](int ck) {
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int e = u * 256 + tid;
            const int r = e / C4, dc = e % C4;
            const int64_t off = (int64_t)r * D + ck * KC + 4 * dc;
            xa[u] = i0 + r < nb ? *reinterpret_cast<const float4 *>(qb + (int64_t)i0 * D + off)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
            xb[u] = j0 + r < nb ? *reinterpret_cast<const float4 *>(kb + (int64_t)j0 * D + off)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int e = u * 256 + tid;
            const int r = e / C4, dc = e % C4;
            As[4 * dc + 0][r] = xa[u].x;
            As[4 * dc + 1][r] = xa[u].y;
            As[4 * dc + 2][r] = xa[u].z;
            As[4 * dc + 3][r] = xa[u].w;
            Bs[4 * dc + 0][r] = xb[u].x;
            Bs[4 * dc + 1][r] = xb[u].y;
            Bs[4 * dc + 2][r] = xb[u].z;
            Bs[4 * dc + 3][r] = xb[u].w;
        }
    };
    const int wi = (w >> 1) * 32, wj = (w & 1) * 32, hi = lane >> 5, l32 = lane & 31;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    load(0);
#pragma unroll 1
    for (int ck = 0; ck < NCK; ++ck) {
        store();
        __syncthreads();                  // chunk ck staged
        if (ck + 1 < NCK) load(ck + 1);   // in flight under this chunk's MFMAs
#pragma unroll
        for (int d = 0; d < KC; d += 2)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[d + hi][wi + l32], Bs[d + hi][wj + l32],
                                                        acc, 0, 0, 0);
        __syncthreads();                  // every wave is done with chunk ck
    }
    float *sb = sbuf + (int64_t)bh * nb * nb;
    const int j = j0 + wj + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = i0 + wi + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (i < nb && j < nb) sb[(int64_t)i * nb + j] = acc[r] / sqrt_d + 0.0f;
    }
}

// ---------------------------------------------------------------- select (long rows)
// Rows of more than 2048 blocks.  grid (ceil(nb / R), B*heads); 512 lanes; lane t owns
// columns j = c*512 + t, c < CPT; the whole workgroup works on one row at a time.
template <int D, int CPT, int R>
__global__ __launch_bounds__(512) void select_kernel(const float *__restrict__ qa,
                                                     const float *__restrict__ ka, int nb,
                                                     const uint8_t *__restrict__ sta,
                                                     float sqrt_d, int64_t cut,
                                                     int32_t *__restrict__ kv_nb,
                                                     int32_t *__restrict__ kv_inds) {
    constexpr int NT = 512, NW = NT / 64;
    __shared__ __attribute__((aligned(16))) float qs[R][D];
    __shared__ SelectShared<NW> sh;
    __shared__ int ccount[CPT][NW];

    const int bh = blockIdx.y;
    const int row0 = blockIdx.x * R;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    for (int e = tid; e < R * D; e += NT) {
        const int r = e / D, d = e - r * D;
        qs[r][d] = (row0 + r < nb) ? qa[((int64_t)bh * nb + row0 + r) * D + d] : 0.0f;
    }
    __syncthreads();

    // ---- scores: acc[r][c] = sum_d fma order, d ascending
    float acc[R][CPT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < CPT; ++c) acc[r][c] = 0.0f;
    const float4 *kab = reinterpret_cast<const float4 *>(ka) + (int64_t)bh * (D / 4) * nb;
    for (int d = 0; d < D; d += 4) {
        float4 kv[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int j = c * NT + tid;
            kv[c] = (j < nb) ? kab[(int64_t)(d / 4) * nb + j] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float4 q4 = *reinterpret_cast<const float4 *>(&qs[r][d]);
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                acc[r][c] = __builtin_fmaf(q4.x, kv[c].x, acc[r][c]);
                acc[r][c] = __builtin_fmaf(q4.y, kv[c].y, acc[r][c]);
                acc[r][c] = __builtin_fmaf(q4.z, kv[c].z, acc[r][c]);
                acc[r][c] = __builtin_fmaf(q4.w, kv[c].w, acc[r][c]);
            }
        }
    }

    // ---- per row selection
#pragma unroll 1
    for (int r = 0; r < R; ++r) {
        const int i = row0 + r;
        if (i >= nb) break;  // uniform over the workgroup
        const int64_t row = (int64_t)bh * nb + i;

        float s[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            float a = 0.0f;
#pragma unroll
            for (int rr = 0; rr < R; ++rr)
                if (rr == r) a = acc[rr][c];
            s[c] = a / sqrt_d + 0.0f;
        }
        bool valid[CPT];
        uint64_t key[CPT];
        uint64_t kmin = ~0ull, kmax = 0;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int j = c * NT + tid;
            valid[c] = j < nb;
            key[c] = ((uint64_t)f32_orderable(s[c]) << 12) | (uint64_t)j;
            if (valid[c]) {
                kmin = key[c] < kmin ? key[c] : kmin;
                kmax = key[c] > kmax ? key[c] : kmax;
            }
        }
        kmin = wave_min_u64(kmin);
        kmax = wave_max_u64(kmax);
        if (lane == 0) { sh.red_min[wave] = kmin; sh.red_max[wave] = kmax; }
        __syncthreads();
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            kmin = sh.red_min[w] < kmin ? sh.red_min[w] : kmin;
            kmax = sh.red_max[w] > kmax ? sh.red_max[w] : kmax;
        }
        kmin = uni_u64(kmin);
        kmax = uni_u64(kmax);
        const float smax = f32_from_orderable((uint32_t)(kmax >> 12));

        // softmax weights on the 2^-48 grid
        float e[CPT];
        int64_t esum = 0;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            e[c] = nabla_exp(valid[c] ? s[c] - smax : -INFINITY);  // 0 off the row
            esum += fix48(e[c]);
        }
        esum = wave_sum_i64(esum);
        if (lane == 0) sh.red_sum[wave] = esum;
        __syncthreads();
        int64_t ze = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) ze += sh.red_sum[w];
        ze = (int64_t)uni_u64((uint64_t)ze);
        const float Z = (float)(double)ze * 0x1p-48f;
        int64_t P[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) P[c] = fix48(e[c] / Z);  // e = 0 off the row

        // cut key T: the smallest key whose inclusive prefix mass reaches cut
        uint64_t T;
        if (cut <= 0) {
            T = kmin;
        } else {
            uint64_t lo = kmin, hi = kmax;
            int64_t below = 0;
            for (;;) {
                const uint64_t range = hi - lo;
                const int shift = range < 1024 ? 0 : (64 - __clzll((long long)range) - 10);
                for (int bn = tid; bn < 1024; bn += NT) {
                    sh.hmass[bn] = 0;
                    sh.hcnt[bn] = 0;
                    sh.hkey[bn] = 0;
                }
                __syncthreads();
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    if (valid[c] && key[c] >= lo && key[c] <= hi) {
                        const int bn = (int)((key[c] - lo) >> shift);
                        atomicAdd((unsigned long long *)&sh.hmass[bn], (unsigned long long)P[c]);
                        atomicAdd(&sh.hcnt[bn], 1);
                        atomicMax((unsigned long long *)&sh.hkey[bn], (unsigned long long)key[c]);
                    }
                }
                __syncthreads();
                if (tid == 0) sh.sel_bin = -1;
                const int64_t m0 = sh.hmass[2 * tid], m1 = sh.hmass[2 * tid + 1];
                const int64_t incl = wave_incl_scan_i64(m0 + m1, lane);
                if (lane == 63) sh.wsum[wave] = incl;
                __syncthreads();
                int64_t before = below + incl - (m0 + m1);
                for (int w = 0; w < wave; ++w) before += sh.wsum[w];
                int found = -1;
                int64_t fb = 0;
                if (before < cut && before + m0 >= cut) {
                    found = 2 * tid;
                    fb = before;
                } else if (before + m0 < cut && before + m0 + m1 >= cut) {
                    found = 2 * tid + 1;
                    fb = before + m0;
                }
                if (found >= 0) {
                    sh.sel_bin = found;
                    sh.sel_below = fb;
                    sh.sel_cnt = sh.hcnt[found];
                    sh.sel_key = sh.hkey[found];
                }
                __syncthreads();
                const int bsel = uni_i32(sh.sel_bin);
                if (bsel < 0) {  // total mass below the cut: keep only the arg-max
                    T = kmax;
                    break;
                }
                if (uni_i32(sh.sel_cnt) == 1 || shift == 0) {
                    T = uni_u64(sh.sel_key);
                    break;
                }
                below = (int64_t)uni_u64((uint64_t)sh.sel_below);
                const uint64_t nlo = lo + ((uint64_t)bsel << shift);
                const uint64_t nhi = nlo + ((1ull << shift) - 1);
                lo = nlo;
                hi = nhi < hi ? nhi : hi;
            }
        }

        // kept = sorted position >= cut position, OR the STA window
        bool kept[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int j = c * NT + tid;
            kept[c] = valid[c] && (key[c] >= T || (sta != nullptr && sta[(int64_t)i * nb + j] != 0));
        }
        // compaction: ascending j = (c, wave, lane)
        uint64_t ball[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            ball[c] = __ballot(kept[c]);
            if (lane == 0) ccount[c][wave] = __popcll(ball[c]);
        }
        __syncthreads();
        int base = 0;
        const uint64_t below_lane = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            int off = base;
            for (int w = 0; w < wave; ++w) off += ccount[c][w];
            for (int w = 0; w < NW; ++w) base += ccount[c][w];
            if (kept[c]) kv_inds[row * nb + off + __popcll(ball[c] & below_lane)] = c * NT + tid;
        }
        if (tid == 0) kv_nb[row] = base;
    }
}

template <int D, int CPT, int R>
static hipError_t launch_select_t(const float *qa, const float *ka, int BH, int nb,
                                  const uint8_t *sta, float sqrt_d, int64_t cut, int32_t *kv_nb,
                                  int32_t *kv_inds, hipStream_t stream) {
    dim3 grid((nb + R - 1) / R, BH);
    hipLaunchKernelGGL((select_kernel<D, CPT, R>), grid, dim3(512), 0, stream, qa, ka, nb, sta,
                       sqrt_d, cut, kv_nb, kv_inds);
    return hipGetLastError();
}

// The query layout the selection kernel pools q from (q null: it reads the pooled qa).
struct QSource {
    const bf16 *q;
    int S, heads;
    NatGrid ng;
};

template <int D, int CPT, int RW, bool TOPK = false, int PH = 0>
static hipError_t launch_rows_t(const float *qa, const float *ka, int BH, int nb,
                                const uint8_t *sta, float sqrt_d, int64_t cut, int32_t *kv_nb,
                                int32_t *kv_inds, hipStream_t stream, QSource qsrc = {},
                                float *sbuf = nullptr) {
    dim3 grid((nb + 4 * RW - 1) / (4 * RW), BH);
    hipLaunchKernelGGL((select_rows_kernel<D, CPT, RW, TOPK, PH>), grid, dim3(256), 0, stream, qa,
                       ka, nb, sta, sqrt_d, cut, kv_nb, kv_inds, qsrc.q, qsrc.S, qsrc.heads,
                       qsrc.ng, sbuf);
    return hipGetLastError();
}

// Rows of 513-2048 blocks in two launches through the score buffer sbuf [BH][nb][nb]: the
// scores as a tiled matrix-core product of the pooled q and k (scores_kernel), then the
// selection, one row per wave up to 16 column groups and one row per pair of waves beyond.
// Without the score accumulators and staged k columns of the fused kernel, the selection
// keeps four waves per SIMD resident to hide the latency of its reductions, LDS histograms
// and ballots.
template <int D, int CPT>
static hipError_t launch_rows_split_t(const float *qa, const float *ka, int BH, int nb,
                                      const uint8_t *sta, float sqrt_d, int64_t cut,
                                      int32_t *kv_nb, int32_t *kv_inds, hipStream_t stream,
                                      float *sbuf) {
    const int nt = (nb + 63) / 64;
    if ((int64_t)nt * nt * BH > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((scores_kernel<D>), dim3(nt * nt * BH), dim3(256), 0, stream, qa, ka, nb,
                       sqrt_d, sbuf);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (CPT <= 16) {
        hipLaunchKernelGGL((select_rows_w4_kernel<D, CPT>), dim3((nb + 3) / 4, BH), dim3(256), 0,
                           stream, qa, ka, nb, sta, sqrt_d, cut, kv_nb, kv_inds, nullptr, 0, 0,
                           NatGrid{}, sbuf);
        return hipGetLastError();
    } else {
        // two waves per row, CPT / 2 column groups each
        hipLaunchKernelGGL((select_pair_kernel<CPT / 2, 2>), dim3(nb, BH), dim3(128), 0, stream,
                           nb, sta, cut, kv_nb, kv_inds, sbuf);
        return hipGetLastError();
    }
}

// top-k variant: rows of up to 2048 blocks (the caller checks)
template <int D>
static hipError_t launch_select_topk_d(const float *qa, const float *ka, int BH, int nb,
                                       const uint8_t *sta, int64_t cut, int32_t *kv_nb,
                                       int32_t *kv_inds, hipStream_t stream) {
#define NABLA_ROWS(CPT, RW) \
    return launch_rows_t<D, CPT, RW, true>(qa, ka, BH, nb, sta, 1.0f, cut, kv_nb, kv_inds, stream)
    if (nb <= 64) NABLA_ROWS(1, 8);
    if (nb <= 128) NABLA_ROWS(2, 8);
    if (nb <= 256) NABLA_ROWS(4, 8);
    if (nb <= 512) NABLA_ROWS(8, 8);
    if (nb <= 1024) NABLA_ROWS(16, 4);
    NABLA_ROWS(32, 2);
#undef NABLA_ROWS
}

// smooth-k for the top-k variant: for every (bh, d) the mean over the nb pooled k blocks
// (fp32, sequential in j, then an IEEE division by nb) is subtracted from those blocks.
// ka is the pooled [bh][D/4][nb] float4 layout.  grid = (B*heads, D/32), 256 threads: a
// workgroup owns 32 dims (8 float4 columns, one contiguous region); it stages 256 blocks
// at a time in LDS with coalesced loads, threads t < 32 add them in order, then all
// threads subtract over the region.
__global__ __launch_bounds__(256) void smooth_k_kernel(float *__restrict__ ka, int nb, int D) {
    constexpr int DB = 32, JC = 256;
    __shared__ float buf[JC * DB];
    __shared__ float km[DB];
    const int t = threadIdx.x;
    float4 *reg = reinterpret_cast<float4 *>(ka) + ((int64_t)blockIdx.x * (D / 4) +
                                                     blockIdx.y * (DB / 4)) * nb;
    float sum = 0.0f;
    for (int j0 = 0; j0 < nb; j0 += JC) {
        const int n = nb - j0 < JC ? nb - j0 : JC;
        for (int e = t; e < (DB / 4) * n; e += 256) {
            const int c = e / n, jj = e - c * n;  // column c (4 dims), block j0 + jj
            const float4 x = reg[(int64_t)c * nb + j0 + jj];
            float *b = &buf[jj * DB + 4 * c];
            b[0] = x.x;
            b[1] = x.y;
            b[2] = x.z;
            b[3] = x.w;
        }
        __syncthreads();
        if (t < DB)
            for (int jj = 0; jj < n; ++jj) sum = sum + buf[jj * DB + t];
        __syncthreads();
    }
    if (t < DB) km[t] = sum / (float)nb;
    __syncthreads();
    float *r = reinterpret_cast<float *>(reg);
    const int64_t len = (int64_t)DB * nb;  // floats: ((c * nb) + j) * 4 + k, dim 4c + k
    for (int64_t e = t; e < len; e += 256) r[e] = r[e] - km[(int)(e / (4 * (int64_t)nb)) * 4 + (int)(e & 3)];
}

// Rows per wave of the selection for rows of nb blocks (as launch_select_d chooses), and
// whether that configuration can pool q itself (16-byte chunks per lane and row).
static int select_rows_per_wave(int nb) { return nb <= 512 ? 8 : 4; }
static bool select_pools_q(int D, int nb) {
    return nb <= 2048 && (D * select_rows_per_wave(nb) / 64) % 8 == 0;
}

template <int D>
static hipError_t launch_select_d(const float *qa, const float *ka, int BH, int nb,
                                  const uint8_t *sta, float sqrt_d, int64_t cut, int32_t *kv_nb,
                                  int32_t *kv_inds, hipStream_t stream, QSource qsrc,
                                  float *sbuf) {
#define NABLA_ROWS(CPT, RW)                                                                   \
    return sbuf != nullptr                                                                    \
               ? launch_rows_split_t<D, CPT>(qa, ka, BH, nb, sta, sqrt_d, cut, kv_nb, kv_inds, \
                                             stream, sbuf)                                    \
               : launch_rows_t<D, CPT, RW>(qa, ka, BH, nb, sta, sqrt_d, cut, kv_nb, kv_inds, \
                                           stream, qsrc)
    if (nb <= 64) NABLA_ROWS(1, 8);
    if (nb <= 128) NABLA_ROWS(2, 8);
    if (nb <= 256) NABLA_ROWS(4, 8);
    if (nb <= 512) NABLA_ROWS(8, 8);
    // 15 and 30 column groups for rows of 897-960 and 1857-1920 blocks (the 720p and the
    // long-clip shapes): the next power of two would score one or two groups holding no block
    if (nb > 896 && nb <= 960) NABLA_ROWS(15, 4);
    if (nb <= 1024) NABLA_ROWS(16, 4);
    if (nb > 1856 && nb <= 1920) NABLA_ROWS(30, 4);
    if (nb <= 2048) NABLA_ROWS(32, 4);
#undef NABLA_ROWS
    return launch_select_t<D, 8, 8>(qa, ka, BH, nb, sta, sqrt_d, cut, kv_nb, kv_inds, stream);
}

// The pooling pass (grid (nb, B)); H > 0 selects the instance with per-row padding checks,
// krow the row-major k means.
static void launch_pool(const void *q, const void *k, bool bf16_in, int B, int S, int heads,
                        int D, int H, int W, NatGrid ng, int first, bool krow, float *qa,
                        float *ka, hipStream_t stream) {
    const dim3 grid(S / kBlock, B);
#define NABLA_POOL(T, PAD, KR)                                                                  \
    hipLaunchKernelGGL((pool_kernel<T, PAD, KR>), grid, dim3(256), 0, stream, (const T *)q,    \
                       (const T *)k, qa, ka, S, heads, D, H, W, ng, first)
#define NABLA_POOL_K(T, PAD)             \
    if (krow) NABLA_POOL(T, PAD, true);  \
    else NABLA_POOL(T, PAD, false)
    if (bf16_in) {
        if (H > 0) { NABLA_POOL_K(bf16, true); }
        else { NABLA_POOL_K(bf16, false); }
    } else {
        if (H > 0) { NABLA_POOL_K(float, true); }
        else { NABLA_POOL_K(float, false); }
    }
#undef NABLA_POOL_K
#undef NABLA_POOL
}

hipError_t launch_block_mask_topk(const void *q, const void *k, bool bf16_in, int B, int S,
                                  int heads, int D, int H, int W, bool natural,
                                  const uint8_t *sta, int topk,
                                  int32_t *kv_nb, int32_t *kv_inds, float *qa, float *ka,
                                  hipStream_t stream) {
    const int nb = S / kBlock;
    launch_pool(q, k, bf16_in, B, S, heads, D, natural ? 0 : H, natural ? 0 : W,
                nat_grid(natural ? W : 0), 0, false, qa, ka, stream);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int BH = B * heads;
    hipLaunchKernelGGL(smooth_k_kernel, dim3(BH, D / 32), dim3(256), 0, stream, ka, nb, D);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    // unit masses: the keys at ascending rank >= nb - k + 1 are the k largest
    const int64_t cut = (int64_t)nb - topk + 1;
    if (D == 64)
        return launch_select_topk_d<64>(qa, ka, BH, nb, sta, cut, kv_nb, kv_inds, stream);
    return launch_select_topk_d<128>(qa, ka, BH, nb, sta, cut, kv_nb, kv_inds, stream);
}

hipError_t launch_block_mask(const void *q, const void *k, bool bf16_in, int B, int S,
                             int heads, int D, int H, int W, bool natural, const uint8_t *sta,
                             int64_t cut_fixed, float sqrt_d, int32_t *kv_nb, int32_t *kv_inds,
                             float *qa, float *ka, float *sbuf, hipStream_t stream) {
    const int nb = S / kBlock;
    // bf16 whole blocks: the selection kernel pools q itself, the pooling pass only k
    const bool padded = !natural && H > 0;
    // rows of 513-2048 blocks with a score buffer: the scores are a tiled product of the pooled
    // q and k (both pooled here); other rows pool q inside the selection kernel where it can
    const bool split = sbuf != nullptr && mask_scores_split(nb);
    const bool qfused = !split && bf16_in && !padded && select_pools_q(D, nb);
    const NatGrid ng = nat_grid(natural ? W : 0);
    launch_pool(q, k, bf16_in, B, S, heads, D, natural ? 0 : H, natural ? 0 : W, ng,
                qfused ? 1 : 0, split, qa, ka, stream);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int BH = B * heads;
    QSource qsrc = {};
    if (qfused) qsrc = QSource{(const bf16 *)q, S, heads, ng};
    if (!split) sbuf = nullptr;
    if (D == 64)
        return launch_select_d<64>(qa, ka, BH, nb, sta, sqrt_d, cut_fixed, kv_nb, kv_inds, stream,
                                   qsrc, sbuf);
    return launch_select_d<128>(qa, ka, BH, nb, sta, sqrt_d, cut_fixed, kv_nb, kv_inds, stream,
                                qsrc, sbuf);
}

}  // namespace nabla
