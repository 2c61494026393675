// attn_tile.h -- device helpers shared by the attention kernels (forward and backward):
// the 32x32 MFMA tile layout, LDS chunk swizzles and direct global -> LDS tile loads.
#pragma once

#include "nabla_device.h"

namespace nabla {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Key row (within a 32-row score tile) fed to MFMA row m: bit layout
// m = a(2) hh(1) b(2)  ->  key = (a>>1)<<4 | hh<<3 | (a&1)<<2 | b.
__device__ __forceinline__ int sigma32(int m) {
    const int a = m >> 3, hh = (m >> 2) & 1, b = m & 3;
    return ((a >> 1) << 4) | (hh << 3) | ((a & 1) << 2) | b;
}

__device__ __forceinline__ f32x16 splat16(float x) {
    f32x16 r;
#pragma unroll
    for (int j = 0; j < 16; ++j) r[j] = x;
    return r;
}

// 16-byte chunk swizzles (CH chunks per row) of the K and V tiles in LDS.
template <int CH>
__device__ __forceinline__ int kswz(int kv) { return kv & (CH - 1); }
template <int CH>
__device__ __forceinline__ int vswz(int kv) { return (kv & 3) * (CH / 4); }

// Query blocks per attention workgroup: kGroup 4 takes a 2 (time) x 1 x 2 (width) box of
// tiles, kGroup 2 the same tile in two consecutive frames.
#ifndef NABLA_ATTN_GROUP
#define NABLA_ATTN_GROUP 4
#endif
constexpr int kGroup = NABLA_ATTN_GROUP;
constexpr int kAttnWaves = 2 * kGroup;
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr int kMaxWords = 4096 / 64;  // bitmap words for up to 4096 blocks per row
static_assert(kGroup == 2 || kGroup == 4, "group of 2 or 4 query blocks");
static_assert(kAttnWaves == 8 || kGroup != 4, "the delayed half of the waves is waves 4-7");

// Member s of query-block group gi (-1 = empty slot).  Known tile grid: kGroup 4 takes
// a 2 (time) x 1 x 2 (width) box of tiles, kGroup 2 the same tile in two consecutive
// frames; unknown grid (Tt == 0): kGroup consecutive blocks.
__device__ __forceinline__ int group_member(int gi, int s, int Tt, int Ht, int Wt, int nb) {
    if (Tt > 0) {
        const int cw = kGroup == 4 ? (Wt + 1) >> 1 : Wt;
        const int a = gi / (Ht * cw), hh = (gi / cw) % Ht, c = gi % cw;
        const int t = 2 * a + (kGroup == 4 ? (s >> 1) : s);
        const int ww = kGroup == 4 ? 2 * c + (s & 1) : c;
        return (t < Tt && ww < Wt) ? (t * Ht + hh) * Wt + ww : -1;
    }
    const int i = gi * kGroup + s;
    return i < nb ? i : -1;
}


// A list length / block index from kv lists, clamped into range (bad lists cannot
// address memory outside the tensors).
__device__ __forceinline__ int clamp_count(int n, int nb) { return n < 0 ? 0 : (n > nb ? nb : n); }
__device__ __forceinline__ int clamp_block(int j, int nb) { return j < 0 ? 0 : (j >= nb ? nb - 1 : j); }

}  // namespace nabla
