// attn_tile.h -- device helpers shared by the attention kernels (forward and backward):
// the 32x32 MFMA tile layout, LDS chunk swizzles and direct global -> LDS tile loads.
#pragma once

#include "nabla_device.h"

namespace nabla {

typedef float f32x16 __attribute__((ext_vector_type(16)));
#define NABLA_LDS __attribute__((address_space(3)))

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

// Byte offset of a __shared__ object in LDS.
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
    return (uint32_t)(uintptr_t)((const NABLA_LDS char *)p);
}

// 16 bytes per lane from global memory straight into LDS: lane l's chunk lands at
// m0 + 16 l (m0 wave-uniform).  Issued from inline asm so that the compiler does not
// treat every later LDS read as depending on it; completion is awaited explicitly
// with vm_wait before the barrier that hands the tile to the other waves.  Nothing
// else in the kernel uses m0.
// The base address is wave-uniform (SGPR pair) and each lane gives a 32-bit byte offset:
// no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void lds_direct16_sv(const void *base, uint32_t off, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(m0)
                 : "memory");
}
template <int N>
__device__ __forceinline__ void vm_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

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
