// nabla_device.h -- device-side types and helpers shared by the libnabla kernels.
// gfx950 (CDNA4) only: 64-lane wavefronts, bf16 MFMA, 160 KiB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nabla {

constexpr int kBlock = 64;  // tokens per block (one 1 x 8 x 8 fractal tile)
constexpr int kTile = 8;    // spatial patch edge
constexpr int kWave = 64;

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// Eight consecutive input elements as bf16 (fp32 inputs are rounded to nearest even).
__device__ __forceinline__ bf16x8 load8_bf16(const bf16 *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}
__device__ __forceinline__ bf16x8 load8_bf16(const float *p) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    bf16x8 r;
    r[0] = (bf16)a.x; r[1] = (bf16)a.y; r[2] = (bf16)a.z; r[3] = (bf16)a.w;
    r[4] = (bf16)b.x; r[5] = (bf16)b.y; r[6] = (bf16)b.z; r[7] = (bf16)b.w;
    return r;
}

#define NABLA_LDS __attribute__((address_space(3)))

// Byte offset of a __shared__ object in LDS.
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
    return (uint32_t)(uintptr_t)((const NABLA_LDS char *)p);
}

// 16 bytes per lane from global memory straight into LDS: lane l's chunk lands at
// m0 + 16 l (m0 wave-uniform).  Issued from inline asm so that the compiler does not
// treat every later LDS read as depending on it; completion is awaited explicitly
// with vm_wait before the barrier that hands the tile to the other waves.  The asm
// declares m0 clobbered.
// The base address is wave-uniform (SGPR pair) and each lane gives a 32-bit byte offset:
// no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void lds_direct16_sv(const void *base, uint32_t off, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(m0)
                 : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void vm_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// 64-bit lane shuffles built from two 32-bit ones.
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    lo = __shfl_xor(lo, mask);
    hi = __shfl_xor(hi, mask);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t v, int delta) {
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    lo = __shfl_up(lo, delta);
    hi = __shfl_up(hi, delta);
    return ((uint64_t)hi << 32) | lo;
}

// Workgroup id -> work item such that each of the 8 XCDs (which receive
// workgroups round-robin) gets one contiguous range of work items, so
// neighbouring items share that XCD's L2.
__device__ __forceinline__ int xcd_contiguous(int bid, int n) {
    const int q = n >> 3, r = n & 7;
    const int x = bid & 7, k = bid >> 3;
    return x * q + min(x, r) + k;
}

// Natural-order addressing of a grid of whole 8 x 8 patches (T frames of H = 8 Ht rows and
// W = 8 Wt columns, tokens row-major as (t, y, x)).  Fractal block j = (t Ht + ht) Wt + wt
// starts at natural token (t H + 8 ht) W + 8 wt = 64 p Wt + 8 wt, where p = j / Wt counts
// the patch rows before it over all frames; its row r = 8 y' + x' lies (r >> 3) W + (r & 7)
// tokens further on.  p is a multiply-high by m = floor(2^32 / Wt) + 1, passed as its high
// (0 or 1) and low words: j m / 2^32 exceeds j / Wt by less than j / 2^32, and the fraction
// of j / Wt is at most 1 - 1 / Wt, so the floor is exact while j Wt < 2^32.  The host allows
// at most 4096 blocks per sequence and Wt < 2^20.
struct NatGrid {
    int W, Wt;
    uint32_t mhi, mlo;
};
inline NatGrid nat_grid(int W) {
    NatGrid g;
    g.W = W;
    g.Wt = W / kTile;
    const uint64_t m = (g.Wt > 0 ? (uint64_t)0x100000000ull / (uint64_t)g.Wt : 0) + 1;
    g.mhi = (uint32_t)(m >> 32);
    g.mlo = (uint32_t)m;
    return g;
}
__device__ __forceinline__ int nat_block_base(int j, const NatGrid &g) {
    const uint32_t uj = (uint32_t)j;
    const uint32_t p = uj * g.mhi + __umulhi(uj, g.mlo);
    return (int)(64u * p * (uint32_t)g.Wt + 8u * (uj - p * (uint32_t)g.Wt));
}
__device__ __forceinline__ int nat_row_off(int r, int W) { return (r >> 3) * W + (r & 7); }
// Token index of row r of fractal block j: in the fractal order (g.W == 0), or in the natural
// order of a grid of whole patches (g.W > 0).
__device__ __forceinline__ int64_t block_row_token(int j, int r, const NatGrid &g) {
    return g.W > 0 ? (int64_t)nat_block_base(j, g) + nat_row_off(r, g.W)
                   : (int64_t)j * kBlock + r;
}

}  // namespace nabla
