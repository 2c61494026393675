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

}  // namespace nabla
