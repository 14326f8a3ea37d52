// argkey.h -- the 64-bit keys of the argmax reductions (device code only).
//
//   key = (order-preserving 32-bit image of the value) << 32 | (0xFFFFFFFF - index)
//
// so that "larger key" means "larger value, or equal value at a lower index".
// -0 is folded onto +0 (IEEE equality) and every NaN maps to the largest image
// (a NaN beats every number; among NaNs the lowest index wins).  The maximum
// of keys does not depend on the order in which keys are combined.
#pragma once

#include "dg_device.h"

namespace dg {

__device__ __forceinline__ uint32_t order_image(float v) {
    uint32_t u = __builtin_bit_cast(uint32_t, v);
    if (v != v) return 0xFFFFFFFFu;       // NaN above everything
    if (u == 0x80000000u) u = 0u;         // -0 == +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t pack_key(uint32_t img, uint32_t idx) {
    return ((uint64_t)img << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ uint32_t key_index(uint64_t key) { return 0xFFFFFFFFu - (uint32_t)key; }

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, off, kWave);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), off, kWave);
        v = umax64(v, ((uint64_t)hi << 32) | lo);
    }
    return v;
}

}  // namespace dg
