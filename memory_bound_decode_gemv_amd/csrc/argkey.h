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

// The key of another lane, moved by one DPP step: both 32-bit halves take the
// same control, so they come from the same source lane.  Lanes whose source
// is outside the row, and rows the mask leaves out, receive 0 -- the
// identity of the maximum, since every key is >= 0 and an empty lane holds 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_key(uint64_t v) {
    const uint32_t lo = dpp_mov_u32<CTRL, ROW_MASK>((uint32_t)v);
    const uint32_t hi = dpp_mov_u32<CTRL, ROW_MASK>((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Maximum key of the wave on DPP (IEEE discussion "ArgCompare Benchmark
// Results and Performance Analysis": the DPP reduction beat the shuffle-only
// one in every configuration it measured).  row_shr 1, 2, 4, 8 leave each
// 16-lane row's maximum in its lane 15; row_bcast:15 folds row 0 into row 1
// and row 2 into row 3, row_bcast:31 rows 0-1 into rows 2-3, so lane 63
// holds the wave's maximum, returned to every lane through readlane.  The
// maximum does not depend on the order of the steps.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = umax64(v, dpp_key<kDppRowShr1, 0xF>(v));
    v = umax64(v, dpp_key<kDppRowShr2, 0xF>(v));
    v = umax64(v, dpp_key<kDppRowShr4, 0xF>(v));
    v = umax64(v, dpp_key<kDppRowShr8, 0xF>(v));
    v = umax64(v, dpp_key<kDppRowBcast15, 0xA>(v));
    v = umax64(v, dpp_key<kDppRowBcast31, 0xC>(v));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

}  // namespace dg
