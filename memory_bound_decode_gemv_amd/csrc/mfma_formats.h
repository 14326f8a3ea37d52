// mfma_formats.h -- weight formats of the int8 matrix-core kernels: how one
// block pair of Q4_0 or Q8_0 weights, as it sits in LDS, becomes the B
// operands of two v_mfma_i32_16x16x32_i8 (one per block) and the two blocks'
// fp32 scales.  Device code only.
#pragma once

#include "q4_common.h"

namespace dg {
namespace mfma {

using namespace q4;

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr long kNeg8 = (long)0xF8F8F8F8F8F8F8F8ull;   // eight int8 k-slots of -8

// Weight formats.  decode(w, g, bop, d): from the dwords w of one block pair
// in LDS, the B operands (k-slots 4g..4g+3 and 16+4g..16+4g+3, as int8) and
// the fp32 scales of the pair's two blocks; scale_bits(w, width, h): the two
// scales' binary16 bits in the low half of h[0], h[1] (width 16), or zeros
// (width 0).
struct FmtQ4_0 {   // 18-byte blocks: binary16 d, 16 bytes of nibbles; weight = (q - 8) d
    static constexpr int kBlockBytes = 18;
    static constexpr bool kOffset = true;   // codes 0..15 stand for q - 8
    __device__ __forceinline__ static void decode(const uint32_t* w, int g, long bop[2], float d[2]) {
        const uint32_t c0 = __builtin_amdgcn_alignbit(w[g + 1], w[g], 16);   // codes at bytes 2..17
        const uint32_t c1 = w[5 + g];                                         // codes at bytes 20..35
        bop[0] = (long)((uint64_t)(c0 & kNib) | ((uint64_t)((c0 >> 4) & kNib) << 32));
        bop[1] = (long)((uint64_t)(c1 & kNib) | ((uint64_t)((c1 >> 4) & kNib) << 32));
        d[0] = half_lo_to_f32(w[0]);
        d[1] = half_hi_to_f32(w[4]);
    }
    __device__ __forceinline__ static void scale_bits(const uint32_t* w, uint32_t width, uint32_t h[2]) {
        h[0] = __builtin_amdgcn_ubfe(w[0], 0, width);
        h[1] = __builtin_amdgcn_ubfe(w[4], 16, width);
    }
};
struct FmtQ8_0 {   // 34-byte blocks: binary16 d, 32 int8 codes; weight = q d
    static constexpr int kBlockBytes = 34;
    static constexpr bool kOffset = false;
    __device__ __forceinline__ static void decode(const uint32_t* w, int g, long bop[2], float d[2]) {
        // block a: codes at bytes 2..33, so code dword i straddles dwords i and i + 1
        const uint32_t a0 = __builtin_amdgcn_alignbit(w[g + 1], w[g], 16);
        const uint32_t a1 = __builtin_amdgcn_alignbit(w[g + 5], w[g + 4], 16);
        bop[0] = (long)((uint64_t)a0 | ((uint64_t)a1 << 32));
        // block b: scale in bytes 34-35 (high half of dword 8), codes in dwords 9..16
        bop[1] = (long)((uint64_t)w[9 + g] | ((uint64_t)w[13 + g] << 32));
        d[0] = half_lo_to_f32(w[0]);
        d[1] = half_hi_to_f32(w[8]);
    }
    __device__ __forceinline__ static void scale_bits(const uint32_t* w, uint32_t width, uint32_t h[2]) {
        h[0] = __builtin_amdgcn_ubfe(w[0], 0, width);
        h[1] = __builtin_amdgcn_ubfe(w[8], 16, width);
    }
};

// The 16 x 16 products d8[c] * d4[n] of one block in the layout of an MFMA
// result (lane l: rows 4(l/16) + r, column l % 16), from one
// v_mfma_f32_16x16x16_f16 in which only k-slot 0 carries a nonzero B: every
// lane passes d8 of A-row l % 16 as k-slot 4(l/16) (a8, binary16 bits in the
// low half, zeros above), and lanes of group 0 pass d4 of B-column l % 16
// (h4), the others zero.  A product of two binary16 values is exact in fp32,
// and the other k-slots add finite x 0 = 0.
__device__ __forceinline__ f32x4 scale_outer(uint32_t a8, uint32_t h4) {
    const f16x4 a = __builtin_bit_cast(f16x4, u32x2{a8, 0u});
    const f16x4 b = __builtin_bit_cast(f16x4, u32x2{h4, 0u});
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
}

}  // namespace mfma
}  // namespace dg
