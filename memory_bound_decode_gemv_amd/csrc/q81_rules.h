// q81_rules.h -- the Q8_1 activation rules as device helpers, shared by the
// standalone quantiser and the quantising prologue of the fused M = 1 GEMV,
// so that both produce the same bytes.  Device code only.
//
// Per 32-activation block (the Q8_1 format of the Q4_0/Q8_1 harness in "The
// kernel that waited for itself"): a = max|x|; d = a / 127 in binary32,
// correctly rounded; code q = x / d correctly rounded to binary32, then
// rounded half away from zero and clamped to [-127, 127] (d = 0 gives q = 0);
// stored d = binary16(d), stored s = binary16(binary32(d * sum q)).  Every
// binary32 result that feeds a rounding to binary16 is bound to a register
// (bind_f32), so no contraction of a product into a conversion can happen.
#pragma once

#include "dg_device.h"

namespace dg {

__device__ __forceinline__ uint16_t q81_half_bits(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);   // v_cvt_f16_f32: round to nearest even
}

// d from the block's largest magnitude.
__device__ __forceinline__ float q81_scale(float amax) {
#pragma clang fp contract(off)
    return bind_f32(amax / 127.0f);
}

// The code of one activation.
__device__ __forceinline__ int q81_code(float x, float d) {
#pragma clang fp contract(off)
    if (d == 0.0f) return 0;
    int c = (int)roundf(x / d);   // halves away from zero
    return c > 127 ? 127 : (c < -127 ? -127 : c);
}

// The block's first dword: binary16 d in the low half, binary16 s above.
__device__ __forceinline__ uint32_t q81_header(float d, int sum) {
#pragma clang fp contract(off)
    return (uint32_t)q81_half_bits(d) | ((uint32_t)q81_half_bits(bind_f32(d * (float)sum)) << 16);
}

// One whole block by one lane: 32 activations (16-byte aligned) -> the 9
// dwords of the Q8_1 block (header, then codes 4i..4i+3 in dword 1 + i).
__device__ __forceinline__ void quantize_q81_block(const float* __restrict__ src, uint32_t out[9]) {
    float v[32];
    const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 f = s4[i];
        v[4 * i + 0] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
    const float d = q81_scale(amax);
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t w = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int c = q81_code(v[4 * i + b], d);
            sum += c;
            w |= (uint32_t)(uint8_t)(int8_t)c << (8 * b);
        }
        out[1 + i] = w;
    }
    out[0] = q81_header(d, sum);
}

}  // namespace dg
