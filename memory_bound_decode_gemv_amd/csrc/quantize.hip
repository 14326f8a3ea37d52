// quantize.hip -- Q8_1 (activations) and Q4_0 (weights) quantisers.
//
// Formats of the Q4_0/Q8_1 harness in "The kernel that waited for itself":
// 32-element blocks with a binary16 scale.  The activation quantiser is the
// step that runs before every quantised GEMV call (the "Capability Gain"
// paper measures an unfused per-call conversion at 27.9 us and finds it can
// cost more than the matmul itself).  Every decision that turns a float into
// a code is taken in IEEE binary32 with correctly rounded division, no
// contraction, and every value stored as binary16 is first rounded to binary32
// (bind_f32), so the bytes are reproducible on any IEEE machine.
#include "dg_device.h"
#include "dg_internal.h"
#include "q81_rules.h"

#pragma clang fp contract(off)

namespace dg {
namespace {

__device__ __forceinline__ uint16_t f32_to_half_bits(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);   // v_cvt_f16_f32: round to nearest even
}

__device__ __forceinline__ void load_block32(const float* __restrict__ src, float v[32]) {
    const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 f = s4[i];
        v[4 * i + 0] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
}

// One lane per activation: the 32 lanes of each half of a wave hold one block
// (block t of the flattened [M][K] input), so a block's largest magnitude
// and its code sum are reductions over 32 lanes (both exact in any order)
// and every lane takes one division.  A wave writes two whole 36-byte blocks:
// lane j of a half stores code byte j, lane 0 the header dword.
__global__ void __launch_bounds__(256)
k_quantize_q8_1(const float* __restrict__ x, uint8_t* __restrict__ Xq, int64_t nblocks) {
    const int64_t t = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 5;
    const int j = threadIdx.x & 31;
    const bool live = t < nblocks;
    const float v = live ? x[t * 32 + j] : 0.0f;
    float amax = fabsf(v);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 32));
    const float d = q81_scale(amax);
    const int c = q81_code(v, d);
    int sum = c;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 32);
    if (!live) return;
    uint8_t* blk = Xq + t * 36;
    blk[4 + j] = (uint8_t)(int8_t)c;
    if (j == 0) *reinterpret_cast<uint32_t*>(blk) = q81_header(d, sum);
}

// One thread per 32-weight block.
__global__ void __launch_bounds__(256)
k_quantize_q4_0(const float* __restrict__ w, uint8_t* __restrict__ Wq, int64_t nblocks) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= nblocks) return;
    float v[32];
    load_block32(w + t * 32, v);
    float amax = 0.0f, m = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const float a = fabsf(v[j]);
        if (a > amax) { amax = a; m = v[j]; }   // first element of largest magnitude, sign kept
    }
    const float d = bind_f32(m / -8.0f);
    uint8_t q[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        if (d == 0.0f) { q[j] = 8; continue; }
        const int c = (int)floorf(v[j] / d + 8.5f);
        q[j] = (uint8_t)(c > 15 ? 15 : c);
    }
    uint16_t* out = reinterpret_cast<uint16_t*>(Wq + t * 18);
    out[0] = f32_to_half_bits(d);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t b0 = q[2 * i] | (q[2 * i + 16] << 4);
        const uint32_t b1 = q[2 * i + 1] | (q[2 * i + 17] << 4);
        out[1 + i] = (uint16_t)(b0 | (b1 << 8));
    }
}

// One thread per 32-weight block: d = max|x| / 127, codes rounded half away
// from zero (the same rule as the activation quantiser, without the sum).
__global__ void __launch_bounds__(256)
k_quantize_q8_0(const float* __restrict__ w, uint8_t* __restrict__ Wq, int64_t nblocks) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= nblocks) return;
    float v[32];
    load_block32(w + t * 32, v);
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
    const float d = bind_f32(amax / 127.0f);
    uint16_t* out = reinterpret_cast<uint16_t*>(Wq + t * 34);   // blocks are 2-byte aligned
    out[0] = f32_to_half_bits(d);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        uint32_t h = 0;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            int c = 0;
            if (d != 0.0f) {
                c = (int)roundf(v[2 * i + b] / d);   // halves away from zero
                c = c > 127 ? 127 : (c < -127 ? -127 : c);
            }
            h |= (uint32_t)(uint8_t)(int8_t)c << (8 * b);
        }
        out[1 + i] = (uint16_t)h;
    }
}

}  // namespace

hipError_t launch_quantize_q8_0(const float* w, void* Wq, int64_t N, int64_t K, hipStream_t s) {
    const int64_t nblocks = N * (K / 32);
    const int64_t grid = (nblocks + 255) / 256;
    hipLaunchKernelGGL(k_quantize_q8_0, dim3((unsigned)grid), dim3(256), 0, s, w, (uint8_t*)Wq, nblocks);
    return hipGetLastError();
}

hipError_t launch_quantize_q8_1(const float* x, void* Xq, int64_t M, int64_t K, hipStream_t s) {
    const int64_t nblocks = M * (K / 32);
    const int64_t grid = (nblocks + 7) / 8;   // eight blocks of 32 lanes per workgroup
    hipLaunchKernelGGL(k_quantize_q8_1, dim3((unsigned)grid), dim3(256), 0, s, x, (uint8_t*)Xq, nblocks);
    return hipGetLastError();
}

hipError_t launch_quantize_q4_0(const float* w, void* Wq, int64_t N, int64_t K, hipStream_t s) {
    const int64_t nblocks = N * (K / 32);
    const int64_t grid = (nblocks + 255) / 256;
    hipLaunchKernelGGL(k_quantize_q4_0, dim3((unsigned)grid), dim3(256), 0, s, w, (uint8_t*)Wq, nblocks);
    return hipGetLastError();
}

}  // namespace dg
