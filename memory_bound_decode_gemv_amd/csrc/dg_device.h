// dg_device.h -- device-side building blocks shared by the libdecodegemv kernels
// (gfx950, wave64).  Nothing here is host code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

// Native compiler vector types: __builtin_nontemporal_load accepts these, not
// HIP's wrapper classes (batch1-cdna README, streaming-read notes on the
// generated assembly).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// Same vectors with only 4-byte alignment promised: global_load_dwordx4 needs
// dword alignment, which is all a packed 36-byte Q4_0 block pair offers.
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// 16-byte load per lane; NT selects the non-temporal hint.
template <bool NT, typename V>
__device__ __forceinline__ V load_vec(const V* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool NT>
__device__ __forceinline__ uint32_t load_u32(const uint32_t* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// ---------------------------------------------------------------------------
// Cross-lane reductions with DPP (row_shr inside each 16-lane row, then
// row_bcast:15 / row_bcast:31 across rows).  The order of additions is fixed,
// so float sums are bit-reproducible.  The full result ends in lane 63 and is
// returned to every lane through readlane.
// ---------------------------------------------------------------------------
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_mov_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, true));
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_mov_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, true);
}

__device__ __forceinline__ float wave_sum_f32(float v) {
    v += dpp_mov_f32<kDppRowShr1, 0xF>(v);
    v += dpp_mov_f32<kDppRowShr2, 0xF>(v);
    v += dpp_mov_f32<kDppRowShr4, 0xF>(v);
    v += dpp_mov_f32<kDppRowShr8, 0xF>(v);
    v += dpp_mov_f32<kDppRowBcast15, 0xA>(v);
    v += dpp_mov_f32<kDppRowBcast31, 0xC>(v);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
    v += dpp_mov_u32<kDppRowShr1, 0xF>(v);
    v += dpp_mov_u32<kDppRowShr2, 0xF>(v);
    v += dpp_mov_u32<kDppRowShr4, 0xF>(v);
    v += dpp_mov_u32<kDppRowShr8, 0xF>(v);
    v += dpp_mov_u32<kDppRowBcast15, 0xA>(v);
    v += dpp_mov_u32<kDppRowBcast31, 0xC>(v);
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// ---------------------------------------------------------------------------
// Packed dot products
// ---------------------------------------------------------------------------

// One packed pair per dword.  The dword is taken by value: __builtin_bit_cast
// applied directly to a vector-element lvalue such as w.y reads element 0
// (seen in the generated gfx950 code), so vector components must reach the
// cast as plain values.
__device__ __forceinline__ float dot2_f16(uint32_t w, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), __builtin_bit_cast(f16x2, x), acc, false);
}

__device__ __forceinline__ float dot2_bf16(uint32_t w, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, x), acc, false);
}

// Four half2 pairs of one 16-byte vector: acc + sum of 8 products (v_dot2_f32_f16).
__device__ __forceinline__ float dot8_f16(u32x4 w, u32x4 x, float acc) {
    acc = dot2_f16(w.x, x.x, acc);
    acc = dot2_f16(w.y, x.y, acc);
    acc = dot2_f16(w.z, x.z, acc);
    acc = dot2_f16(w.w, x.w, acc);
    return acc;
}

// Same for bfloat16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot8_bf16(u32x4 w, u32x4 x, float acc) {
    acc = dot2_bf16(w.x, x.x, acc);
    acc = dot2_bf16(w.y, x.y, acc);
    acc = dot2_bf16(w.z, x.z, acc);
    acc = dot2_bf16(w.w, x.w, acc);
    return acc;
}

// Signed 4 x int8 dot product into an int32 accumulator (v_dot4_i32_i8).
__device__ __forceinline__ int dot4_i8(uint32_t a, uint32_t b, int acc) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, acc, false);
}

// Binds an fp32 value to a VGPR so that the operation producing it cannot be
// fused into its consumer (the "bind values, not memory" countermeasure of
// "The kernel that waited for itself", Finding 3).  Without it the compiler
// turns binary16(a * b) into v_fma_mixlo_f16, which rounds the exact product
// once to binary16 instead of first to fp32.
__device__ __forceinline__ float bind_f32(float v) {
    asm volatile("" : "+v"(v));
    return v;
}

// Low 16 bits of a dword as binary16 -> fp32.
__device__ __forceinline__ float half_lo_to_f32(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float half_hi_to_f32(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

}  // namespace dg
