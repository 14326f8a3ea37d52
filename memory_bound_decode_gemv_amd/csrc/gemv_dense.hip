// gemv_dense.hip -- batch-1 GEMV y = W x over binary16 or bfloat16 weights.
//
// batch1-cdna README, "FP16 GEMV" section: each wavefront computes one output
// element as the dot product of x with one row of W; lanes stride across the
// row so that one load instruction of the wave touches one contiguous span;
// products accumulate in fp32 (v_dot2_f32_f16) and the lanes' partial sums are
// reduced with a DPP row_shr / row_bcast chain.  The page's three versions
// (one accumulator; four accumulators with the loads issued as a batch; 16
// bytes per lane) are all here: the last is the default, the first two are
// kept as the ablation variants.
//
// gfx950 specifics: wave64; 16-byte non-temporal loads (the weights are read
// once, so installing them in the last-level cache only evicts other lines);
// U independent loads and accumulators per lane so that all of a row's loads
// are in flight before the first wait.
#include "dg_device.h"
#include "dg_internal.h"

namespace dg {
namespace {

template <bool BF16>
__device__ __forceinline__ float dot8(u32x4 w, u32x4 x, float acc) {
    if constexpr (BF16) return dot8_bf16(w, x, acc);
    else return dot8_f16(w, x, acc);
}

template <bool BF16>
__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float acc) {
    if constexpr (BF16) return dot2_bf16(w, x, acc);
    else return dot2_f16(w, x, acc);
}

template <bool BF16>
__device__ __forceinline__ void store_out(void* y, int row, float s) {
    if constexpr (BF16) reinterpret_cast<float*>(y)[row] = s;
    else reinterpret_cast<_Float16*>(y)[row] = (_Float16)s;  // round to nearest even
}

// Wave-uniform wave index inside the workgroup.
__device__ __forceinline__ int wave_in_block() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
}

// 16 bytes (8 elements) per lane; U loads in flight per lane per step.
// XREG: the lane's share of x (at most U vectors) is loaded once and kept in
// registers for every row the wave handles; requires K/8 <= 64*U.
// KS (split K): KS waves of a workgroup share one row, wave j taking the
// steps j, j+KS, j+2KS, ... of 64*U vectors; their partial sums meet in LDS
// and are added in the fixed order 0..KS-1 (deterministic).  This multiplies
// the waves, and so the bytes in flight, of shapes with few rows.  The row loop
// runs the same number of times in every wave of a workgroup, so that every
// wave reaches every barrier.
template <bool BF16, int U, bool XREG, int KS>
__global__ void __launch_bounds__(1024)
k_gemv_wide(const uint16_t* __restrict__ W, const uint16_t* __restrict__ x,
            void* __restrict__ y, int N, int K, int64_t ldw) {
    static_assert(!XREG || KS == 1, "x in registers needs whole rows per wave");
    const int lane = lane_id();
    const int wave = wave_in_block();
    const int wpb = blockDim.x / kWave;
    const int rows_per_block = wpb / KS;
    const int kpart = wave % KS;
    const int rslot = wave / KS;
    const int nvec = K >> 3;
    const u32x4* __restrict__ xv = reinterpret_cast<const u32x4*>(x);
    const u32x4 zero = {0u, 0u, 0u, 0u};
    __shared__ float part[KS > 1 ? 1024 / kWave : 1];

    u32x4 xr[XREG ? U : 1];
    if constexpr (XREG) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = u * kWave + lane;
            xr[u] = (idx < nvec) ? xv[idx] : zero;
        }
    }

    for (int row0 = blockIdx.x * rows_per_block; row0 < N; row0 += gridDim.x * rows_per_block) {
        const int row = row0 + rslot;
        float s = 0.0f;
        if (row < N) {   // wave-uniform
            const u32x4* __restrict__ wr = reinterpret_cast<const u32x4*>(W + (int64_t)row * ldw);
            float acc[U];
#pragma unroll
            for (int u = 0; u < U; ++u) acc[u] = 0.0f;

            if constexpr (XREG) {
                if (nvec > 0) {
                    u32x4 wv[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int idx = u * kWave + lane;
                        wv[u] = load_vec<true>(wr + (idx < nvec ? idx : nvec - 1));
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int idx = u * kWave + lane;
                        acc[u] = dot8<BF16>(idx < nvec ? wv[u] : zero, xr[u], acc[u]);
                    }
                }
            } else {
                int v0 = kpart * kWave * U;
                for (; v0 + kWave * U <= nvec; v0 += KS * kWave * U) {
                    u32x4 wv[U], xw[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) wv[u] = load_vec<true>(wr + v0 + u * kWave + lane);
#pragma unroll
                    for (int u = 0; u < U; ++u) xw[u] = xv[v0 + u * kWave + lane];
#pragma unroll
                    for (int u = 0; u < U; ++u) acc[u] = dot8<BF16>(wv[u], xw[u], acc[u]);
                }
                if (v0 < nvec) {  // ragged last step: out-of-range lanes read a valid vector, then zero it
                    u32x4 wv[U], xw[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int idx = v0 + u * kWave + lane;
                        const int idc = idx < nvec ? idx : nvec - 1;
                        wv[u] = load_vec<true>(wr + idc);
                        xw[u] = xv[idc];
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const bool ok = v0 + u * kWave + lane < nvec;
                        acc[u] = dot8<BF16>(ok ? wv[u] : zero, ok ? xw[u] : zero, acc[u]);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) s += acc[u];
            s = wave_sum_f32(s);
        }
        if constexpr (KS == 1) {
            if (row < N && lane == 0) store_out<BF16>(y, row, s);
        } else {
            if (lane == 0) part[wave] = s;
            __syncthreads();
            if (kpart == 0 && row < N && lane == 0) {
                float t = part[wave];
#pragma unroll
                for (int j = 1; j < KS; ++j) t += part[wave + j];
                store_out<BF16>(y, row, t);
            }
            __syncthreads();
        }
    }
}

// Ablation variants with 4 bytes (one half2 / bf16x2 pair) per lane.
// NACC = 1: one accumulator, each iteration's load consumed immediately.
// NACC = 4: four independent accumulators, four loads issued as a batch.
template <bool BF16, int NACC>
__global__ void __launch_bounds__(1024)
k_gemv_narrow(const uint16_t* __restrict__ W, const uint16_t* __restrict__ x,
              void* __restrict__ y, int N, int K, int64_t ldw) {
    const int lane = lane_id();
    const int wpb = blockDim.x / kWave;
    const int n2 = K >> 1;
    const uint32_t* __restrict__ x2 = reinterpret_cast<const uint32_t*>(x);
    for (int row = blockIdx.x * wpb + wave_in_block(); row < N; row += gridDim.x * wpb) {
        const uint32_t* __restrict__ w2 = reinterpret_cast<const uint32_t*>(W + (int64_t)row * ldw);
        float acc[NACC];
#pragma unroll
        for (int a = 0; a < NACC; ++a) acc[a] = 0.0f;
        int k = lane;
        for (; k + (NACC - 1) * kWave < n2; k += NACC * kWave) {
            uint32_t wv[NACC], xw[NACC];
#pragma unroll
            for (int a = 0; a < NACC; ++a) wv[a] = load_u32<true>(w2 + k + a * kWave);
#pragma unroll
            for (int a = 0; a < NACC; ++a) xw[a] = x2[k + a * kWave];
#pragma unroll
            for (int a = 0; a < NACC; ++a) acc[a] = dot2<BF16>(wv[a], xw[a], acc[a]);
        }
        for (; k < n2; k += kWave) acc[0] = dot2<BF16>(load_u32<true>(w2 + k), x2[k], acc[0]);
        float s = 0.0f;
#pragma unroll
        for (int a = 0; a < NACC; ++a) s += acc[a];
        s = wave_sum_f32(s);
        if (lane == 0) store_out<BF16>(y, row, s);
    }
}

template <bool BF16, int KS>
hipError_t launch_wide_ks(int U, bool xreg, const uint16_t* w16, const uint16_t* x16, void* y, int N, int K,
                          int64_t ldw, int grid, int block, hipStream_t s) {
#define DG_WIDE_CASE(UU)                                                                         \
    case UU:                                                                                     \
        if (xreg) {                                                                              \
            if constexpr (KS == 1)                                                               \
                hipLaunchKernelGGL((k_gemv_wide<BF16, UU, true, 1>), dim3(grid), dim3(block), 0, \
                                   s, w16, x16, y, N, K, ldw);                                   \
            else                                                                                 \
                return hipErrorInvalidValue;                                                     \
        } else {                                                                                 \
            hipLaunchKernelGGL((k_gemv_wide<BF16, UU, false, KS>), dim3(grid), dim3(block), 0,   \
                               s, w16, x16, y, N, K, ldw);                                       \
        }                                                                                        \
        break;
    switch (U) {
        DG_WIDE_CASE(1)
        DG_WIDE_CASE(2)
        DG_WIDE_CASE(4)
        DG_WIDE_CASE(8)
        default:
            return hipErrorInvalidValue;
    }
#undef DG_WIDE_CASE
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_wide(int U, int KS, bool xreg, const void* W, const void* x, void* y, int N, int K,
                       int64_t ldw, int grid, int block, hipStream_t s) {
    const uint16_t* w16 = (const uint16_t*)W;
    const uint16_t* x16 = (const uint16_t*)x;
    switch (KS) {
        case 1: return launch_wide_ks<BF16, 1>(U, xreg, w16, x16, y, N, K, ldw, grid, block, s);
        case 2: return launch_wide_ks<BF16, 2>(U, xreg, w16, x16, y, N, K, ldw, grid, block, s);
        case 4: return launch_wide_ks<BF16, 4>(U, xreg, w16, x16, y, N, K, ldw, grid, block, s);
        default: return hipErrorInvalidValue;
    }
}

int round_up_pow2_unroll(int v) {
    int u = 1;
    while (u < v && u < 16) u *= 2;
    return u;
}

}  // namespace

hipError_t launch_gemv_dense(bool bf16, const void* W, const void* x, void* y,
                             int N, int K, int64_t ldw, const dg_launch* cfg, hipStream_t s) {
    const int nvec = K / 8;
    const int variant = cfg && cfg->variant ? cfg->variant : DG_VARIANT_DENSE_WIDE;
    const int block = cfg && cfg->block ? cfg->block : 256;
    const int wpb = block / kWave;

    if (variant == DG_VARIANT_DENSE_WIDE || variant == DG_VARIANT_DENSE_XREG) {
        const bool xreg = variant == DG_VARIANT_DENSE_XREG;
        int U = 8, KS = 1;
        if (xreg) {
            U = round_up_pow2_unroll((nvec + kWave - 1) / kWave);
            if (cfg && cfg->unroll) U = cfg->unroll;
            if (U * kWave < nvec || U > 8) return hipErrorInvalidValue;
        } else if (cfg && cfg->unroll) {
            // explicit: unroll = U + 100 * (KS - 1) lets a sweep pick both
            U = cfg->unroll % 100;
            KS = cfg->unroll / 100 + 1;
        } else {
            // Measured on MI355X over the decoder shapes and the lm-head: two
            // 16-byte loads per lane per step with each row's K split over two
            // waves (four below 2048 rows) keep the most bytes in flight, since
            // the small register footprint lets more waves stay resident.
            U = 2;
            if (wpb >= 2 && nvec >= 2 * kWave * U) KS = 2;
            if (wpb >= 4 && N < 2048 && nvec >= 4 * kWave * U) KS = 4;
        }
        if (wpb % KS != 0) return hipErrorInvalidValue;
        const int rows_per_block = wpb / KS;
        const int grid = cfg && cfg->grid ? cfg->grid : (N + rows_per_block - 1) / rows_per_block;
        return bf16 ? launch_wide<true>(U, KS, xreg, W, x, y, N, K, ldw, grid, block, s)
                    : launch_wide<false>(U, KS, xreg, W, x, y, N, K, ldw, grid, block, s);
    }
    const int grid = cfg && cfg->grid ? cfg->grid : (N + wpb - 1) / wpb;
    if (variant == DG_VARIANT_DENSE_NARROW1 || variant == DG_VARIANT_DENSE_NARROW4) {
        const uint16_t* w16 = (const uint16_t*)W;
        const uint16_t* x16 = (const uint16_t*)x;
        if (variant == DG_VARIANT_DENSE_NARROW1) {
            if (bf16) hipLaunchKernelGGL((k_gemv_narrow<true, 1>), dim3(grid), dim3(block), 0, s, w16, x16, y, N, K, ldw);
            else hipLaunchKernelGGL((k_gemv_narrow<false, 1>), dim3(grid), dim3(block), 0, s, w16, x16, y, N, K, ldw);
        } else {
            if (bf16) hipLaunchKernelGGL((k_gemv_narrow<true, 4>), dim3(grid), dim3(block), 0, s, w16, x16, y, N, K, ldw);
            else hipLaunchKernelGGL((k_gemv_narrow<false, 4>), dim3(grid), dim3(block), 0, s, w16, x16, y, N, K, ldw);
        }
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

}  // namespace dg
