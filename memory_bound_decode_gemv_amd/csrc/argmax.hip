// argmax.hip -- per-row argmax of float32 logits, lowest index on ties.
//
// IEEE discussion "ArgCompare Benchmark Results and Performance Analysis":
// "VD_Split" tiles a long reduction over many workgroups and merges their
// results, which is what keeps a single 128K-vocabulary row from being
// serialised on one workgroup; the reductions inside a wave are cross-lane.
// Any row length is handled by masking (the discussion's VD pipeline needed
// power-of-two padding instead).
//
// Determinism: every element is mapped to a 64-bit key
//   (order-preserving 32-bit image of the value) << 32 | (0xFFFFFFFF - index)
// so that "larger key" means "larger value, or equal value at a lower index".
// -0 is folded onto +0 before the mapping (IEEE equality) and every NaN maps
// to the largest image (a NaN beats every number; among NaNs the lowest index
// wins).  The maximum of keys is order-independent, so the split into chunks
// and the order of the merges cannot change the result.
#include "argkey.h"
#include "dg_device.h"
#include "dg_internal.h"

#include <mutex>

namespace dg {
namespace {

constexpr int kArgBlock = 256;
constexpr int kMaxChunk = 16384;
constexpr int kMinChunk = 1024;
constexpr int kTargetGroups = 256;
constexpr double kNonTemporalBytes = 64.0 * 1024 * 1024;   // inputs from this size on are read non-temporally

__device__ __forceinline__ uint64_t block_max_u64(uint64_t v) {
    __shared__ uint64_t part[kArgBlock / kWave];
    v = wave_max_u64(v);
    const int wave = threadIdx.x / kWave;
    if (lane_id() == 0) part[wave] = v;
    __syncthreads();
    uint64_t r = part[0];
#pragma unroll
    for (int w = 1; w < kArgBlock / kWave; ++w) r = umax64(r, part[w]);
    return r;
}

// Input element types: decode(raw) is exact (binary16 and bfloat16 widen to
// binary32 without rounding); a 16-byte vector holds kPerVec elements.
struct ElemF32 {
    using raw = float;
    static constexpr int kPerVec = 4;
    __device__ __forceinline__ static float load(const raw* p) { return *p; }
    __device__ __forceinline__ static float from_vec(const u32x4& v, int j) {
        const uint32_t w = j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
        return __builtin_bit_cast(float, w);
    }
};
struct ElemF16 {
    using raw = uint16_t;
    static constexpr int kPerVec = 8;
    __device__ __forceinline__ static float load(const raw* p) { return (float)__builtin_bit_cast(_Float16, *p); }
    __device__ __forceinline__ static float from_vec(const u32x4& v, int j) {
        const uint32_t w = (j >> 1) == 0 ? v.x : (j >> 1) == 1 ? v.y : (j >> 1) == 2 ? v.z : v.w;
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> (16 * (j & 1))));
    }
};
struct ElemBF16 {
    using raw = uint16_t;
    static constexpr int kPerVec = 8;
    __device__ __forceinline__ static float load(const raw* p) { return __builtin_bit_cast(float, (uint32_t)*p << 16); }
    __device__ __forceinline__ static float from_vec(const u32x4& v, int j) {
        const uint32_t w = (j >> 1) == 0 ? v.x : (j >> 1) == 1 ? v.y : (j >> 1) == 2 ? v.z : v.w;
        return __builtin_bit_cast(float, (j & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
};

// The 32-bit image an element contributes to the key: larger image = more
// extreme value (MIN reverses the order of numbers); every NaN maps to the
// top, so a NaN wins for both operations.
template <bool MIN>
__device__ __forceinline__ uint32_t extreme_image(float v) {
    if (v != v) return 0xFFFFFFFFu;
    const uint32_t img = order_image(v);   // never 0xFFFFFFFF for a number
    return MIN ? ~img : img;
}

// Pass 1: workgroup (s, r) reduces elements [s*chunk, min(C, (s+1)*chunk)) of
// row r into one key.  VEC: rows are 16-byte aligned and C is a multiple of
// the elements per 16-byte vector, so every thread reads whole vectors; each
// thread visits its elements in increasing index order and keeps the first
// of equal extremes.  NTL: non-temporal vector loads, for inputs much larger
// than the last-level cache (measured on MI355X: [64, 1M] float32 read from
// HBM 10% faster; logits a GEMV has just written, still in the cache, 15%
// slower).
template <class E, bool MIN, bool VEC, bool NTL>
__global__ void __launch_bounds__(kArgBlock)
k_argcmp_partial(const typename E::raw* __restrict__ x, uint64_t* __restrict__ ws, int C, int64_t ld, int chunk) {
    constexpr int kP = E::kPerVec;
    const int r = blockIdx.y;
    const int s = blockIdx.x;
    const typename E::raw* __restrict__ row = x + (int64_t)r * ld;
    const int c0 = s * chunk;
    const int c1 = min(C, c0 + chunk);
    uint32_t best = 0u, bidx = 0xFFFFFFFFu;
    if constexpr (VEC) {
        constexpr int kU = 4;   // 16-byte loads in flight per thread
        const u32x4* __restrict__ rv = reinterpret_cast<const u32x4*>(row);
        const int v0 = c0 / kP;
        const int v1 = (c1 + kP - 1) / kP;   // the last vector may be partial
        const int vlast = (C - 1) / kP;
        for (int vb = v0 + threadIdx.x; vb < v1; vb += kU * kArgBlock) {
            u32x4 f[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int v = vb + u * kArgBlock;
                f[u] = load_vec<NTL>(rv + (v < v1 ? v : vlast));
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int v = vb + u * kArgBlock;
#pragma unroll
                for (int j = 0; j < kP; ++j) {
                    const int c = kP * v + j;
                    const uint32_t img = extreme_image<MIN>(E::from_vec(f[u], j));
                    if (v < v1 && c < c1 && img > best) { best = img; bidx = (uint32_t)c; }
                }
            }
        }
    } else {
        for (int c = c0 + threadIdx.x; c < c1; c += kArgBlock) {
            const uint32_t img = extreme_image<MIN>(E::load(row + c));
            if (img > best) { best = img; bidx = (uint32_t)c; }
        }
    }
    const uint64_t k = block_max_u64(bidx == 0xFFFFFFFFu ? 0ull : pack_key(best, bidx));
    if (threadIdx.x == 0) ws[(int64_t)r * gridDim.x + s] = k;
}

// Pass 2: one wave per row merges the row's S chunk keys.
__global__ void __launch_bounds__(256)
k_argmax_final(const uint64_t* __restrict__ ws, int64_t* __restrict__ idx, int R, int S) {
    const int r = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (r >= R) return;
    const uint64_t* __restrict__ kr = ws + (int64_t)r * S;
    uint64_t best = 0ull;
    for (int s = lane_id(); s < S; s += kWave) best = umax64(best, kr[s]);
    best = wave_max_u64(best);
    if (lane_id() == 0) idx[r] = (int64_t)key_index(best);
}

int pick_chunk(int64_t R, int64_t C) {
    int chunk = kMaxChunk;
    while (chunk > kMinChunk && R * ((C + chunk - 1) / chunk) < kTargetGroups) chunk >>= 1;
    return chunk;
}

}  // namespace

size_t argmax_workspace_bytes(int64_t R, int64_t C) {
    if (R <= 0 || C <= 0) return 0;
    const int chunk = pick_chunk(R, C);
    const int64_t S = (C + chunk - 1) / chunk;
    return (size_t)(R * S) * sizeof(uint64_t);
}

namespace {

template <class E, bool MIN>
hipError_t launch_argcmp(const void* xv, int64_t* idx, int64_t R, int64_t C, int64_t ld, void* ws, hipStream_t s) {
    const typename E::raw* x = (const typename E::raw*)xv;
    const int chunk = pick_chunk(R, C);
    const int S = (int)((C + chunk - 1) / chunk);
    // vector path only when no vector can reach past column C-1 of any row
    const bool vec = ((uintptr_t)x % 16 == 0) && (ld % E::kPerVec == 0) && (C % E::kPerVec == 0);
    const bool big = (double)R * (double)C * sizeof(typename E::raw) >= kNonTemporalBytes;
    uint64_t* w = (uint64_t*)ws;
    constexpr int64_t kMaxGridY = 65535;
    for (int64_t r0 = 0; r0 < R; r0 += kMaxGridY) {   // grid.y is limited to 65535 rows per launch
        const int64_t rn = R - r0 < kMaxGridY ? R - r0 : kMaxGridY;
        dim3 g1((unsigned)S, (unsigned)rn);
        const typename E::raw* xr = x + r0 * ld;
        uint64_t* wr = w + r0 * S;
        if (vec && big)
            hipLaunchKernelGGL((k_argcmp_partial<E, MIN, true, true>), g1, dim3(kArgBlock), 0, s, xr, wr, (int)C, ld, chunk);
        else if (vec)
            hipLaunchKernelGGL((k_argcmp_partial<E, MIN, true, false>), g1, dim3(kArgBlock), 0, s, xr, wr, (int)C, ld, chunk);
        else
            hipLaunchKernelGGL((k_argcmp_partial<E, MIN, false, false>), g1, dim3(kArgBlock), 0, s, xr, wr, (int)C, ld, chunk);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int rows_per_block = 256 / kWave;
    hipLaunchKernelGGL(k_argmax_final, dim3((unsigned)((R + rows_per_block - 1) / rows_per_block)), dim3(256), 0, s,
                       (const uint64_t*)w, idx, (int)R, S);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_argcompare_rows(const void* x, int dtype, int op, int64_t* idx, int64_t R, int64_t C, int64_t ld,
                                  void* ws, hipStream_t s) {
    const bool mn = op == DG_ARG_MIN;
    switch (dtype) {
        case DG_DTYPE_F32: return mn ? launch_argcmp<ElemF32, true>(x, idx, R, C, ld, ws, s)
                                     : launch_argcmp<ElemF32, false>(x, idx, R, C, ld, ws, s);
        case DG_DTYPE_F16: return mn ? launch_argcmp<ElemF16, true>(x, idx, R, C, ld, ws, s)
                                     : launch_argcmp<ElemF16, false>(x, idx, R, C, ld, ws, s);
        case DG_DTYPE_BF16: return mn ? launch_argcmp<ElemBF16, true>(x, idx, R, C, ld, ws, s)
                                      : launch_argcmp<ElemBF16, false>(x, idx, R, C, ld, ws, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_argmax_rows(const float* x, int64_t* idx, int64_t R, int64_t C, int64_t ld, void* ws,
                              hipStream_t s) {
    return launch_argcompare_rows(x, DG_DTYPE_F32, DG_ARG_MAX, idx, R, C, ld, ws, s);
}

// ---------------------------------------------------------------------------
// The argmax without a caller workspace: its chunk keys go to a fixed array in
// device memory that the library's code object holds (one copy per GPU, alive
// until the process ends), so the call allocates nothing.  The array's name is
// a host-side stand-in in host code; its device address is looked up once per
// device with hipGetSymbolAddress and only that address reaches the kernels.
// Every call on a GPU shares the array: calls that overlap on one GPU race.
// The keys need no clearing: pass 1 writes every key that pass 2 reads.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint64_t scratch[DG_ARGMAX_SCRATCH_BYTES / sizeof(uint64_t)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device ordinal
}  // namespace

hipError_t argmax_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));   // with `dev` current: its own copy
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_argmax_rows_noalloc(const float* x, int64_t* idx, int64_t R, int64_t C, int64_t ld,
                                      hipStream_t s) {
    void* ws = nullptr;
    hipError_t e = argmax_scratch(&ws);
    if (e != hipSuccess) return e;
    return launch_argcompare_rows(x, DG_DTYPE_F32, DG_ARG_MAX, idx, R, C, ld, ws, s);
}

}  // namespace dg
