// stream_read.hip -- HBM streaming-read ceiling probe.
//
// batch1-cdna README, "01-ceiling": a read of a buffer many times larger than
// the last-level cache, 16 bytes per lane per load, with ordinary or
// non-temporal loads; the achieved rate is the denominator of every
// bandwidth-utilisation figure.  The loaded words are summed into a wrapping
// uint32 per workgroup, stored to partials[blockIdx.x] with a plain store, so
// that the loads stay live and the result can be checked exactly.  There is
// no atomic: same-address atomics from every workgroup serialise (about 12 ns
// each on MI355X), which made a probe with thousands of workgroups measure
// the atomics instead of HBM.
//
// Two access orders:
//  * wave-contiguous (default): each wave reads 64 lanes x U x 16 B = 8 KiB
//    (U = 8), 16 KiB (U = 16, DG_READ_DEEP), 4 KiB (U = 4, DG_READ_SHORT) or
//    2 KiB (U = 2, DG_READ_SHORTER) of consecutive bytes per step, then jumps
//    by the whole grid's share -- the order in which a GEMV wave reads its
//    weight row.  With a grid of bytes / (waves * chunk) workgroups every wave
//    reads one chunk and exits, the shape of a one-shot GEMV launch;
//  * grid-stride (the page's kernel): consecutive lanes of the whole grid read
//    consecutive 16-byte vectors, and a lane's kUnroll loads in flight are one
//    grid-size apart.
// The ceiling is the best rate over both orders and the launch shapes, with
// and without a cap on the workgroups resident per CU: a read with every
// wave slot of the chip streaming (tens of MB in flight) was measured slower
// on MI355X than one with a few streams per CU.
#include "dg_device.h"
#include "dg_internal.h"

namespace dg {
namespace {

constexpr int kUnroll = 8;  // 16-byte loads in flight per lane per step (grid-stride order)
constexpr int kLdsPerCu = 160 * 1024;

__device__ __forceinline__ uint32_t add4(u32x4 v) { return (v.x + v.y) + (v.z + v.w); }

__device__ __forceinline__ void finish(uint32_t acc, uint32_t* __restrict__ partials) {
    acc = wave_sum_u32(acc);
    __shared__ uint32_t part[1024 / kWave];
    const int wave = threadIdx.x / kWave;
    if (lane_id() == 0) part[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
        for (int w = 0; w < (int)(blockDim.x / kWave); ++w) s += part[w];
        partials[blockIdx.x] = s;
    }
}

template <bool NT>
__global__ void __launch_bounds__(1024)
k_stream_read_grid(const u32x4* __restrict__ p, uint64_t nvec, uint32_t* __restrict__ partials) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kUnroll - 1) * stride < nvec; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = load_vec<NT>(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc += add4(v[u]);
    }
    for (; i < nvec; i += stride) acc += add4(load_vec<NT>(p + i));
    finish(acc, partials);
}

// HALF: only the even waves of a workgroup read; the odd ones hold their
// slots and meet the workgroup's barrier (the occupancy of a GEMV launch that
// splits each row over two waves when one wave's span covers the row).
template <bool NT, int U, bool HALF>
__global__ void __launch_bounds__(1024)
k_stream_read_wave(const u32x4* __restrict__ p, uint64_t nvec, uint32_t* __restrict__ partials) {
    constexpr uint64_t kChunk = (uint64_t)kWave * U;   // vectors per wave step
    constexpr int kShift = HALF ? 1 : 0;
    const int wib = threadIdx.x / kWave;
    const uint64_t nwaves = (uint64_t)gridDim.x * ((blockDim.x / kWave) >> kShift);
    const uint64_t wave = (uint64_t)blockIdx.x * ((blockDim.x / kWave) >> kShift) + (wib >> kShift);
    const int lane = lane_id();
    uint32_t acc = 0;
    if (!(HALF && (wib & 1))) {   // wave-uniform
        uint64_t c = wave;
        for (; (c + 1) * kChunk <= nvec; c += nwaves) {
            const u32x4* q = p + c * kChunk + lane;
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = load_vec<NT>(q + u * kWave);
#pragma unroll
            for (int u = 0; u < U; ++u) acc += add4(v[u]);
        }
        if (c * kChunk < nvec) {   // the one partial chunk at the end of the buffer
            for (uint64_t i = c * kChunk + lane; i < nvec; i += kWave) acc += add4(load_vec<NT>(p + i));
        }
    }
    finish(acc, partials);
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* d_partials,
                              int grid, int block, int flags, hipStream_t s) {
    const uint64_t nvec = bytes / 16;
    const bool nt = flags & DG_READ_NONTEMPORAL;
    const u32x4* p = (const u32x4*)buf;
    // Occupancy cap: dynamic LDS nobody reads, sized so that at most `cap`
    // workgroups fit one CU's 160 KiB, limits the streams in flight per CU.
    const int cap = (flags >> DG_READ_CAP_SHIFT) & 0xF;
    const size_t lds = cap ? (size_t)(kLdsPerCu / cap / 512 * 512) - 256 : 0;
    if (flags & DG_READ_GRID_STRIDE) {
        if (nt) hipLaunchKernelGGL(k_stream_read_grid<true>, dim3(grid), dim3(block), lds, s, p, nvec, d_partials);
        else hipLaunchKernelGGL(k_stream_read_grid<false>, dim3(grid), dim3(block), lds, s, p, nvec, d_partials);
        return hipGetLastError();
    }
    const int u = (flags & DG_READ_DEEP) ? 16 : (flags & DG_READ_SHORT) ? 4 : (flags & DG_READ_SHORTER) ? 2 : 8;
    const bool half = flags & DG_READ_HALF;
#define DG_READ_CASE(UU)                                                                                        \
    case UU:                                                                                                    \
        if (half) {                                                                                             \
            if (nt) hipLaunchKernelGGL((k_stream_read_wave<true, UU, true>), dim3(grid), dim3(block), lds, s, p, \
                                       nvec, d_partials);                                                       \
            else hipLaunchKernelGGL((k_stream_read_wave<false, UU, true>), dim3(grid), dim3(block), lds, s, p,  \
                                    nvec, d_partials);                                                          \
        } else {                                                                                                \
            if (nt) hipLaunchKernelGGL((k_stream_read_wave<true, UU, false>), dim3(grid), dim3(block), lds, s,   \
                                       p, nvec, d_partials);                                                    \
            else hipLaunchKernelGGL((k_stream_read_wave<false, UU, false>), dim3(grid), dim3(block), lds, s, p, \
                                    nvec, d_partials);                                                          \
        }                                                                                                       \
        break;
    switch (u) {
        DG_READ_CASE(2)
        DG_READ_CASE(4)
        DG_READ_CASE(8)
        DG_READ_CASE(16)
    }
#undef DG_READ_CASE
    return hipGetLastError();
}

}  // namespace dg
