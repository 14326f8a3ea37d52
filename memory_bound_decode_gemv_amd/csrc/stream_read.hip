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
// The ceiling is the best rate over both orders and the launch shapes.
#include "dg_device.h"
#include "dg_internal.h"

namespace dg {
namespace {

constexpr int kUnroll = 8;  // 16-byte loads in flight per lane per step (grid-stride order)

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

template <bool NT, int U>
__global__ void __launch_bounds__(1024)
k_stream_read_wave(const u32x4* __restrict__ p, uint64_t nvec, uint32_t* __restrict__ partials) {
    constexpr uint64_t kChunk = (uint64_t)kWave * U;   // vectors per wave step
    const uint64_t nwaves = (uint64_t)gridDim.x * (blockDim.x / kWave);
    const uint64_t wave = (uint64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int lane = lane_id();
    uint32_t acc = 0;
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
    finish(acc, partials);
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* d_partials,
                              int grid, int block, int flags, hipStream_t s) {
    const uint64_t nvec = bytes / 16;
    const bool nt = flags & DG_READ_NONTEMPORAL;
    const u32x4* p = (const u32x4*)buf;
    if (flags & DG_READ_GRID_STRIDE) {
        if (nt) hipLaunchKernelGGL(k_stream_read_grid<true>, dim3(grid), dim3(block), 0, s, p, nvec, d_partials);
        else hipLaunchKernelGGL(k_stream_read_grid<false>, dim3(grid), dim3(block), 0, s, p, nvec, d_partials);
    } else if (flags & DG_READ_DEEP) {
        if (nt) hipLaunchKernelGGL((k_stream_read_wave<true, 16>), dim3(grid), dim3(block), 0, s, p, nvec, d_partials);
        else hipLaunchKernelGGL((k_stream_read_wave<false, 16>), dim3(grid), dim3(block), 0, s, p, nvec, d_partials);
    } else if (flags & DG_READ_SHORT) {
        if (nt) hipLaunchKernelGGL((k_stream_read_wave<true, 4>), dim3(grid), dim3(block), 0, s, p, nvec, d_partials);
        else hipLaunchKernelGGL((k_stream_read_wave<false, 4>), dim3(grid), dim3(block), 0, s, p, nvec, d_partials);
    } else if (flags & DG_READ_SHORTER) {
        if (nt) hipLaunchKernelGGL((k_stream_read_wave<true, 2>), dim3(grid), dim3(block), 0, s, p, nvec, d_partials);
        else hipLaunchKernelGGL((k_stream_read_wave<false, 2>), dim3(grid), dim3(block), 0, s, p, nvec, d_partials);
    } else {
        if (nt) hipLaunchKernelGGL((k_stream_read_wave<true, 8>), dim3(grid), dim3(block), 0, s, p, nvec, d_partials);
        else hipLaunchKernelGGL((k_stream_read_wave<false, 8>), dim3(grid), dim3(block), 0, s, p, nvec, d_partials);
    }
    return hipGetLastError();
}

}  // namespace dg
