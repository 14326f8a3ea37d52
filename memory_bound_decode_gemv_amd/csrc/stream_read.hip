// stream_read.hip -- HBM streaming-read ceiling probe.
//
// batch1-cdna README, "01-ceiling": a grid-stride read of a buffer many times
// larger than the last-level cache, 16 bytes per lane per load, with ordinary
// or non-temporal loads; the achieved rate is the denominator of every
// bandwidth-utilisation figure.  Here the loaded words are summed into a
// wrapping uint32 checksum (one atomic add per workgroup) so that the loads
// stay live and the result can be checked exactly.
#include "dg_device.h"
#include "dg_internal.h"

namespace dg {
namespace {

constexpr int kUnroll = 8;  // 16-byte loads in flight per lane per step

template <bool NT>
__global__ void __launch_bounds__(1024)
k_stream_read(const u32x4* __restrict__ p, uint64_t nvec, uint32_t* __restrict__ checksum) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    // Full steps: kUnroll independent loads are issued before any is consumed.
    for (; i + (kUnroll - 1) * stride < nvec; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = load_vec<NT>(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
    }
    for (; i < nvec; i += stride) {
        u32x4 v = load_vec<NT>(p + i);
        acc += (v.x + v.y) + (v.z + v.w);
    }
    acc = wave_sum_u32(acc);
    __shared__ uint32_t part[1024 / kWave];
    const int wave = threadIdx.x / kWave;
    if (lane_id() == 0) part[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
        for (int w = 0; w < (int)(blockDim.x / kWave); ++w) s += part[w];
        atomicAdd(checksum, s);
    }
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* d_checksum,
                              int grid, int block, bool nontemporal, hipStream_t s) {
    const uint64_t nvec = bytes / 16;
    if (nontemporal)
        hipLaunchKernelGGL(k_stream_read<true>, dim3(grid), dim3(block), 0, s,
                           (const u32x4*)buf, nvec, d_checksum);
    else
        hipLaunchKernelGGL(k_stream_read<false>, dim3(grid), dim3(block), 0, s,
                           (const u32x4*)buf, nvec, d_checksum);
    return hipGetLastError();
}

}  // namespace dg
