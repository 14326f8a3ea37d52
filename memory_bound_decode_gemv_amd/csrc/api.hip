// api.hip -- the extern "C" entry points of libdecodegemv: argument checks
// (all done before anything touches the HIP runtime), launch-configuration
// defaults, and error reporting.  The contracts are documented in
// include/decodegemv.h.
#include <atomic>
#include <string>

#include "dg_device.h"
#include "dg_internal.h"

namespace dg {
namespace {

thread_local std::string g_last_hip_error;

constexpr int64_t kI32Max = 2147483647;
constexpr int64_t kQuantMaxK = int64_t(1) << 26;   // Q4_0 / Q8_0 rows: 32-bit copy offsets in every kernel

dg_status hip_status(hipError_t e) {
    if (e == hipSuccess) return DG_OK;
    g_last_hip_error = std::string(hipGetErrorName(e)) + ": " + hipGetErrorString(e);
    return DG_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool launch_ok(const dg_launch* cfg) {
    if (!cfg) return true;
    if (cfg->variant < 0 || cfg->grid < 0 || cfg->block < 0 || cfg->unroll < 0) return false;
    if (cfg->block && (cfg->block % kWave != 0 || cfg->block > 1024)) return false;
    return true;
}

__global__ void k_fill_zero_f32(float* __restrict__ y, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) y[i] = 0.0f;
}

dg_status gemv_dense_checked(bool bf16, const void* W, const void* x, void* y, int64_t N, int64_t K,
                             int64_t ldw, const dg_launch* cfg, dg_stream stream) {
    if (N < 0 || N > kI32Max || K < 0 || K > kI32Max || K % 8 != 0 || ldw < K || ldw % 8 != 0)
        return DG_ERR_SHAPE;
    if (!launch_ok(cfg)) return DG_ERR_ARG;
    if (N == 0) return DG_OK;
    if (!y || (K > 0 && (!W || !x))) return DG_ERR_NULL;
    if (!aligned(y, bf16 ? 4 : 2)) return DG_ERR_MISALIGNED;
    if (K > 0 && (!aligned(W, 16) || !aligned(x, 16))) return DG_ERR_MISALIGNED;
    hipError_t e = launch_gemv_dense(bf16, W, x, y, (int)N, (int)K, ldw, cfg, (hipStream_t)stream);
    if (e == hipErrorInvalidValue && cfg && (cfg->variant || cfg->unroll)) return DG_ERR_ARG;
    return hip_status(e);
}

dg_status gemv_quant_checked(bool q8, const void* Wq, const void* Xq, float* Y, int64_t N, int64_t K, int M,
                             const dg_launch* cfg, dg_stream stream) {
    if (N < 0 || N > kI32Max || K < 0 || K > kQuantMaxK || K % 256 != 0 || M < 0 || M > 24)
        return DG_ERR_SHAPE;
    if (!launch_ok(cfg)) return DG_ERR_ARG;
    if (N == 0 || M == 0) return DG_OK;
    if (!Y || (K > 0 && (!Wq || !Xq))) return DG_ERR_NULL;
    if (!aligned(Y, 4)) return DG_ERR_MISALIGNED;
    if (K > 0 && (!aligned(Wq, 16) || !aligned(Xq, 16))) return DG_ERR_MISALIGNED;
    if (K == 0) {   // empty sums: Y = 0
        const int64_t n = N * (int64_t)M;
        hipLaunchKernelGGL(k_fill_zero_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                           (hipStream_t)stream, Y, n);
        return hip_status(hipGetLastError());
    }
    hipError_t e = q8 ? launch_gemv_q8_0(Wq, Xq, Y, (int)N, (int)K, M, cfg, (hipStream_t)stream)
                      : launch_gemv_q4_0(Wq, Xq, Y, (int)N, (int)K, M, cfg, (hipStream_t)stream);
    if (e == hipErrorInvalidValue && cfg && (cfg->variant || cfg->unroll || cfg->block)) return DG_ERR_ARG;
    return hip_status(e);
}

dg_status gemv_tiles_checked(bool q8, const void* Wt, const void* Xq, float* Y, int64_t N, int64_t K, int M,
                             void* ws, size_t ws_bytes, const dg_launch* cfg, dg_stream stream) {
    if (N < 0 || N > kI32Max || K < 0 || K > kQuantMaxK || K % 256 != 0 || M < 0 || M > 24)
        return DG_ERR_SHAPE;
    if (!launch_ok(cfg) || (cfg && (cfg->variant || cfg->grid || cfg->block))) return DG_ERR_ARG;
    if (N == 0 || M == 0) return DG_OK;
    if (!Y || (K > 0 && (!Wt || !Xq))) return DG_ERR_NULL;
    if (!aligned(Y, 4)) return DG_ERR_MISALIGNED;
    if (K > 0 && (!aligned(Wt, 16) || !aligned(Xq, 16) || !aligned(ws, 16))) return DG_ERR_MISALIGNED;
    if (K == 0) {   // empty sums: Y = 0
        const int64_t n = N * (int64_t)M;
        hipLaunchKernelGGL(k_fill_zero_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                           (hipStream_t)stream, Y, n);
        return hip_status(hipGetLastError());
    }
    size_t need = 0;
    if (!tiles_config(q8, (int)N, (int)K, M, cfg ? cfg->unroll : 0, &need)) return DG_ERR_ARG;
    if (need > 0 && (!ws || ws_bytes < need)) return DG_ERR_WORKSPACE;
    hipError_t e = launch_tiles(q8, M, cfg ? cfg->unroll : 0, Wt, Xq, Y, ws, (int)N, (int)K, (hipStream_t)stream);
    if (e == hipErrorInvalidValue) return DG_ERR_ARG;
    return hip_status(e);
}

size_t tiles_bytes_checked(bool q8, int64_t N, int64_t K) {
    if (N < 0 || N > kI32Max || K < 0 || K > kQuantMaxK || K % 256 != 0) return 0;
    return tiles_bytes(q8, N, K);
}

dg_status repack_tiles_checked(bool q8, const void* Wq, void* Wt, int64_t N, int64_t K, dg_stream stream) {
    if (N < 0 || N > kI32Max || K < 0 || K > kQuantMaxK || K % 256 != 0) return DG_ERR_SHAPE;
    if (N == 0 || K == 0) return DG_OK;
    if (!Wq || !Wt) return DG_ERR_NULL;
    if (!aligned(Wq, 2) || !aligned(Wt, 16)) return DG_ERR_MISALIGNED;
    return hip_status(launch_tiles_pack(q8, Wq, Wt, N, K, (hipStream_t)stream));
}

size_t tiles_workspace_checked(bool q8, int64_t N, int64_t K, int M) {
    size_t need = 0;
    if (N <= 0 || N > kI32Max || K <= 0 || K > kQuantMaxK || K % 256 != 0 || M <= 0 || M > 24) return 0;
    return tiles_config(q8, (int)N, (int)K, M, 0, &need) ? need : 0;
}

bool nf4_block_ok(int B) { return B == 32 || B == 64 || B == 128 || B == 256; }

dg_status gemv_nf4_checked(const void* codes, const float* absmax, const float* table, const void* x, float* y,
                           int64_t N, int64_t K, int B, const dg_launch* cfg, dg_stream stream) {
    if (N < 0 || N > kI32Max || K < 0 || K > 32768 || K % 256 != 0 || !nf4_block_ok(B) || K % (4 * B) != 0)
        return DG_ERR_SHAPE;
    if (!launch_ok(cfg)) return DG_ERR_ARG;
    if (N == 0) return DG_OK;
    if (!y || (K > 0 && (!codes || !absmax || !table || !x))) return DG_ERR_NULL;
    if (!aligned(y, 4)) return DG_ERR_MISALIGNED;
    if (K > 0 && (!aligned(codes, 16) || !aligned(absmax, 16) || !aligned(table, 16) || !aligned(x, 16)))
        return DG_ERR_MISALIGNED;
    if (K == 0) {   // empty sums: y = 0
        hipLaunchKernelGGL(k_fill_zero_f32, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                           y, N);
        return hip_status(hipGetLastError());
    }
    hipError_t e = launch_gemv_nf4(codes, absmax, table, x, y, (int)N, (int)K, B, cfg, (hipStream_t)stream);
    if (e == hipErrorInvalidValue && cfg && (cfg->variant || cfg->unroll || cfg->block)) return DG_ERR_ARG;
    return hip_status(e);
}

}  // namespace

int device_cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cached[dev].store(v, std::memory_order_relaxed);
    return v;
}

size_t device_max_lds_per_block() {
    static std::atomic<long long> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 64 * 1024;
    long long v = cached[dev].load(std::memory_order_relaxed);
    if (v > 0) return (size_t)v;
    int a = 0;
    if (hipDeviceGetAttribute(&a, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || a <= 0)
        a = 64 * 1024;
    cached[dev].store(a, std::memory_order_relaxed);
    return (size_t)a;
}

}  // namespace dg

using namespace dg;

extern "C" {

const char* dg_status_string(dg_status status) {
    switch (status) {
        case DG_OK: return "DG_OK";
        case DG_ERR_NULL: return "DG_ERR_NULL: a required pointer is NULL";
        case DG_ERR_MISALIGNED: return "DG_ERR_MISALIGNED: a pointer breaks its alignment contract";
        case DG_ERR_SHAPE: return "DG_ERR_SHAPE: a size is outside the documented contract";
        case DG_ERR_WORKSPACE: return "DG_ERR_WORKSPACE: workspace missing or too small";
        case DG_ERR_HIP: return "DG_ERR_HIP: the HIP runtime reported an error";
        case DG_ERR_ARG: return "DG_ERR_ARG: invalid argument or launch override";
    }
    return "unknown dg_status";
}

const char* dg_last_hip_error(void) { return g_last_hip_error.c_str(); }

dg_status dg_stream_read(const void* buf, size_t bytes, uint32_t* d_partials, int grid_blocks,
                         int block_threads, int flags, dg_stream stream) {
    if (bytes % 16 != 0) return DG_ERR_SHAPE;
    constexpr int kDepthFlags = DG_READ_DEEP | DG_READ_SHORT | DG_READ_SHORTER;
    if (grid_blocks < 0 || block_threads < 0 ||
        (flags & ~(DG_READ_NONTEMPORAL | DG_READ_GRID_STRIDE | kDepthFlags | DG_READ_HALF |
                   (0xF << DG_READ_CAP_SHIFT))))
        return DG_ERR_ARG;
    const int depth = flags & kDepthFlags;
    if ((depth & (depth - 1)) != 0 || (depth && (flags & DG_READ_GRID_STRIDE))) return DG_ERR_ARG;
    if ((flags & DG_READ_HALF) && ((flags & DG_READ_GRID_STRIDE) || (block_threads ? block_threads : 512) % 128 != 0))
        return DG_ERR_ARG;
    if (block_threads && (block_threads % kWave != 0 || block_threads > 1024)) return DG_ERR_ARG;
    if (bytes == 0) return DG_OK;
    if (!buf || !d_partials) return DG_ERR_NULL;
    if (!aligned(buf, 16) || !aligned(d_partials, 4)) return DG_ERR_MISALIGNED;
    const int grid = grid_blocks ? grid_blocks : DG_READ_DEFAULT_GRID;
    const int block = block_threads ? block_threads : 512;
    return hip_status(launch_stream_read(buf, bytes, d_partials, grid, block, flags, (hipStream_t)stream));
}

dg_status dg_gemv_f16(const void* W, const void* x, void* y, int64_t N, int64_t K, int64_t ldw,
                      dg_stream stream) {
    return gemv_dense_checked(false, W, x, y, N, K, ldw, nullptr, stream);
}

dg_status dg_gemv_bf16(const void* W, const void* x, float* y, int64_t N, int64_t K, int64_t ldw,
                       dg_stream stream) {
    return gemv_dense_checked(true, W, x, y, N, K, ldw, nullptr, stream);
}

dg_status dg_gemv_f16_ex(const void* W, const void* x, void* y, int64_t N, int64_t K, int64_t ldw,
                         const dg_launch* cfg, dg_stream stream) {
    return gemv_dense_checked(false, W, x, y, N, K, ldw, cfg, stream);
}

dg_status dg_gemv_bf16_ex(const void* W, const void* x, float* y, int64_t N, int64_t K, int64_t ldw,
                          const dg_launch* cfg, dg_stream stream) {
    return gemv_dense_checked(true, W, x, y, N, K, ldw, cfg, stream);
}

dg_status dg_gemv_q4_0(const void* Wq, const void* Xq, float* Y, int64_t N, int64_t K, int M,
                       dg_stream stream) {
    return gemv_quant_checked(false, Wq, Xq, Y, N, K, M, nullptr, stream);
}

dg_status dg_gemv_q4_0_ex(const void* Wq, const void* Xq, float* Y, int64_t N, int64_t K, int M,
                          const dg_launch* cfg, dg_stream stream) {
    return gemv_quant_checked(false, Wq, Xq, Y, N, K, M, cfg, stream);
}

dg_status dg_gemv_q8_0(const void* Wq, const void* Xq, float* Y, int64_t N, int64_t K, int M,
                       dg_stream stream) {
    return gemv_quant_checked(true, Wq, Xq, Y, N, K, M, nullptr, stream);
}

dg_status dg_gemv_q8_0_ex(const void* Wq, const void* Xq, float* Y, int64_t N, int64_t K, int M,
                          const dg_launch* cfg, dg_stream stream) {
    return gemv_quant_checked(true, Wq, Xq, Y, N, K, M, cfg, stream);
}

size_t dg_q4_0_tiles_bytes(int64_t N, int64_t K) { return tiles_bytes_checked(false, N, K); }
size_t dg_q8_0_tiles_bytes(int64_t N, int64_t K) { return tiles_bytes_checked(true, N, K); }

dg_status dg_repack_q4_0_tiles(const void* Wq, void* Wt, int64_t N, int64_t K, dg_stream stream) {
    return repack_tiles_checked(false, Wq, Wt, N, K, stream);
}
dg_status dg_repack_q8_0_tiles(const void* Wq, void* Wt, int64_t N, int64_t K, dg_stream stream) {
    return repack_tiles_checked(true, Wq, Wt, N, K, stream);
}

size_t dg_gemv_q4_0_tiles_workspace_bytes(int64_t N, int64_t K, int M) {
    return tiles_workspace_checked(false, N, K, M);
}
size_t dg_gemv_q8_0_tiles_workspace_bytes(int64_t N, int64_t K, int M) {
    return tiles_workspace_checked(true, N, K, M);
}

dg_status dg_gemv_q4_0_tiles(const void* Wt, const void* Xq, float* Y, int64_t N, int64_t K, int M, void* ws,
                             size_t ws_bytes, dg_stream stream) {
    return gemv_tiles_checked(false, Wt, Xq, Y, N, K, M, ws, ws_bytes, nullptr, stream);
}

dg_status dg_gemv_q4_0_tiles_ex(const void* Wt, const void* Xq, float* Y, int64_t N, int64_t K, int M, void* ws,
                                size_t ws_bytes, const dg_launch* cfg, dg_stream stream) {
    return gemv_tiles_checked(false, Wt, Xq, Y, N, K, M, ws, ws_bytes, cfg, stream);
}

dg_status dg_gemv_q8_0_tiles(const void* Wt, const void* Xq, float* Y, int64_t N, int64_t K, int M, void* ws,
                             size_t ws_bytes, dg_stream stream) {
    return gemv_tiles_checked(true, Wt, Xq, Y, N, K, M, ws, ws_bytes, nullptr, stream);
}

dg_status dg_gemv_q8_0_tiles_ex(const void* Wt, const void* Xq, float* Y, int64_t N, int64_t K, int M, void* ws,
                                size_t ws_bytes, const dg_launch* cfg, dg_stream stream) {
    return gemv_tiles_checked(true, Wt, Xq, Y, N, K, M, ws, ws_bytes, cfg, stream);
}

dg_status dg_gemv_q4_0_f32_ex(const void* Wq, const float* x, float* Y, void* Xq, int64_t N, int64_t K, int M,
                              const dg_launch* cfg, dg_stream stream) {
    if (N < 0 || N > kI32Max || K < 0 || K > kQuantMaxK || K % 256 != 0 || M < 0 || M > 24) return DG_ERR_SHAPE;
    if (!launch_ok(cfg) || (cfg && cfg->variant && cfg->variant != DG_VARIANT_Q4_LDSROW)) return DG_ERR_ARG;
    if (N == 0 || M == 0) return DG_OK;
    const bool one_launch = cfg && cfg->variant == DG_VARIANT_Q4_LDSROW;
    if (!Y || (K > 0 && (!Wq || !x || (!one_launch && !Xq)))) return DG_ERR_NULL;
    if (!aligned(Y, 4)) return DG_ERR_MISALIGNED;
    if (K > 0 && (!aligned(Wq, 16) || !aligned(x, 16) || (Xq && !aligned(Xq, 16)))) return DG_ERR_MISALIGNED;
    if (K == 0) {   // empty sums: Y = 0 (there are no blocks to store)
        const int64_t n = N * (int64_t)M;
        hipLaunchKernelGGL(k_fill_zero_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                           (hipStream_t)stream, Y, n);
        return hip_status(hipGetLastError());
    }
    hipError_t e = launch_gemv_q4_0_f32(Wq, x, Xq, Y, (int)N, (int)K, M, cfg, (hipStream_t)stream);
    if (e == hipErrorInvalidValue && cfg) return DG_ERR_ARG;
    return hip_status(e);
}

dg_status dg_gemv_q4_0_f32(const void* Wq, const float* x, float* Y, void* Xq, int64_t N, int64_t K, int M,
                           dg_stream stream) {
    return dg_gemv_q4_0_f32_ex(Wq, x, Y, Xq, N, K, M, nullptr, stream);
}

dg_status dg_quantize_q8_1(const float* x, void* Xq, int64_t M, int64_t K, dg_stream stream) {
    if (M < 0 || K < 0 || K % 32 != 0 || M * (K / 32) > kI32Max * 8LL) return DG_ERR_SHAPE;   // 8 blocks per workgroup
    if (M == 0 || K == 0) return DG_OK;
    if (!x || !Xq) return DG_ERR_NULL;
    if (!aligned(x, 16) || !aligned(Xq, 4)) return DG_ERR_MISALIGNED;
    return hip_status(launch_quantize_q8_1(x, Xq, M, K, (hipStream_t)stream));
}

dg_status dg_quantize_q4_0(const float* w, void* Wq, int64_t N, int64_t K, dg_stream stream) {
    if (N < 0 || K < 0 || K % 32 != 0 || N * (K / 32) > kI32Max * 256LL) return DG_ERR_SHAPE;
    if (N == 0 || K == 0) return DG_OK;
    if (!w || !Wq) return DG_ERR_NULL;
    if (!aligned(w, 16) || !aligned(Wq, 2)) return DG_ERR_MISALIGNED;
    return hip_status(launch_quantize_q4_0(w, Wq, N, K, (hipStream_t)stream));
}

dg_status dg_quantize_q8_0(const float* w, void* Wq, int64_t N, int64_t K, dg_stream stream) {
    if (N < 0 || K < 0 || K % 32 != 0 || N * (K / 32) > kI32Max * 256LL) return DG_ERR_SHAPE;
    if (N == 0 || K == 0) return DG_OK;
    if (!w || !Wq) return DG_ERR_NULL;
    if (!aligned(w, 16) || !aligned(Wq, 2)) return DG_ERR_MISALIGNED;
    return hip_status(launch_quantize_q8_0(w, Wq, N, K, (hipStream_t)stream));
}

dg_status dg_gemv_nf4(const void* codes, const float* absmax, const float* table, const void* x, float* y,
                      int64_t N, int64_t K, int B, dg_stream stream) {
    return gemv_nf4_checked(codes, absmax, table, x, y, N, K, B, nullptr, stream);
}

dg_status dg_gemv_nf4_ex(const void* codes, const float* absmax, const float* table, const void* x, float* y,
                         int64_t N, int64_t K, int B, const dg_launch* cfg, dg_stream stream) {
    return gemv_nf4_checked(codes, absmax, table, x, y, N, K, B, cfg, stream);
}

dg_status dg_quantize_nf4(const float* w, void* codes, float* absmax, const float* table, int64_t N, int64_t K,
                          int B, dg_stream stream) {
    if (N < 0 || K < 0 || !nf4_block_ok(B) || K % B != 0 || N * (K / B) > kI32Max * 256LL) return DG_ERR_SHAPE;
    if (N == 0 || K == 0) return DG_OK;
    if (!w || !codes || !absmax || !table) return DG_ERR_NULL;
    if (!aligned(w, 16) || !aligned(codes, 2) || !aligned(absmax, 4) || !aligned(table, 4)) return DG_ERR_MISALIGNED;
    return hip_status(launch_quantize_nf4(w, codes, absmax, table, N, K, B, (hipStream_t)stream));
}

size_t dg_argmax_workspace_bytes(int64_t R, int64_t C) { return argmax_workspace_bytes(R, C); }

// The greedy tail as one call: the GEMV, then the split argmax of its
// logits.  (Argmax epilogues inside the GEMV were measured and were slower on
// MI355X: a grid-stride GEMV capped at 2048 workgroups, 167 us, and one
// device-scope atomic max per workgroup, 177 us, against 153 us for this.)
// Workspace: the logits when the caller stores none, then the argmax's.
size_t tail_logits_bytes(int64_t N) { return ((size_t)N * sizeof(float) + 15) & ~(size_t)15; }

size_t dg_gemv_bf16_argmax_workspace_bytes(int64_t N, int64_t K) {
    (void)K;
    if (N < 1) return 0;
    return tail_logits_bytes(N) + argmax_workspace_bytes(1, N);
}

dg_status dg_gemv_bf16_argmax(const void* W, const void* x, float* y, int64_t* idx, int64_t N, int64_t K,
                              int64_t ldw, void* ws, size_t ws_bytes, dg_stream stream) {
    if (N < 1 || N > kI32Max || K < 0 || K > kI32Max || K % 8 != 0 || ldw < K || ldw % 8 != 0)
        return DG_ERR_SHAPE;
    if (!idx || (K > 0 && (!W || !x))) return DG_ERR_NULL;
    if (!aligned(idx, 8) || (y && !aligned(y, 4))) return DG_ERR_MISALIGNED;
    if (K > 0 && (!aligned(W, 16) || !aligned(x, 16))) return DG_ERR_MISALIGNED;
    const size_t need = dg_gemv_bf16_argmax_workspace_bytes(N, K);
    if (!ws || ws_bytes < need) return DG_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return DG_ERR_MISALIGNED;
    float* logits = y ? y : (float*)ws;
    void* aws = (uint8_t*)ws + tail_logits_bytes(N);
    dg_status st = gemv_dense_checked(true, W, x, logits, N, K, ldw, nullptr, stream);
    if (st != DG_OK) return st;
    return hip_status(launch_argmax_rows(logits, idx, 1, N, N, aws, (hipStream_t)stream));
}

dg_status dg_argcompare_rows(const void* x, int dtype, int op, int64_t* idx, int64_t R, int64_t C, int64_t ld,
                             void* ws, size_t ws_bytes, dg_stream stream) {
    if (dtype != DG_DTYPE_F32 && dtype != DG_DTYPE_F16 && dtype != DG_DTYPE_BF16) return DG_ERR_ARG;
    if (op != DG_ARG_MAX && op != DG_ARG_MIN) return DG_ERR_ARG;
    if (R < 0 || R > kI32Max || C < 1 || C >= kI32Max || ld < C) return DG_ERR_SHAPE;
    if (R == 0) return DG_OK;
    if (!x || !idx) return DG_ERR_NULL;
    if (!aligned(x, dtype == DG_DTYPE_F32 ? 4 : 2) || !aligned(idx, 8)) return DG_ERR_MISALIGNED;
    const size_t need = argmax_workspace_bytes(R, C);
    if (need > 0 && (!ws || ws_bytes < need)) return DG_ERR_WORKSPACE;
    if (ws && !aligned(ws, 8)) return DG_ERR_MISALIGNED;
    return hip_status(launch_argcompare_rows(x, dtype, op, idx, R, C, ld, ws, (hipStream_t)stream));
}

dg_status dg_argmax_rows_noalloc(const float* x, int64_t* idx, int64_t R, int64_t C, int64_t ld,
                                 dg_stream stream) {
    if (R < 0 || R > kI32Max || C < 1 || C >= kI32Max || ld < C) return DG_ERR_SHAPE;
    if (R == 0) return DG_OK;
    if (!x || !idx) return DG_ERR_NULL;
    if (!aligned(x, 4) || !aligned(idx, 8)) return DG_ERR_MISALIGNED;
    if (argmax_workspace_bytes(R, C) > DG_ARGMAX_SCRATCH_BYTES) return DG_ERR_WORKSPACE;
    return hip_status(launch_argmax_rows_noalloc(x, idx, R, C, ld, (hipStream_t)stream));
}

dg_status dg_argmax_rows(const float* x, int64_t* idx, int64_t R, int64_t C, int64_t ld, void* ws,
                         size_t ws_bytes, dg_stream stream) {
    if (R < 0 || R > kI32Max || C < 1 || C >= kI32Max || ld < C) return DG_ERR_SHAPE;
    if (R == 0) return DG_OK;
    if (!x || !idx) return DG_ERR_NULL;
    if (!aligned(x, 4) || !aligned(idx, 8)) return DG_ERR_MISALIGNED;
    const size_t need = argmax_workspace_bytes(R, C);
    if (need > 0 && (!ws || ws_bytes < need)) return DG_ERR_WORKSPACE;
    if (ws && !aligned(ws, 8)) return DG_ERR_MISALIGNED;
    return hip_status(launch_argmax_rows(x, idx, R, C, ld, ws, (hipStream_t)stream));
}

}  // extern "C"
