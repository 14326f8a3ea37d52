// dg_internal.h -- host-side declarations shared by the C-ABI layer (api.hip)
// and the kernel launchers in the other translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decodegemv.h"

namespace dg {

// A resolved launch configuration (no zero fields left).
struct Launch {
    int variant;
    int grid;
    int block;
    int unroll;
};

// Launch shape of the LDS-row M = 1 kernels when no grid or block is given
// (the Q4_0 default from 16384 rows on at K <= 8192; measured on MI355X over
// the decoder shapes and the 70B MLP, both formats): every wave gets at least
// two rows so that its copy pipeline has something to overlap (one row per
// wave leaves the pipeline empty), with about 2048 waves for up to 8192 rows
// and 1024 or 2048 workgroups of four waves beyond.
inline void m1_default_launch(int N, int& grid, int& block) {
    block = N <= 8192 ? 128 : 256;
    const int wpb = block / 64;
    const int g = N >= 16384 ? 2048 : 1024;
    const int need = (N + wpb - 1) / wpb;
    grid = need < g ? need : g;
}

// Default grid of the kernels that stream rows in 64-pair units, the default
// path of both quantised formats for few columns (measured on MI355X over
// the decoder shapes, the 70B MLP and 3584 and 7168 rows at K = 8192, against
// the LDS-row kernels and other grids, depths and workgroup sizes):
// workgroups of four waves, 512 of them (2048 from 16384 rows on for one
// column) but never more than the rows need.  The unit depth is chosen by
// the launcher, which knows the LDS a workgroup needs.
inline void units_default_grid(int N, int M, int& grid, int& block) {
    block = 256;
    const int need = (N + 3) / 4;
    const int g = M == 1 && N >= 16384 ? 2048 : 512;
    grid = need < g ? need : g;
}

// Device properties used to size grids and check launches; cached per device.
int device_cu_count();
size_t device_max_lds_per_block();

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* d_partials,
                              int grid, int block, int flags, hipStream_t s);

// Dense GEMV launcher; `bf16` selects bfloat16 operands with fp32 output,
// otherwise binary16 operands with binary16 output.  Returns hipErrorInvalidValue
// for a variant that cannot run this shape.
hipError_t launch_gemv_dense(bool bf16, const void* W, const void* x, void* y,
                             int N, int K, int64_t ldw, const dg_launch* cfg, hipStream_t s);

hipError_t launch_gemv_q4_0(const void* Wq, const void* Xq, float* Y, int N, int K, int M,
                            const dg_launch* cfg, hipStream_t s);
// The M = 1 kernel with rows copied to LDS (depth = row buffers per wave) and
// the matrix-core kernel for M = 2..24 (unroll = RT*10000 + KS*100 + DEPTH*10
// + CB/8); a zero
// depth, unroll, grid or block selects the default.
// xf != nullptr: fp32 activations quantised by each workgroup into its LDS
// column (Xq unused); Xq_out, when given, receives the Q8_1 bytes.
hipError_t launch_q4_m1_ldsrow(int K, int depth, const void* Wq, const void* Xq, float* Y, int N, int grid,
                               int block, hipStream_t s, const float* xf = nullptr, void* Xq_out = nullptr);
// Q4_0 GEMV from fp32 activations: M = 1 (K <= 16384) quantises inside the
// GEMV (one launch); otherwise the quantiser into Xq, then the GEMV.
hipError_t launch_gemv_q4_0_f32(const void* Wq, const float* x, void* Xq, float* Y, int N, int K, int M,
                                const dg_launch* cfg, hipStream_t s);
// M columns with rows streamed through LDS in units of 64 block pairs (depth
// = unit buffers per wave); M * ceil(K / 4096) <= 8 (activation pairs held in
// registers).
hipError_t launch_q4_units(int K, int M, int depth, const void* Wq, const void* Xq, float* Y, int N, int grid,
                           int block, hipStream_t s);
hipError_t launch_q8_units(int K, int M, int depth, const void* Wq, const void* Xq, float* Y, int N, int grid,
                           int block, hipStream_t s);
hipError_t launch_q4_mfma(int M, int unroll, const void* Wq, const void* Xq, float* Y, int N, int K, int grid,
                          hipStream_t s);

// Q4_0 or Q8_0 (q8) in 16-row tiles (the layouts of dg_repack_q4_0_tiles
// and dg_repack_q8_0_tiles): their size, the rearrangement, and the
// matrix-core GEMV over them for 1..24 columns (unroll = CS*100000000 +
// KP*1000000 + RT*10000 + KW*100 + D; 0 = the format's default).
// tiles_config is false for a configuration that is not built or does not
// fit, else gives the workspace bytes it needs (0 when K is not split over
// workgroups).
size_t tiles_bytes(bool q8, int64_t N, int64_t K);
hipError_t launch_tiles_pack(bool q8, const void* Wq, void* Wt, int64_t N, int64_t K, hipStream_t s);
bool tiles_config(bool q8, int N, int K, int M, int unroll, size_t* ws_bytes);
hipError_t launch_tiles(bool q8, int M, int unroll, const void* Wt, const void* Xq, float* Y, void* ws, int N, int K,
                        hipStream_t s);

hipError_t launch_gemv_q8_0(const void* Wq, const void* Xq, float* Y, int N, int K, int M,
                            const dg_launch* cfg, hipStream_t s);
hipError_t launch_q8_mfma(int M, int unroll, const void* Wq, const void* Xq, float* Y, int N, int K, int grid,
                          hipStream_t s);

// The matrix-core kernel with the activation columns resident in LDS, for
// both formats (unroll = RT*10000 + KS*100 + P*10: row tiles and K parts per
// workgroup, chunks in flight per wave; 0 = default).  hipErrorInvalidValue
// when the configuration is not built, K/32 is not a multiple of 8*KS, or
// the workgroup's LDS would not fit.
hipError_t launch_q4_res(int M, int unroll, const void* Wq, const void* Xq, float* Y, int N, int K, int grid,
                         hipStream_t s);
hipError_t launch_q8_res(int M, int unroll, const void* Wq, const void* Xq, float* Y, int N, int K, int grid,
                         hipStream_t s);

hipError_t launch_quantize_q8_0(const float* w, void* Wq, int64_t N, int64_t K, hipStream_t s);

// NF4 x bfloat16, one column (K <= 32768; B in {32, 64, 128, 256}; K % (4B) == 0),
// and the NF4 quantiser.
hipError_t launch_gemv_nf4(const void* codes, const float* absmax, const float* table, const void* x, float* y,
                           int N, int K, int B, const dg_launch* cfg, hipStream_t s);
hipError_t launch_quantize_nf4(const float* w, void* codes, float* absmax, const float* table, int64_t N,
                               int64_t K, int B, hipStream_t s);
hipError_t launch_quantize_q8_1(const float* x, void* Xq, int64_t M, int64_t K, hipStream_t s);
hipError_t launch_quantize_q4_0(const float* w, void* Wq, int64_t N, int64_t K, hipStream_t s);

size_t argmax_workspace_bytes(int64_t R, int64_t C);
hipError_t launch_argmax_rows(const float* x, int64_t* idx, int64_t R, int64_t C, int64_t ld,
                              void* ws, hipStream_t s);
hipError_t launch_argcompare_rows(const void* x, int dtype, int op, int64_t* idx, int64_t R, int64_t C, int64_t ld,
                                  void* ws, hipStream_t s);
// The same argmax with its chunk keys in the library's fixed per-device array
// (DG_ARGMAX_SCRATCH_BYTES); the caller has checked the size.
hipError_t launch_argmax_rows_noalloc(const float* x, int64_t* idx, int64_t R, int64_t C, int64_t ld,
                                      hipStream_t s);

}  // namespace dg
