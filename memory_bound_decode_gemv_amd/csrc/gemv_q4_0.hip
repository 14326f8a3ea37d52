// gemv_q4_0.hip -- Q4_0 weights x Q8_1 activations, M = 1..24 columns.
//
// Y[m][n] = sum_b d4(n,b) d8(m,b) sum_{j<32} (q4 - 8) q8, the quantised decode
// GEMV of "The kernel that waited for itself" (Q4_0/Q8_1 harness, small-batch
// kernel for many columns) and of the bitsandbytes issue on 4-bit M = 1 decode
// (70B MLP shape).  Design rules taken from those pages and kept here:
//  * dequantise inside the load loop, never as a separate pass (bitsandbytes
//    issue, "Path Comparison": fused 1147 us vs dequantise + matmul 7574 us);
//  * one 64-lane wavefront per row, consecutive lanes reading consecutive
//    bytes of the row (same issue, 64 threads per block and coalescing notes);
//  * loads issued as a batch before any is consumed, and register use kept low
//    enough for several waves per SIMD ("The kernel that waited for itself",
//    the 105-117 VGPR / 2 waves per SIMD wall);
//  * one kernel family for every column count, so there is no dispatch cliff
//    between 12 and 16 columns (same page, "A dip at sixteen").
//
// Arithmetic.  Each lane owns pairs of consecutive blocks (36 bytes, dword
// aligned because rows are 16-byte aligned when K % 256 == 0).  The 16 code
// bytes of a block split into low nibbles (weights 0..15) and high nibbles
// (weights 16..31) with one mask each; the unsigned codes 0..15 go straight
// into v_dot4_i32_i8 against the signed activation codes, and the -8 offset
// enters as the initial accumulator -8 * sum(q8), computed exactly once per
// activation block.  The int32 block sum is then scaled by d4 * d8 in fp32.
#include "dg_internal.h"
#include "q4_common.h"

namespace dg {
namespace {

using namespace q4;

// ---------------------------------------------------------------------------
// M = 1: the lane's activation pairs stay in registers for every row the wave
// handles (S * 64 pairs cover one row).  Bytes in flight are what a bandwidth
// kernel lives on, so the wave
//  * requests its first row's weights before it touches the activations
//    (their loads and the -8 * sum(q8) preparation hide under HBM latency);
//  * requests row r + stride before it computes row r (a two-row software
//    pipeline: while one row is unpacked and reduced, the next is in flight).
// The branch that guards the prefetch is wave-uniform.
// ---------------------------------------------------------------------------
template <int S>
__global__ void __launch_bounds__(256)
k_q4_m1_regs(const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Xq,
             float* __restrict__ Y, int N, int K) {
    const int lane = lane_id();
    const int wpb = blockDim.x / kWave;
    const int npairs = K >> 6;
    const size_t row_bytes = (size_t)(K >> 5) * 18;
    const int rstride = gridDim.x * wpb;
    int row = blockIdx.x * wpb + wave_in_block();
    if (row >= N) return;

    int pc[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int p = s * kWave + lane;
        pc[s] = p < npairs ? p : npairs - 1;
    }

    uint32_t w[S][9];
#pragma unroll
    for (int s = 0; s < S; ++s) load_weight_pair(Wq + (size_t)row * row_bytes, pc[s], w[s]);

    uint32_t araw[S][18];
#pragma unroll
    for (int s = 0; s < S; ++s) load_act_raw(Xq, pc[s], araw[s]);
    ActPair act[S];
#pragma unroll
    for (int s = 0; s < S; ++s) decode_act_pair(araw[s], s * kWave + lane < npairs, act[s]);   // past the row: 0

    while (true) {
        const int next = row + rstride;
        const bool more = next < N;
        uint32_t wn[S][9];
        if (more) {
#pragma unroll
            for (int s = 0; s < S; ++s) load_weight_pair(Wq + (size_t)next * row_bytes, pc[s], wn[s]);
        }
        float acc = 0.0f;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            WeightPair u;
            unpack_weight_pair(w[s], u);
            acc = pair_dot(u, act[s].qa, act[s].qb, act[s].da, act[s].db, act[s].ca, act[s].cb, acc);
        }
        acc = wave_sum_f32(acc);
        if (lane == 0) Y[row] = acc;
        if (!more) break;
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
            for (int i = 0; i < 9; ++i) w[s][i] = wn[s][i];
        row = next;
    }
}

// ---------------------------------------------------------------------------
// General M: activations of a 64-pair (4096-element) chunk of K, for all M
// columns, are staged once per workgroup in LDS in structure-of-arrays form
// (quad j of pair p of column m at ((m*5 + j)*64 + p)): quads 0-1 hold block
// a's codes, 2-3 block b's, quad 4 holds (d8a, d8b, ca, cb).  Lane p of every
// wave reads pair p, so one ds_read_b128 of the wave covers 1 KiB of
// consecutive LDS.  Each wave owns R rows; each activation quad read from LDS
// serves all R rows.
// ---------------------------------------------------------------------------
constexpr int kChunkPairs = 64;
constexpr int kQuadsPerPair = 5;
constexpr int kLdsBlock = 256;   // threads per workgroup of the LDS kernel

template <int M, int R>
__global__ void __launch_bounds__(kLdsBlock)
k_q4_lds(const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Xq,
         float* __restrict__ Y, int N, int K) {
    extern __shared__ u32x4 lds[];
    const int lane = lane_id();
    const int wave = wave_in_block();
    constexpr int kWaves = kLdsBlock / kWave;
    const int npairs = K >> 6;
    const int nblk = K >> 5;
    const size_t row_bytes = (size_t)nblk * 18;
    const int ntiles = (N + kWaves * R - 1) / (kWaves * R);

    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int row0 = tile * kWaves * R + wave * R;
        float acc[R][M];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

        for (int c0 = 0; c0 < npairs; c0 += kChunkPairs) {
            // weights of this chunk: issued before the staging so that they are in flight meanwhile
            const int gp = c0 + lane;
            const bool pvalid = gp < npairs;
            const int gpc = pvalid ? gp : npairs - 1;
            uint32_t w[R][9];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int row = row0 + r < N ? row0 + r : N - 1;
                load_weight_pair(Wq + (size_t)row * row_bytes, gpc, w[r]);
            }

            __syncthreads();   // the previous chunk's readers are done
            for (int e = threadIdx.x; e < M * 2 * kChunkPairs; e += kLdsBlock) {
                const int m = e / (2 * kChunkPairs);
                const int bl = e % (2 * kChunkPairs);
                const int p = bl >> 1, half = bl & 1;
                const int gb = 2 * (c0 + p) + half;
                uint32_t q[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                float d = 0.0f;
                int c = 0;
                if (c0 + p < npairs) {
                    const uint32_t* b = reinterpret_cast<const uint32_t*>(
                        Xq + ((size_t)m * nblk + gb) * kQ81Bytes);
                    const uint32_t d0 = b[0];
#pragma unroll
                    for (int i = 0; i < 8; ++i) q[i] = b[1 + i];
                    d = half_lo_to_f32(d0);
                    c = -8 * block_code_sum(q);
                }
                u32x4* base = lds + (m * kQuadsPerPair) * kChunkPairs + p;
                base[(half * 2 + 0) * kChunkPairs] = u32x4{q[0], q[1], q[2], q[3]};
                base[(half * 2 + 1) * kChunkPairs] = u32x4{q[4], q[5], q[6], q[7]};
                uint32_t* sc = reinterpret_cast<uint32_t*>(base + 4 * kChunkPairs);
                sc[half] = __builtin_bit_cast(uint32_t, d);
                sc[2 + half] = (uint32_t)c;
            }
            __syncthreads();

            WeightPair u[R];
#pragma unroll
            for (int r = 0; r < R; ++r) unpack_weight_pair(w[r], u[r]);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const u32x4* base = lds + (m * kQuadsPerPair) * kChunkPairs + lane;
                const u32x4 a0 = base[0 * kChunkPairs];
                const u32x4 a1 = base[1 * kChunkPairs];
                const u32x4 b0 = base[2 * kChunkPairs];
                const u32x4 b1 = base[3 * kChunkPairs];
                const u32x4 sc = base[4 * kChunkPairs];
                const uint32_t qa[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                const uint32_t qb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
                const float da = __builtin_bit_cast(float, (uint32_t)sc.x);
                const float db = __builtin_bit_cast(float, (uint32_t)sc.y);
#pragma unroll
                for (int r = 0; r < R; ++r)
                    acc[r][m] = pair_dot(u[r], qa, qb, da, db, (int)sc.z, (int)sc.w, acc[r][m]);
            }
        }

#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float s = wave_sum_f32(acc[r][m]);
                if (lane == 0 && row0 + r < N) Y[(size_t)m * N + row0 + r] = s;
            }
        }
    }
}

size_t lds_bytes(int M) { return (size_t)M * kQuadsPerPair * kChunkPairs * sizeof(u32x4); }

template <int M, int R>
hipError_t launch_lds_mr(const void* Wq, const void* Xq, float* Y, int N, int K, int grid, hipStream_t s) {
    if (lds_bytes(M) > device_max_lds_per_block()) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_q4_lds<M, R>), dim3(grid), dim3(kLdsBlock), lds_bytes(M), s,
                       (const uint8_t*)Wq, (const uint8_t*)Xq, Y, N, K);
    return hipGetLastError();
}

template <int M>
hipError_t launch_lds_m(int R, const void* Wq, const void* Xq, float* Y, int N, int K, int grid, hipStream_t s) {
    if (R == 1) return launch_lds_mr<M, 1>(Wq, Xq, Y, N, K, grid, s);
    if (R == 2) return launch_lds_mr<M, 2>(Wq, Xq, Y, N, K, grid, s);
    if constexpr (M <= 4) {
        if (R == 4) return launch_lds_mr<M, 4>(Wq, Xq, Y, N, K, grid, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_lds(int M, int R, const void* Wq, const void* Xq, float* Y, int N, int K, int grid,
                      hipStream_t s) {
    switch (M) {
#define DG_M(MM) case MM: return launch_lds_m<MM>(R, Wq, Xq, Y, N, K, grid, s);
        DG_M(1) DG_M(2) DG_M(3) DG_M(4) DG_M(5) DG_M(6) DG_M(7) DG_M(8)
        DG_M(9) DG_M(10) DG_M(11) DG_M(12) DG_M(13) DG_M(14) DG_M(15) DG_M(16)
        DG_M(17) DG_M(18) DG_M(19) DG_M(20) DG_M(21) DG_M(22) DG_M(23) DG_M(24)
#undef DG_M
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_regs(int S, const void* Wq, const void* Xq, float* Y, int N, int K, int grid, int block,
                       hipStream_t s) {
    const uint8_t* w = (const uint8_t*)Wq;
    const uint8_t* x = (const uint8_t*)Xq;
    switch (S) {
        case 1: hipLaunchKernelGGL((k_q4_m1_regs<1>), dim3(grid), dim3(block), 0, s, w, x, Y, N, K); break;
        case 2: hipLaunchKernelGGL((k_q4_m1_regs<2>), dim3(grid), dim3(block), 0, s, w, x, Y, N, K); break;
        case 3: hipLaunchKernelGGL((k_q4_m1_regs<3>), dim3(grid), dim3(block), 0, s, w, x, Y, N, K); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

// Default: the quantiser's launch, then the GEMV's.  variant
// DG_VARIANT_Q4_LDSROW selects the one-launch form for one column (K <=
// 16384): every workgroup of the row-streaming kernel quantises the column
// into its LDS copy.  Measured on MI355X it is slower than the two launches
// at every decoder shape (28672 x 8192: 23.8 us at its best grid of 768
// workgroups against 23.6 us), because each of hundreds of workgroups
// repeats the conversion of the whole column, while the quantiser's launch
// costs about 1.8 us.
hipError_t launch_gemv_q4_0_f32(const void* Wq, const float* x, void* Xq, float* Y, int N, int K, int M,
                                const dg_launch* cfg, hipStream_t s) {
    const int S = (K / 64 + kWave - 1) / kWave;
    if (cfg && cfg->variant == DG_VARIANT_Q4_LDSROW) {
        if (M != 1 || S > 4) return hipErrorInvalidValue;
        int grid = cfg->grid, block = cfg->block;
        if (!grid && !block) { grid = N < 3072 ? (N + 3) / 4 : 768; block = 256; }
        return launch_q4_m1_ldsrow(K, cfg->unroll, Wq, nullptr, Y, N, grid, block, s, x, Xq);
    }
    if (cfg && (cfg->grid || cfg->block || cfg->unroll || cfg->variant)) return hipErrorInvalidValue;
    hipError_t e = launch_quantize_q8_1(x, Xq, M, K, s);
    if (e != hipSuccess) return e;
    return launch_gemv_q4_0(Wq, Xq, Y, N, K, M, nullptr, s);
}

hipError_t launch_gemv_q4_0(const void* Wq, const void* Xq, float* Y, int N, int K, int M,
                            const dg_launch* cfg, hipStream_t s) {
    const int npairs = K / 64;
    const int S = (npairs + kWave - 1) / kWave;
    int variant = cfg && cfg->variant ? cfg->variant : 0;
    int lds_rows = 0;   // rows per wave of the dot4 LDS kernel chosen by default
    if (variant == 0) {
        // Measured on MI355X over the decoder shapes, the 70B MLP and M =
        // 1..24 (every kernel family is exact to the same bound, so the
        // choice is speed only): one column streams rows through LDS, whole
        // and two deep for many short rows (16384 rows and more, K <= 8192),
        // in 64-pair units otherwise; up to four columns share the units
        // kernel's weight reads while M * ceil(K / 4096) <= 8 (beyond two
        // columns only above 1024 rows); the rest of two columns, and up to
        // ten columns of a matrix of at most 1024 rows, take the dot4 kernel
        // (the matrix cores' fixed cost per 16 x 16 tile does not pay there:
        // 1024 x 4096 at 9 and 10 columns, 5.1 and 5.0 us against 5.4); the
        // rest take the matrix cores, with the columns resident in LDS for
        // 9..16 columns of matrices of many row tiles.
        if (M == 1) {
            variant = S > 4 ? DG_VARIANT_Q4_LDS : (N >= 16384 && S <= 2 ? DG_VARIANT_Q4_LDSROW : DG_VARIANT_Q4_UNITS);
        } else if (M <= 4 && M * S <= 8 && (N > 1024 || M <= 2)) {
            variant = DG_VARIANT_Q4_UNITS;
        } else if (M == 2 || (N <= 1024 && M <= 10)) {
            variant = DG_VARIANT_Q4_LDS;
            lds_rows = N > 2048 ? 2 : 1;
        } else if (N >= 8192 && K <= 4096 && M >= 9 && M <= 16) {
            variant = DG_VARIANT_Q4_MFMA_RES;
        } else {
            variant = DG_VARIANT_Q4_MFMA;
        }
    }

    if (variant == DG_VARIANT_Q4_REGS) {
        const int block = cfg && cfg->block ? cfg->block : 256;
        if (M != 1 || S > 3 || block > 256) return hipErrorInvalidValue;   // compiled for <= 256 threads
        const int wpb = block / kWave;
        const int grid = cfg && cfg->grid ? cfg->grid : (N + wpb - 1) / wpb;
        return launch_regs(S, Wq, Xq, Y, N, K, grid, block, s);
    }
    if (variant == DG_VARIANT_Q4_LDSROW) {
        if (M != 1) return hipErrorInvalidValue;
        int grid = cfg ? cfg->grid : 0, block = cfg ? cfg->block : 0;
        if (!grid && !block) m1_default_launch(N, grid, block);
        return launch_q4_m1_ldsrow(K, cfg ? cfg->unroll : 0, Wq, Xq, Y, N, grid, block, s);
    }
    if (variant == DG_VARIANT_Q4_UNITS) {
        if (S > 4 || M * S > 8) return hipErrorInvalidValue;
        int grid = cfg ? cfg->grid : 0, block = cfg ? cfg->block : 0;
        if (!grid && !block) units_default_grid(N, M, grid, block);
        return launch_q4_units(K, M, cfg ? cfg->unroll : 0, Wq, Xq, Y, N, grid, block, s);
    }
    if (variant == DG_VARIANT_Q4_MFMA) {
        if (cfg && cfg->block) return hipErrorInvalidValue;   // the configuration fixes the workgroup size
        return launch_q4_mfma(M, cfg ? cfg->unroll : 0, Wq, Xq, Y, N, K, cfg ? cfg->grid : 0, s);
    }
    if (variant == DG_VARIANT_Q4_MFMA_RES) {
        if (cfg && cfg->block) return hipErrorInvalidValue;   // the configuration fixes the workgroup size
        return launch_q4_res(M, cfg ? cfg->unroll : 0, Wq, Xq, Y, N, K, cfg ? cfg->grid : 0, s);
    }
    if (variant == DG_VARIANT_Q4_LDS) {
        if (cfg && cfg->block && cfg->block != kLdsBlock) return hipErrorInvalidValue;
        int R = cfg && cfg->unroll ? cfg->unroll : (lds_rows ? lds_rows : (M <= 8 ? 2 : 1));
        const int rows_per_tile = (kLdsBlock / kWave) * R;
        const int ntiles = (N + rows_per_tile - 1) / rows_per_tile;
        const int grid = cfg && cfg->grid ? cfg->grid : ntiles;
        return launch_lds(M, R, Wq, Xq, Y, N, K, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace dg
