// gemv_q8_0.hip -- Q8_0 weights x Q8_1 activations, M = 1..24 columns.
//
// Y[m][n] = sum_b dw(n,b) d8(m,b) sum_{j<32} qw q8: the Q8_0 model files that
// "The kernel that waited for itself" runs through the same Q8_1-activation
// path as Q4_0 (four-model comparison).  A Q8_0 block is 34 bytes (binary16 d,
// 32 int8 codes), so a row moves 34/32 bytes per weight, 1.9 times the Q4_0
// row; the decode is simpler (no nibbles, no -8 offset).
//  * M = 1: the rows stream through LDS like the Q4_0 M = 1 kernel (one wave
//    per row, global_load_lds_dwordx4 copies, DEPTH row buffers per wave,
//    explicit vmcnt waits); a block pair is 68 bytes = 17 dwords, an odd lane
//    stride, so the ds_read of the 64 lanes are free of bank conflicts.
//  * M = 2..24, and M = 1 rows longer than 256 block pairs: the matrix-core
//    kernel of the Q4_0 path with a Q8_0 decoder (one v_mfma_i32_16x16x32_i8
//    per block and 16 x 16 tile, no offset operation).
#include "dg_internal.h"
#include "q4_common.h"

namespace dg {
namespace {

using namespace q4;

constexpr int kQ80PairBytes = 68;

template <int S, int C, int DEPTH>
__global__ void __launch_bounds__(256)
k_q8_m1_ldsrow(const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Xq, float* __restrict__ Y, int N, int K) {
    static_assert(DEPTH >= 2 && DEPTH <= 4, "pipeline depth");
    static_assert(C * (DEPTH - 1) <= 63, "wait count exceeds the vmcnt field");
    extern __shared__ u32x4 lds_rows8[];
    const int lane = lane_id();
    const int wave = wave_in_block();
    const int wpb = blockDim.x / kWave;
    const int npairs = K >> 6;
    const int row_bytes = (K >> 5) * 34;
    const int nchunks = row_bytes >> 4;
    const int rstride = gridDim.x * wpb;
    const int row0 = blockIdx.x * wpb + wave;
    uint8_t* const acts = reinterpret_cast<uint8_t*>(lds_rows8);
    uint8_t* const lds_base = acts + column_lds_bytes(K) + wave * DEPTH * row_bytes;

    // the workgroup's copy of the activation column first, then the first rows
    copy_column_to_lds(Xq, K, acts, wave, wpb, lane);
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d) {
        const int r = row0 + d * rstride;
        if (r < N) copy_row_to_lds<C>(Wq + (size_t)r * row_bytes, lds_base + d * row_bytes, nchunks, lane);
    }
    {   // this wave's column copies have landed once only its issued rows can be outstanding
        const int rows = row0 < N ? (N - 1 - row0) / rstride + 1 : 0;   // wave-uniform
        wait_rows_ahead<C, DEPTH>(rows < DEPTH - 1 ? rows : DEPTH - 1);
        lds_barrier();
    }
    if (row0 >= N) return;   // after the barrier: every wave takes part in it

    int pc[S];
    ActPair act[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int p = s * kWave + lane;
        pc[s] = p < npairs ? p : npairs - 1;
        uint32_t v[18];
        load_act_raw(acts, pc[s], v);
        decode_act_pair(v, p < npairs, act[s]);   // past the row: contributes 0
    }

    // outputs held back and stored 64 rows at a time (lane i holds the i-th row)
    float out = 0.0f;
    int nout = 0;
    int out_row0 = row0;
    int slot = 0;
    for (int row = row0; row < N; row += rstride) {
        const int ahead = row + (DEPTH - 1) * rstride;
        if (ahead < N) {
            int aslot = slot + DEPTH - 1;
            if (aslot >= DEPTH) aslot -= DEPTH;
            copy_row_to_lds<C>(Wq + (size_t)ahead * row_bytes, lds_base + aslot * row_bytes, nchunks, lane);
        }
        const int left = __builtin_amdgcn_readfirstlane((N - 1 - row) / rstride);   // wave-uniform
        wait_rows_ahead<C, DEPTH>(left < DEPTH - 1 ? left : DEPTH - 1);

        const uint8_t* rowbuf = lds_base + slot * row_bytes;
        float acc = 0.0f;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const uint32_t* w = reinterpret_cast<const uint32_t*>(rowbuf + (size_t)pc[s] * kQ80PairBytes);
            uint32_t v[17];
#pragma unroll
            for (int i = 0; i < 17; ++i) v[i] = w[i];
            int sa = 0, sb = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                sa = dot4_i8(__builtin_amdgcn_alignbit(v[i + 1], v[i], 16), act[s].qa[i], sa);   // codes at bytes 2..33
                sb = dot4_i8(v[9 + i], act[s].qb[i], sb);                                         // codes at bytes 36..67
            }
            acc = fmaf((float)sa, half_lo_to_f32(v[0]) * act[s].da, acc);
            acc = fmaf((float)sb, half_hi_to_f32(v[8]) * act[s].db, acc);
        }
        acc = wave_sum_f32(acc);   // wave-uniform
        if (lane == nout) out = acc;
        if (++nout == kWave) {
            Y[out_row0 + (int64_t)lane * rstride] = out;
            nout = 0;
            out_row0 = row + rstride;
        }
        slot = slot + 1 == DEPTH ? 0 : slot + 1;
    }
    if (lane < nout) Y[out_row0 + (int64_t)lane * rstride] = out;
}

hipError_t launch_q8_m1_ldsrow(int K, int depth, const void* Wq, const void* Xq, float* Y, int N, int grid,
                               int block, hipStream_t s) {
    if (!depth) depth = 2;
    if (!block) block = 256;
    if (block > 256) return hipErrorInvalidValue;   // compiled for <= 256 threads
    if (!grid) {
        const int rows_grid = (N + block / kWave - 1) / (block / kWave);
        grid = rows_grid < 2048 ? rows_grid : 2048;
    }
    const size_t row_bytes = (size_t)(K / 32) * 34;
    const size_t lds = (size_t)column_lds_bytes(K) + (size_t)(block / kWave) * depth * row_bytes;
    if (lds > device_max_lds_per_block()) return hipErrorInvalidValue;
    const int C = (int)((row_bytes + 1023) / 1024);
    const int S = (K / 64 + kWave - 1) / kWave;
    const uint8_t* w = (const uint8_t*)Wq;
    const uint8_t* x = (const uint8_t*)Xq;
#define DG_SCD(SS, CC, DD)                                                                              \
    else if (S == SS && C == CC && depth == DD)                                                         \
        hipLaunchKernelGGL((k_q8_m1_ldsrow<SS, CC, DD>), dim3(grid), dim3(block), lds, s, w, x, Y, N, K);
#define DG_SC(SS, CC) DG_SCD(SS, CC, 2) DG_SCD(SS, CC, 3) DG_SCD(SS, CC, 4)
    // C = ceil(34 K / 32768) for the K % 256 == 0 of each S = ceil(K / 4096)
    if (false) {
    }
    DG_SC(1, 1) DG_SC(1, 2) DG_SC(1, 3) DG_SC(1, 4) DG_SC(1, 5)
    DG_SC(2, 5) DG_SC(2, 6) DG_SC(2, 7) DG_SC(2, 8) DG_SC(2, 9)
    DG_SC(3, 9) DG_SC(3, 10) DG_SC(3, 11) DG_SC(3, 12) DG_SC(3, 13)
    DG_SC(4, 14) DG_SC(4, 15) DG_SC(4, 16) DG_SC(4, 17)
    else return hipErrorInvalidValue;
#undef DG_SC
#undef DG_SCD
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_q8_0(const void* Wq, const void* Xq, float* Y, int N, int K, int M,
                            const dg_launch* cfg, hipStream_t s) {
    const int S = (K / 64 + kWave - 1) / kWave;
    int variant = cfg && cfg->variant ? cfg->variant : 0;
    int depth = cfg ? cfg->unroll : 0;
    if (variant == 0) {
        // Measured on MI355X over the decoder shapes, the 70B MLP and M =
        // 1..24: up to four columns stream rows through LDS in 64-pair units
        // while M * ceil(K / 4096) <= 8, and so do up to eight columns of a
        // matrix of more than 512 row tiles and, on matrices of at most 1024
        // rows with rows of one unit, up to twelve columns for K of
        // 2049..4096 and ten below (1024 x 4096 at 9..12 columns: 4.9, 5.1,
        // 5.3 and 5.5 us against 6.0 on the matrix cores, whose 64 row tiles
        // leave most of the chip idle; at K = 2048 the matrix cores win from
        // 11 columns); in between, the matrix cores' parts of K run every
        // CU.  The rest take the matrix cores, with the columns resident in
        // LDS for 9..16 columns of matrices of many row tiles (14336 x 4096
        // at 9..11 columns: 16.7-16.8 us against 16.9-17.0 streaming).
        const bool units_small = N <= 1024 && S == 1 && (M <= 10 || (M <= 12 && K > 2048));
        const bool units_m = M <= 4 || (M <= 8 && (N <= 1024 || N > 8192)) || units_small;
        const bool units_fit = M * S <= 8 || (S == 1 && M <= 12);
        variant = S <= 4 && units_fit && units_m                 ? DG_VARIANT_Q8_UNITS
                  : (N >= 8192 && K <= 4096 && M >= 9 && M <= 16)  ? DG_VARIANT_Q8_MFMA_RES
                                                             : DG_VARIANT_Q8_MFMA;
    }
    if (variant == DG_VARIANT_Q8_UNITS) {
        if (S > 4 || (M * S > 8 && !(S == 1 && M <= 12))) return hipErrorInvalidValue;
        int grid = cfg ? cfg->grid : 0, block = cfg ? cfg->block : 0;
        if (!grid && !block) units_default_grid(N, M, grid, block);
        return launch_q8_units(K, M, depth, Wq, Xq, Y, N, grid, block, s);
    }
    if (variant == DG_VARIANT_Q8_LDSROW) {
        if (M != 1 || S > 4) return hipErrorInvalidValue;
        int grid = cfg ? cfg->grid : 0, block = cfg ? cfg->block : 0;
        if (!grid && !block) m1_default_launch(N, grid, block);
        return launch_q8_m1_ldsrow(K, depth, Wq, Xq, Y, N, grid, block, s);
    }
    if (variant == DG_VARIANT_Q8_MFMA) {
        if (cfg && cfg->block) return hipErrorInvalidValue;   // the configuration fixes the workgroup size
        return launch_q8_mfma(M, cfg ? cfg->unroll : 0, Wq, Xq, Y, N, K, cfg ? cfg->grid : 0, s);
    }
    if (variant == DG_VARIANT_Q8_MFMA_RES) {
        if (cfg && cfg->block) return hipErrorInvalidValue;
        return launch_q8_res(M, cfg ? cfg->unroll : 0, Wq, Xq, Y, N, K, cfg ? cfg->grid : 0, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace dg
