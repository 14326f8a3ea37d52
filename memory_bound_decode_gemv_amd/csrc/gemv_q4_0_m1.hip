// gemv_q4_0_m1.hip -- Q4_0 x Q8_1 decode GEMV for one activation column
// (M = 1), the 4-bit batch-1 GEMV of the bitsandbytes issue on 70B decode
// (8192 x 28672 MLP shape) and of the Q4_0/Q8_1 harness in "The kernel that
// waited for itself".
#include "dg_internal.h"
#include "q4_common.h"
#include "q81_rules.h"

namespace dg {
namespace {

using namespace q4;

// ---------------------------------------------------------------------------
// M = 1 with coalesced weight loads through LDS.  A packed Q4_0 row is a
// contiguous, 16-byte aligned run of 18-byte blocks; read 16 bytes per lane at
// a 36-byte lane stride (the block pairs), every cache line is touched by
// three separate load instructions.  Here the wave instead copies the row
// into its own LDS buffer with global_load_lds_dwordx4 (64 lanes x 16 B = one
// contiguous KiB per instruction, straight into LDS without passing through
// VGPRs; non-temporal), then each lane reads its block pairs back with
// ds_read2_b32 at a 9-dword lane stride (9 is odd: no bank conflicts).  DEPTH
// row buffers per wave keep DEPTH - 1 rows in flight while one is computed.
//
// The compiler does not track these LDS writes, so the waits are explicit.
// Loads complete in issue order, and each of the C loads of a row has at least
// one active lane; so once the wave has issued the loads of q further rows
// after row r, "at most q*C vector-memory operations outstanding" implies that
// row r has arrived (stores only make the wait longer).  C = ceil(row bytes /
// 1 KiB) is a template parameter because the wait count is an immediate.
// ---------------------------------------------------------------------------
//
// FX (fp32 activations): the workgroup quantises the column itself instead of
// copying Q8_1 blocks.  The first DEPTH - 1 rows' copies are issued first, so
// their latency overlaps the quantisation; each lane then takes whole
// 32-element blocks of x (16-byte loads), applies the Q8_1 rules of
// q81_rules.h (the standalone quantiser's, byte for byte) and writes the
// 36-byte block into the LDS column; workgroup 0 also stores the blocks to
// Xq_out when it is given.
template <int S, int C, int DEPTH, bool FX>
__global__ void __launch_bounds__(256)
k_q4_m1_ldsrow(const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Xq, const float* __restrict__ xf,
               uint8_t* __restrict__ Xq_out, float* __restrict__ Y, int N, int K) {
    static_assert(DEPTH >= 2 && DEPTH <= 4, "pipeline depth");
    extern __shared__ u32x4 lds_rows[];
    const int lane = lane_id();
    const int wave = wave_in_block();
    const int wpb = blockDim.x / kWave;
    const int npairs = K >> 6;
    const int row_bytes = (K >> 5) * 18;
    const int nchunks = row_bytes >> 4;
    const int rstride = gridDim.x * wpb;
    const int row0 = blockIdx.x * wpb + wave;
    // Byte offsets of the column and the wave's buffers; addresses are always
    // formed from the __shared__ array itself, so that they stay LDS
    // addresses (ds_read) rather than generic ones (flat_load).
    uint8_t* const acts = reinterpret_cast<uint8_t*>(lds_rows);
    uint8_t* const lds_base = acts + column_lds_bytes(K) + wave * DEPTH * row_bytes;

    if constexpr (FX) {
        // the first DEPTH - 1 rows' copies, then the column quantised into LDS
#pragma unroll
        for (int d = 0; d < DEPTH - 1; ++d) {
            const int r = row0 + d * rstride;
            if (r < N) copy_row_to_lds<C>(Wq + (size_t)r * row_bytes, lds_base + d * row_bytes, nchunks, lane);
        }
        const int nblk = K >> 5;
        const bool store = Xq_out != nullptr && blockIdx.x == 0;
        for (int b = wave * kWave + lane; b < nblk; b += wpb * kWave) {
            uint32_t blk[9];
            quantize_q81_block(xf + (size_t)b * 32, blk);
            uint32_t* dst = reinterpret_cast<uint32_t*>(acts + b * kQ81Bytes);
#pragma unroll
            for (int i = 0; i < 9; ++i) dst[i] = blk[i];
            if (store) {
                uint32_t* g = reinterpret_cast<uint32_t*>(Xq_out + (size_t)b * kQ81Bytes);
#pragma unroll
                for (int i = 0; i < 9; ++i) g[i] = blk[i];
            }
        }
        lds_barrier();   // every wave's blocks are in the column
    } else {
        // the workgroup's copy of the activation column first, then the copies of
        // the first DEPTH - 1 rows (rows row0 + i*rstride for i = 0, 1, ...)
        copy_column_to_lds(Xq, K, acts, wave, wpb, lane);
#pragma unroll
        for (int d = 0; d < DEPTH - 1; ++d) {
            const int r = row0 + d * rstride;
            if (r < N) copy_row_to_lds<C>(Wq + (size_t)r * row_bytes, lds_base + d * row_bytes, nchunks, lane);
        }
        // this wave's column copies have landed once only its issued rows can be outstanding
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

    // Results are held back and stored 64 rows at a time (lane i holds the
    // i-th row of the batch): a store between two rows' loads would count
    // in vmcnt ahead of the next row's copies, so every row wait would also
    // wait for the previous row's write to be acknowledged.
    float out = 0.0f;
    int nout = 0;
    int out_row0 = row0;

    int slot = 0;   // buffer of the current row
    for (int row = row0; row < N; row += rstride) {
        const int ahead = row + (DEPTH - 1) * rstride;
        if (ahead < N) {
            int aslot = slot + DEPTH - 1;
            if (aslot >= DEPTH) aslot -= DEPTH;
            copy_row_to_lds<C>(Wq + (size_t)ahead * row_bytes, lds_base + aslot * row_bytes, nchunks, lane);
        }
        // rows requested after this one: min(DEPTH - 1, rows left after it)
        const int left = __builtin_amdgcn_readfirstlane((N - 1 - row) / rstride);   // wave-uniform
        wait_rows_ahead<C, DEPTH>(left < DEPTH - 1 ? left : DEPTH - 1);

        const uint8_t* rowbuf = lds_base + slot * row_bytes;
        float acc = 0.0f;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            uint32_t w[9];
            read_pair_lds(rowbuf, pc[s], w);
            WeightPair u;
            unpack_weight_pair(w, u);
            acc = pair_dot(u, act[s].qa, act[s].qb, act[s].da, act[s].db, act[s].ca, act[s].cb, acc);
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

}  // namespace

// depth, grid and block 0 select the defaults.  Measured on MI355X at
// 28672 x 8192: two row buffers per wave and at most 2048 workgroups of four
// waves (a few rows per wave) read fastest.
hipError_t launch_q4_m1_ldsrow(int K, int depth, const void* Wq, const void* Xq, float* Y, int N, int grid,
                               int block, hipStream_t s, const float* xf, void* Xq_out) {
    if (!depth) depth = 2;
    if (!block) block = 256;
    if (block > 256) return hipErrorInvalidValue;   // compiled for <= 256 threads
    if (!grid) {
        const int rows_grid = (N + block / kWave - 1) / (block / kWave);
        grid = rows_grid < 2048 ? rows_grid : 2048;
    }
    const uint8_t* w = (const uint8_t*)Wq;
    const uint8_t* x = (const uint8_t*)Xq;
    const size_t row_bytes = (size_t)(K / 32) * 18;
    const size_t lds = (size_t)column_lds_bytes(K) + (size_t)(block / kWave) * depth * row_bytes;
    if (lds > device_max_lds_per_block()) return hipErrorInvalidValue;
    const int C = (int)((row_bytes + 1023) / 1024);
    const int S = (K / 64 + kWave - 1) / kWave;
    uint8_t* xo = (uint8_t*)Xq_out;
#define DG_SCD(SS, CC, DD)                                                                                   \
    else if (S == SS && C == CC && depth == DD) {                                                            \
        if (xf)                                                                                              \
            hipLaunchKernelGGL((k_q4_m1_ldsrow<SS, CC, DD, true>), dim3(grid), dim3(block), lds, s, w, x, xf,   \
                               xo, Y, N, K);                                                                 \
        else                                                                                                 \
            hipLaunchKernelGGL((k_q4_m1_ldsrow<SS, CC, DD, false>), dim3(grid), dim3(block), lds, s, w, x, xf,  \
                               xo, Y, N, K);                                                                 \
    }
#define DG_SC(SS, CC) DG_SCD(SS, CC, 2) DG_SCD(SS, CC, 3) DG_SCD(SS, CC, 4)
    if (false) {
    }
    DG_SC(1, 1) DG_SC(1, 2) DG_SC(1, 3) DG_SC(2, 3) DG_SC(2, 4) DG_SC(2, 5) DG_SC(3, 5) DG_SC(3, 6) DG_SC(3, 7)
    DG_SC(4, 7) DG_SC(4, 8) DG_SC(4, 9)
    else return hipErrorInvalidValue;
#undef DG_SC
#undef DG_SCD
    return hipGetLastError();
}

}  // namespace dg
