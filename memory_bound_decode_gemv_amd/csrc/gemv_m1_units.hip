// gemv_m1_units.hip -- quantised GEMV for one activation column (M = 1) with
// the weight rows streamed through LDS in units of 64 block pairs.
//
// The M = 1 decode GEMV of the bitsandbytes issue on 70B 4-bit decode and of
// the Q4_0/Q8_0 harness of "The kernel that waited for itself".  The LDS-row
// kernels give each wave DEPTH buffers of a whole row; for long rows (K of
// 14336 and more, or 8-bit weights) those buffers bound the number of waves
// a CU can hold.  Here the unit of the copy pipeline is 64 block pairs of a
// row -- exactly one pair per lane, the lane's share of the row being one
// pair per unit -- so a wave's buffers no longer grow with K:
//   Q4_0: 64 x 36 bytes = 2304 bytes = 3 copies of 1 KiB per unit;
//   Q8_0: 64 x 68 bytes = 4352 bytes = 5 copies of 1 KiB per unit.
// A wave walks the units (row, s) of its rows in order, with DEPTH - 1 units
// in flight while it computes one.  Every copy instruction has all 64 lanes
// active (lanes past the unit's bytes re-read the unit's first 16 bytes into
// the unused tail of the buffer), so each unit is exactly kC vector-memory
// operations and "at most q * kC outstanding" proves that the unit q steps
// back has landed (loads complete in issue order; the workgroup's copy of
// the activation column is issued before the first unit and the outputs are
// stored after the last wait).
#include "dg_internal.h"
#include "q4_common.h"

namespace dg {
namespace {

using namespace q4;

// A format policy reads one weight block pair of a unit from LDS once and
// adds its products with MC activation columns into acc[0..MC-1] (each
// column summed exactly as with one column alone).
struct UnitsQ4_0 {
    static constexpr int kBlockBytes = 18;
    static constexpr int kPairDwords = 9;
    template <int MC>
    __device__ __forceinline__ static void pairs(const uint32_t* w, const ActPair* a, float* acc) {
        uint32_t v[9];
#pragma unroll
        for (int i = 0; i < 9; ++i) v[i] = w[i];
        WeightPair u;
        unpack_weight_pair(v, u);
#pragma unroll
        for (int m = 0; m < MC; ++m)
            acc[m] = pair_dot(u, a[m].qa, a[m].qb, a[m].da, a[m].db, a[m].ca, a[m].cb, acc[m]);
    }
};

struct UnitsQ8_0 {
    static constexpr int kBlockBytes = 34;
    static constexpr int kPairDwords = 17;
    template <int MC>
    __device__ __forceinline__ static void pairs(const uint32_t* w, const ActPair* a, float* acc) {
        uint32_t v[17];
#pragma unroll
        for (int i = 0; i < 17; ++i) v[i] = w[i];
        uint32_t qa[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) qa[i] = __builtin_amdgcn_alignbit(v[i + 1], v[i], 16);   // codes at bytes 2..33
        const float dwa = half_lo_to_f32(v[0]), dwb = half_hi_to_f32(v[8]);
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            int sa = 0, sb = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                sa = dot4_i8(qa[i], a[m].qa[i], sa);
                sb = dot4_i8(v[9 + i], a[m].qb[i], sb);   // codes at bytes 36..67
            }
            acc[m] = fmaf((float)sa, dwa * a[m].da, acc[m]);
            acc[m] = fmaf((float)sb, dwb * a[m].db, acc[m]);
        }
    }
};

template <class F>
struct UnitGeom {
    static constexpr int kUnitBytes = 64 * 2 * F::kBlockBytes;
    static constexpr int kC = (kUnitBytes + 1023) / 1024;   // copy instructions per unit
    static constexpr int kBufBytes = kC * 1024;
};

// Copies unit s of a row (pairs 64s .. 64s + 63, clipped to the row) into buf.
template <class F>
__device__ __forceinline__ void copy_unit(const uint8_t* __restrict__ row, int s, int npairs, uint8_t* buf,
                                          int lane) {
    using G = UnitGeom<F>;
    const int p0 = s * 64;
    const int pairs = npairs - p0 < 64 ? npairs - p0 : 64;
    const int slots = pairs * 2 * F::kBlockBytes / 16;   // pairs of K % 256 == 0 rows fill whole slots
    const uint8_t* base = row + (size_t)p0 * 2 * F::kBlockBytes;
#pragma unroll
    for (int j = 0; j < G::kC; ++j) {
        const int c = j * kWave + lane;
        const uint8_t* src = base + (size_t)(c < slots ? c : 0) * 16;
        __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(buf + j * 1024), 16, 0, kAuxNonTemporal);
    }
}

template <class F, int S, int MC, int DEPTH>
__global__ void __launch_bounds__(256)
k_units(const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Xq, float* __restrict__ Y, int N, int K) {
    using G = UnitGeom<F>;
    static_assert(DEPTH >= 2 && DEPTH <= 4, "pipeline depth");
    static_assert(G::kC * (DEPTH - 1) <= 63, "wait count exceeds the vmcnt field");
    static_assert(MC >= 1 && (MC * S <= 8 || (S == 1 && MC <= 12)), "activation pairs held in registers");
    extern __shared__ u32x4 lds_units[];
    const int lane = lane_id();
    const int wave = wave_in_block();
    const int wpb = blockDim.x / kWave;
    const int npairs = K >> 6;
    const size_t row_bytes = (size_t)(K >> 5) * F::kBlockBytes;
    const size_t col_bytes = (size_t)(K >> 5) * kQ81Bytes;
    const int col_lds = column_lds_bytes(K);
    const int rstride = gridDim.x * wpb;
    const int row0 = blockIdx.x * wpb + wave;
    uint8_t* const acts = reinterpret_cast<uint8_t*>(lds_units);
    uint8_t* const bufs = acts + MC * col_lds + wave * DEPTH * G::kBufBytes;

    // the workgroup's copy of the activation columns first, then the first units
#pragma unroll
    for (int m = 0; m < MC; ++m) copy_column_to_lds(Xq + m * col_bytes, K, acts + m * col_lds, wave, wpb, lane);

    // issue pointer: the next unit (irow, is) to copy, into slot islot
    int irow = row0, is = 0, islot = 0;
    auto issue = [&]() {
        if (irow < N) {
            copy_unit<F>(Wq + (size_t)irow * row_bytes, is, npairs, bufs + islot * G::kBufBytes, lane);
            islot = islot + 1 == DEPTH ? 0 : islot + 1;
            if (++is == S) { is = 0; irow += rstride; }
        }
    };
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d) issue();

    {   // this wave's column copies have landed once only its issued units can be outstanding
        const int units = row0 < N ? ((N - 1 - row0) / rstride + 1) * S : 0;   // wave-uniform
        wait_ahead<G::kC, DEPTH>(units < DEPTH - 1 ? units : DEPTH - 1);
        lds_barrier();
    }
    if (row0 >= N) return;   // after the barrier: every wave takes part in it

    ActPair act[S][MC];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int p = s * kWave + lane;
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            uint32_t v[18];
            load_act_raw(acts + m * col_lds, p < npairs ? p : npairs - 1, v);
            decode_act_pair(v, p < npairs, act[s][m]);   // past the row: contributes 0
        }
    }

    float out[MC];
#pragma unroll
    for (int m = 0; m < MC; ++m) out[m] = 0.0f;
    int nout = 0;
    int out_row0 = row0;
    int slot = 0;
    for (int row = row0; row < N; row += rstride) {
        // units left after the last one of this row (wave-uniform)
        const int rows_after = __builtin_amdgcn_readfirstlane((N - 1 - row) / rstride);
        float acc[MC];
#pragma unroll
        for (int m = 0; m < MC; ++m) acc[m] = 0.0f;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            issue();
            const int after = rows_after * S + (S - 1 - s);
            wait_ahead<G::kC, DEPTH>(after < DEPTH - 1 ? after : DEPTH - 1);
            const int p = s * kWave + lane;
            const uint32_t* w = reinterpret_cast<const uint32_t*>(bufs + slot * G::kBufBytes) +
                                (p < npairs ? lane : 0) * F::kPairDwords;
            F::template pairs<MC>(w, act[s], acc);
            slot = slot + 1 == DEPTH ? 0 : slot + 1;
        }
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            const float r = wave_sum_f32(acc[m]);   // wave-uniform
            if (lane == nout) out[m] = r;
        }
        if (++nout == kWave) {
#pragma unroll
            for (int m = 0; m < MC; ++m) Y[(int64_t)m * N + out_row0 + (int64_t)lane * rstride] = out[m];
            nout = 0;
            out_row0 = row + rstride;
        }
    }
    if (lane < nout) {
#pragma unroll
        for (int m = 0; m < MC; ++m) Y[(int64_t)m * N + out_row0 + (int64_t)lane * rstride] = out[m];
    }
}

template <class F>
hipError_t launch_units(int K, int M, int depth, const void* Wq, const void* Xq, float* Y, int N, int grid, int block,
                        hipStream_t s) {
    using G = UnitGeom<F>;
    if (!block) block = 256;
    if (block > 256) return hipErrorInvalidValue;   // compiled for <= 256 threads
    if (!grid) {
        const int rows_grid = (N + block / kWave - 1) / (block / kWave);
        grid = rows_grid < 2048 ? rows_grid : 2048;
    }
    const int S = (K / 64 + kWave - 1) / kWave;
    const size_t cols = (size_t)M * column_lds_bytes(K), per_depth = (size_t)(block / kWave) * G::kBufBytes;
    if (!depth) {
        // Measured on MI355X: one column keeps two units in flight when a row
        // is one unit and three otherwise; several columns keep two, or three
        // for rows of three units and more when two workgroups still fit a CU.
        if (M == 1) depth = S == 1 ? 2 : 3;
        else depth = S >= 3 && cols + 3 * per_depth <= 80 * 1024 ? 3 : 2;
    }
    const size_t lds = cols + depth * per_depth;
    if (lds > device_max_lds_per_block()) return hipErrorInvalidValue;
    const uint8_t* w = (const uint8_t*)Wq;
    const uint8_t* x = (const uint8_t*)Xq;
#define DG_SMD(SS, MM, DD)                                                                                 \
    if (S == SS && M == MM && depth == DD) {                                                               \
        hipLaunchKernelGGL((k_units<F, SS, MM, DD>), dim3(grid), dim3(block), lds, s, w, x, Y, N, K);  \
        return hipGetLastError();                                                                          \
    }
#define DG_SM(SS, MM) DG_SMD(SS, MM, 2) DG_SMD(SS, MM, 3) DG_SMD(SS, MM, 4)
    DG_SM(1, 1) DG_SM(1, 2) DG_SM(1, 3) DG_SM(1, 4) DG_SM(1, 5) DG_SM(1, 6) DG_SM(1, 7) DG_SM(1, 8)
    if constexpr (F::kBlockBytes == 34) {   // 8-bit weights: 9..12 columns of rows of one unit
        DG_SM(1, 9) DG_SM(1, 10) DG_SM(1, 11) DG_SM(1, 12)
    }
    DG_SM(2, 1) DG_SM(2, 2) DG_SM(2, 3) DG_SM(2, 4)
    DG_SM(3, 1) DG_SM(3, 2)
    DG_SM(4, 1) DG_SM(4, 2)
#undef DG_SM
#undef DG_SMD
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_q4_units(int K, int M, int depth, const void* Wq, const void* Xq, float* Y, int N, int grid,
                           int block, hipStream_t s) {
    return launch_units<UnitsQ4_0>(K, M, depth, Wq, Xq, Y, N, grid, block, s);
}

hipError_t launch_q8_units(int K, int M, int depth, const void* Wq, const void* Xq, float* Y, int N, int grid,
                           int block, hipStream_t s) {
    return launch_units<UnitsQ8_0>(K, M, depth, Wq, Xq, Y, N, grid, block, s);
}

}  // namespace dg
