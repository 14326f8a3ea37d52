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

struct UnitsQ4_0 {
    static constexpr int kBlockBytes = 18;
    static constexpr int kPairDwords = 9;
    __device__ __forceinline__ static float pair(const uint32_t* w, const ActPair& a, float acc) {
        uint32_t v[9];
#pragma unroll
        for (int i = 0; i < 9; ++i) v[i] = w[i];
        WeightPair u;
        unpack_weight_pair(v, u);
        return pair_dot(u, a.qa, a.qb, a.da, a.db, a.ca, a.cb, acc);
    }
};

struct UnitsQ8_0 {
    static constexpr int kBlockBytes = 34;
    static constexpr int kPairDwords = 17;
    __device__ __forceinline__ static float pair(const uint32_t* w, const ActPair& a, float acc) {
        uint32_t v[17];
#pragma unroll
        for (int i = 0; i < 17; ++i) v[i] = w[i];
        int sa = 0, sb = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            sa = dot4_i8(__builtin_amdgcn_alignbit(v[i + 1], v[i], 16), a.qa[i], sa);   // codes at bytes 2..33
            sb = dot4_i8(v[9 + i], a.qb[i], sb);                                         // codes at bytes 36..67
        }
        acc = fmaf((float)sa, half_lo_to_f32(v[0]) * a.da, acc);
        return fmaf((float)sb, half_hi_to_f32(v[8]) * a.db, acc);
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

template <class F, int S, int DEPTH>
__global__ void __launch_bounds__(256)
k_m1_units(const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Xq, float* __restrict__ Y, int N, int K) {
    using G = UnitGeom<F>;
    static_assert(DEPTH >= 2 && DEPTH <= 4, "pipeline depth");
    static_assert(G::kC * (DEPTH - 1) <= 63, "wait count exceeds the vmcnt field");
    extern __shared__ u32x4 lds_units[];
    const int lane = lane_id();
    const int wave = wave_in_block();
    const int wpb = blockDim.x / kWave;
    const int npairs = K >> 6;
    const size_t row_bytes = (size_t)(K >> 5) * F::kBlockBytes;
    const int rstride = gridDim.x * wpb;
    const int row0 = blockIdx.x * wpb + wave;
    uint8_t* const acts = reinterpret_cast<uint8_t*>(lds_units);
    uint8_t* const bufs = acts + column_lds_bytes(K) + wave * DEPTH * G::kBufBytes;

    // the workgroup's copy of the activation column first, then the first units
    copy_column_to_lds(Xq, K, acts, wave, wpb, lane);

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

    ActPair act[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int p = s * kWave + lane;
        uint32_t v[18];
        load_act_raw(acts, p < npairs ? p : npairs - 1, v);
        decode_act_pair(v, p < npairs, act[s]);   // past the row: contributes 0
    }

    float out = 0.0f;
    int nout = 0;
    int out_row0 = row0;
    int slot = 0;
    for (int row = row0; row < N; row += rstride) {
        // units left after the last one of this row (wave-uniform)
        const int rows_after = __builtin_amdgcn_readfirstlane((N - 1 - row) / rstride);
        float acc = 0.0f;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            issue();
            const int after = rows_after * S + (S - 1 - s);
            wait_ahead<G::kC, DEPTH>(after < DEPTH - 1 ? after : DEPTH - 1);
            const int p = s * kWave + lane;
            const uint32_t* w = reinterpret_cast<const uint32_t*>(bufs + slot * G::kBufBytes) +
                                (p < npairs ? lane : 0) * F::kPairDwords;
            acc = F::pair(w, act[s], acc);
            slot = slot + 1 == DEPTH ? 0 : slot + 1;
        }
        acc = wave_sum_f32(acc);   // wave-uniform
        if (lane == nout) out = acc;
        if (++nout == kWave) {
            Y[out_row0 + (int64_t)lane * rstride] = out;
            nout = 0;
            out_row0 = row + rstride;
        }
    }
    if (lane < nout) Y[out_row0 + (int64_t)lane * rstride] = out;
}

template <class F>
hipError_t launch_units(int K, int depth, const void* Wq, const void* Xq, float* Y, int N, int grid, int block,
                        hipStream_t s) {
    using G = UnitGeom<F>;
    if (!depth) depth = 3;
    if (!block) block = 256;
    if (block > 256) return hipErrorInvalidValue;   // compiled for <= 256 threads
    if (!grid) {
        const int rows_grid = (N + block / kWave - 1) / (block / kWave);
        grid = rows_grid < 2048 ? rows_grid : 2048;
    }
    const size_t lds = (size_t)column_lds_bytes(K) + (size_t)(block / kWave) * depth * G::kBufBytes;
    if (lds > device_max_lds_per_block()) return hipErrorInvalidValue;
    const int S = (K / 64 + kWave - 1) / kWave;
    const uint8_t* w = (const uint8_t*)Wq;
    const uint8_t* x = (const uint8_t*)Xq;
#define DG_SD(SS, DD)                                                                                    \
    if (S == SS && depth == DD) {                                                                        \
        hipLaunchKernelGGL((k_m1_units<F, SS, DD>), dim3(grid), dim3(block), lds, s, w, x, Y, N, K);    \
        return hipGetLastError();                                                                        \
    }
#define DG_S(SS) DG_SD(SS, 2) DG_SD(SS, 3) DG_SD(SS, 4)
    DG_S(1) DG_S(2) DG_S(3) DG_S(4)
#undef DG_S
#undef DG_SD
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_q4_m1_units(int K, int depth, const void* Wq, const void* Xq, float* Y, int N, int grid,
                              int block, hipStream_t s) {
    return launch_units<UnitsQ4_0>(K, depth, Wq, Xq, Y, N, grid, block, s);
}

hipError_t launch_q8_m1_units(int K, int depth, const void* Wq, const void* Xq, float* Y, int N, int grid,
                              int block, hipStream_t s) {
    return launch_units<UnitsQ8_0>(K, depth, Wq, Xq, Y, N, grid, block, s);
}

}  // namespace dg
