// gemv_q4_0_mfma.hip -- Q4_0 x Q8_1 for 2..24 activation columns on the int8
// matrix cores (the small-batch kernel of "The kernel that waited for itself").
#include "dg_internal.h"
#include "q4_common.h"

namespace dg {
namespace {

using namespace q4;

// ---------------------------------------------------------------------------
// Small-M path on the matrix cores: v_mfma_i32_16x16x32_i8.
//
// For M >= 2 the column loop of the dot4 path makes the kernel VALU-bound
// (every weight block is unpacked once but multiplied M times), which is what
// pushed the mini-GEMM of "The kernel that waited for itself" to 76% of the
// decode step.  The sum over one Q4_0 block is an int8 contraction of length
// 32, exactly the K of v_mfma_i32_16x16x32_i8, so every block keeps its own
// scales:
//   A (16 x 32, int8)  = the q8 codes of 16 activation columns for block b,
//   B (32 x 16, int8)  = the 4-bit codes (0..15) of 16 weight rows for block b,
//   C (16 x 16, int32) = -8 * sum(q8) per column (the offset of q - 8),
//   D = A*B + C        = the exact int32 block sums, then scaled by d4*d8 in fp32.
// The order of the 32 terms inside the instruction is irrelevant (integers);
// each lane supplies A and B bytes for the same 8 k-slots: lane group g = l/16
// carries weights 4g..4g+3 (low nibbles of code dword g) and 16+4g..16+4g+3
// (high nibbles), and the matching activation dwords g and 4+g.  Output lane
// l holds D[4g + r][l % 16]: columns m = 4g + r of weight row l % 16.
//
// Data flow per workgroup (4 waves = RT row tiles of 16 rows x KS parts of K):
//  * each wave copies its 16 weight rows x CB blocks (one chunk) from HBM to a
//    private LDS buffer with global_load_lds_dwordx4 (coalesced 1 KiB per
//    instruction; rows padded to an odd number of 16-byte slots against bank
//    conflicts), the next chunk in flight while the current one is computed;
//  * all 256 threads stage the matching activation chunks in LDS in operand
//    order (A dwords per lane, and per column group the -8*sum(q8) and d8);
//  * the KS partial results of a row tile meet in LDS in the fixed order
//    0..KS-1 (deterministic).
// Every lane of every copy instruction is active (lanes without a slot of the
// chunk re-read the tile's first slot into an unused LDS slot), so a chunk is
// always exactly C vector-memory instructions and the explicit vmcnt waits
// are exact.
// ---------------------------------------------------------------------------
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int CB>
struct MfmaGeom {
    static_assert(CB % 8 == 0, "chunks hold whole 144-byte groups of 8 blocks");
    static constexpr int kSlotsUsed = CB * 18 / 16;        // 16-byte slots of one row's chunk
    static constexpr int kRowSlots = kSlotsUsed + 1;         // odd stride in slots
    static constexpr int kC = (16 * kRowSlots + 63) / 64;    // copy instructions per chunk
    static constexpr int kBufBytes = kC * 1024;              // per wave, per buffer
};

template <int CB, int NT>
struct MfmaActGeom {
    // A operand: [block][tile][lane] x 8 bytes; scales: [block][tile][group] x 32 bytes
    static constexpr int kABytes = CB * NT * 64 * 8;
    static constexpr int kSBytes = CB * NT * 4 * 32;
    static constexpr int kBytes = kABytes + kSBytes;
};

template <int CB, int NT, int KS>
constexpr size_t mfma_lds_bytes() {
    return (size_t)4 * 2 * MfmaGeom<CB>::kBufBytes + (size_t)KS * MfmaActGeom<CB, NT>::kBytes;
}

// Copies 16 rows x cb blocks (starting at block blk0) into buf.  cb <= CB,
// cb % 8 == 0.  Rows past the end of the matrix are clamped to the last row.
template <int CB>
__device__ __forceinline__ void mfma_copy_chunk(const uint8_t* __restrict__ Wq, size_t row_bytes, int n0, int N,
                                                int blk0, int cb, uint8_t* buf, int lane) {
    using G = MfmaGeom<CB>;
    const int slots_used = cb * 18 / 16;
    const uint8_t* safe = Wq + (size_t)(n0 < N ? n0 : N - 1) * row_bytes + (size_t)blk0 * 18;
#pragma unroll
    for (int j = 0; j < G::kC; ++j) {
        const int q = j * kWave + lane;
        const int r = q / G::kRowSlots;
        const int c = q - r * G::kRowSlots;
        const uint8_t* src = safe;
        if (r < 16 && c < slots_used) {
            const int n = n0 + r < N ? n0 + r : N - 1;
            src = Wq + (size_t)n * row_bytes + (size_t)blk0 * 18 + (size_t)c * 16;
        }
        __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(buf + j * 1024), 16, 0, kAuxNonTemporal);
    }
}

// Stages the activation chunks of the KS parts of one iteration: item e of
// part s2 is column m = e / CB, block b = e % CB (consecutive threads read
// consecutive blocks of one column).  Each thread owns kItems items, and all
// of their global loads are issued before any is consumed, so the staging
// costs one L2 round trip rather than one per item.
template <int CB, int NT, int KS>
__device__ __forceinline__ void mfma_stage_acts(const uint8_t* __restrict__ Xq, int nblk, int M, int it,
                                                int nchunks, uint8_t* abase) {
    using A = MfmaActGeom<CB, NT>;
    constexpr int kPerPart = CB * 16 * NT;
    constexpr int kItems = (kPerPart * KS + 255) / 256;
    uint32_t q[kItems][8];
    uint32_t d0[kItems];
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const int e = threadIdx.x + i * 256;
        const int s2 = e / kPerPart;
        const int e2 = e - s2 * kPerPart;
        const int m = e2 / CB;
        const int b = e2 - m * CB;
        const int ch = it * KS + s2;
        const int blk0 = ch * CB;
        const bool ok = e < kPerPart * KS && ch < nchunks && m < M && blk0 + b < nblk;
        d0[i] = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) q[i][j] = 0;
        if (ok) {
            const uint32_t* src = reinterpret_cast<const uint32_t*>(Xq + ((size_t)m * nblk + blk0 + b) * kQ81Bytes);
            d0[i] = src[0];
#pragma unroll
            for (int j = 0; j < 8; ++j) q[i][j] = src[1 + j];
        }
    }
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        const int e = threadIdx.x + i * 256;
        if (e >= kPerPart * KS) continue;
        const int s2 = e / kPerPart;
        const int e2 = e - s2 * kPerPart;
        const int m = e2 / CB;
        const int b = e2 - m * CB;
        uint8_t* abuf = abase + s2 * A::kBytes;
        uint64_t* a64 = reinterpret_cast<uint64_t*>(abuf);
        uint32_t* sc = reinterpret_cast<uint32_t*>(abuf + A::kABytes);
        const float d = half_lo_to_f32(d0[i]);
        const int c = -8 * block_code_sum(q[i]);
        const int t = m >> 4, mm = m & 15, g = mm >> 2, r = mm & 3;
#pragma unroll
        for (int gg = 0; gg < 4; ++gg)
            a64[(b * NT + t) * 64 + gg * 16 + mm] = (uint64_t)q[i][gg] | ((uint64_t)q[i][4 + gg] << 32);
        uint32_t* rec = sc + ((b * NT + t) * 4 + g) * 8;
        rec[r] = (uint32_t)c;
        rec[4 + r] = __builtin_bit_cast(uint32_t, d);
    }
}

template <int CB, int NT, int KS>
__global__ void __launch_bounds__(256)
k_q4_mfma(const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Xq, float* __restrict__ Y,
          int N, int K, int M) {
    using G = MfmaGeom<CB>;
    using A = MfmaActGeom<CB, NT>;
    constexpr int RT = 4 / KS;                 // row tiles per workgroup
    extern __shared__ u32x4 mfma_lds[];
    uint8_t* const lds = reinterpret_cast<uint8_t*>(mfma_lds);
    const int lane = lane_id();
    const int wave = wave_in_block();
    const int tile = wave / KS;                // this wave's row tile
    const int part = wave - tile * KS;         // this wave's part of K
    const int g = lane >> 4, rn = lane & 15;
    const int nblk = K >> 5;
    const size_t row_bytes = (size_t)nblk * 18;
    const int nchunks = (nblk + CB - 1) / CB;
    const int iters = (nchunks + KS - 1) / KS;
    const int n0 = (blockIdx.x * RT + tile) * 16;
    uint8_t* const wbuf = lds + wave * 2 * G::kBufBytes;
    uint8_t* const abase = lds + 4 * 2 * G::kBufBytes;

    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // chunk handled by this wave in iteration it: it*KS + part.  Order inside an
    // iteration: barrier; stage the activations (their loads drain this
    // wave's copy of the current chunk, which is needed now anyway); request
    // the next chunk; barrier; compute while that copy is in flight.
    if (part < nchunks) {
        const int cb = nblk - part * CB < CB ? nblk - part * CB : CB;
        mfma_copy_chunk<CB>(Wq, row_bytes, n0, N, part * CB, cb, wbuf, lane);
    }
    for (int it = 0; it < iters; ++it) {
        const int ch = it * KS + part;
        const int nch = ch + KS;
        const bool have = ch < nchunks;                 // wave-uniform
        const bool ahead = nch < nchunks;               // wave-uniform
        lds_barrier();   // every wave is done reading the previous activation chunks
        mfma_stage_acts<CB, NT, KS>(Xq, nblk, M, it, nchunks, abase);
        if (ahead) {
            const int cbn = nblk - nch * CB < CB ? nblk - nch * CB : CB;
            mfma_copy_chunk<CB>(Wq, row_bytes, n0, N, nch * CB, cbn, wbuf + ((it + 1) & 1) * G::kBufBytes, lane);
        }
        lds_barrier();   // activation chunks staged
        if (ahead) wait_vmcnt<G::kC>();   // the current chunk's copy is complete
        else wait_vmcnt<0>();
        if (have) {
            const int cb = nblk - ch * CB < CB ? nblk - ch * CB : CB;
            const uint8_t* rowp = wbuf + (it & 1) * G::kBufBytes + rn * G::kRowSlots * 16;
            const uint8_t* abuf = abase + part * A::kBytes;
            const uint64_t* a64 = reinterpret_cast<const uint64_t*>(abuf);
            const i32x4* sci = reinterpret_cast<const i32x4*>(abuf + A::kABytes);
#pragma unroll 4
            for (int p = 0; p < (cb >> 1); ++p) {   // cb / 2 is a multiple of 4
                const uint32_t* w = reinterpret_cast<const uint32_t*>(rowp + p * kPairBytes);
                const uint32_t wg0 = w[g], wg1 = w[g + 1], ws0 = w[0], ws4 = w[4], wb = w[5 + g];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t code = h == 0 ? __builtin_amdgcn_alignbit(wg1, wg0, 16) : wb;
                    const float d4 = h == 0 ? half_lo_to_f32(ws0) : half_hi_to_f32(ws4);
                    const long bop = (long)((uint64_t)(code & kNib) | ((uint64_t)((code >> 4) & kNib) << 32));
                    const int b = 2 * p + h;
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const long aop = (long)a64[(b * NT + t) * 64 + lane];
                        const i32x4 cinit = sci[((b * NT + t) * 4 + g) * 2];
                        const f32x4 d8 = __builtin_bit_cast(f32x4, sci[((b * NT + t) * 4 + g) * 2 + 1]);
                        const i32x4 dsum = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, bop, cinit, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[t][r] = fmaf((float)dsum[r], d4 * d8[r], acc[t][r]);
                    }
                }
            }
        }
    }

    // combine the KS parts of each row tile (fixed order) and store
    if constexpr (KS > 1) {
        lds_barrier();   // all activation reads done: reuse the activation area
        float* red = reinterpret_cast<float*>(abase);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[((wave * NT + t) * 4 + r) * 64 + lane] = acc[t][r];
        lds_barrier();
        if (part == 0) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = acc[t][r];
                    for (int s2 = 1; s2 < KS; ++s2) v += red[(((wave + s2) * NT + t) * 4 + r) * 64 + lane];
                    acc[t][r] = v;
                }
        }
    }
    if (part == 0) {
        const int n = n0 + rn;
        if (n < N) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = t * 16 + g * 4 + r;
                    if (m < M) Y[(size_t)m * N + n] = acc[t][r];
                }
        }
    }
}

template <int CB, int NT, int KS>
hipError_t launch_mfma_cfg(const void* Wq, const void* Xq, float* Y, int N, int K, int M, int grid, hipStream_t s) {
    const size_t lds = mfma_lds_bytes<CB, NT, KS>();
    if (lds > device_max_lds_per_block()) return hipErrorInvalidValue;
    constexpr int rows_per_block = 16 * (4 / KS);
    const int g = grid ? grid : (N + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((k_q4_mfma<CB, NT, KS>), dim3(g), dim3(256), lds, s, (const uint8_t*)Wq, (const uint8_t*)Xq,
                       Y, N, K, M);
    return hipGetLastError();
}

}  // namespace

// unroll selects the chunk and K split for sweeps: CB (16 or 32) + 100 * KS (1, 2, 4).
hipError_t launch_q4_mfma(int M, int unroll, const void* Wq, const void* Xq, float* Y, int N, int K, int grid,
                       hipStream_t s) {
    int CB = 16, KS = 1;
    if (unroll) {
        CB = unroll % 100;
        KS = unroll / 100;
    } else {
        const int tiles = (N + 15) / 16;
        KS = tiles >= 1024 ? 1 : (tiles >= 512 ? 2 : 4);
    }
    const int NT = M <= 16 ? 1 : 2;
#define DG_MF(CC, TT, SS) \
    if (CB == CC && NT == TT && KS == SS) return launch_mfma_cfg<CC, TT, SS>(Wq, Xq, Y, N, K, M, grid, s);
    DG_MF(16, 1, 1) DG_MF(16, 1, 2) DG_MF(16, 1, 4) DG_MF(16, 2, 1) DG_MF(16, 2, 2) DG_MF(16, 2, 4)
    DG_MF(32, 1, 1) DG_MF(32, 1, 2) DG_MF(32, 1, 4) DG_MF(32, 2, 1) DG_MF(32, 2, 2)
#undef DG_MF
    return hipErrorInvalidValue;
}

}  // namespace dg
