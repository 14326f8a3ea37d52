// gemv_q4_0_mfma.hip -- Q4_0 x Q8_1 for 2..24 activation columns on the int8
// matrix cores (the small-batch kernel of "The kernel that waited for itself").
#include "dg_internal.h"
#include "mfma_formats.h"

namespace dg {
namespace {

using namespace q4;
using namespace mfma;

// ---------------------------------------------------------------------------
// Small-M path on the matrix cores: v_mfma_i32_16x16x32_i8.
//
// For M >= 2 the column loop of the dot4 path makes the kernel VALU-bound
// (every weight block is unpacked once but multiplied M times), which is what
// pushed the mini-GEMM of "The kernel that waited for itself" to 76% of the
// decode step.  The sum over one Q4_0 block is an int8 contraction of length
// 32, exactly the K of v_mfma_i32_16x16x32_i8, so every block keeps its own
// scales.  Per block b and per tile of 16 weight rows x 16 columns:
//   A (16 x 32, int8)  = the q8 codes of 16 activation columns,
//   B (32 x 16, int8)  = the 4-bit codes (0..15) of 16 weight rows,
//   D0 = A * (-8)      = -8 * sum(q8) per column (a second MFMA against a
//                        constant operand: the offset of q - 8, exact),
//   D  = A * B + D0    = the exact int32 block sums, scaled by d4 * d8 in fp32,
//   S  = d8 (x) d4     = those 16 x 16 scale products, from one f16 MFMA
//                        of the raw binary16 scales (exact in fp32).
// The order of the 32 terms inside the instruction is irrelevant (integers);
// each lane supplies A and B bytes for the same 8 k-slots: lane group g = l/16
// carries weights 4g..4g+3 (low nibbles of code dword g) and 16+4g..16+4g+3
// (high nibbles), and the matching activation code dwords g and 4+g.  Output
// lane l holds D[4g + r][l % 16]: column m = 4g + r of weight row l % 16.
//
// Data flow.  A workgroup of W = RT * KS waves (4, 8 or 16) covers RT row
// tiles, each split into KS parts of K, so that small matrices still give
// every CU several waves; K is walked in chunks of CB blocks, iteration `it`
// giving part p the chunk it * KS + p.  Everything reaches LDS by
// global_load_lds_dwordx4 (1 KiB of contiguous LDS per instruction, no VGPRs):
//  * each wave copies its 16 rows x CB blocks of weights (non-temporal: read
//    once) into a private buffer, rows padded to an odd number of 16-byte
//    slots so that the 16 rows of a lane group fall in different banks;
//  * the W waves together copy the raw Q8_1 blocks of the iteration's KS
//    activation chunks for MP >= M columns (MP = 4, 8, 16 or 32; 36 bytes per
//    block, column spans padded to an odd number of slots) into a buffer
//    shared by the workgroup; every weight row tile reuses it, and L2 serves
//    it to every workgroup.  With MP < 16 the MFMA rows past MP re-read
//    columns (their results are discarded).  With one row tile per
//    workgroup (RT = 1) nothing is shared: each wave copies its own part's
//    columns into a region of its own and waits only for its own copies, so
//    the waves of a workgroup drift apart and overlap one another's loads
//    and arithmetic.
// DEPTH buffers of each kind keep DEPTH - 1 iterations in flight while one is
// computed.  No global load goes through VGPRs inside the loop, so the only
// vector-memory operations a wave has outstanding are its own copies, which
// complete in issue order; each wave issues exactly kCw + kCa copy
// instructions per iteration (lanes without a slot of the data re-read a
// valid address next to the real data into a slot nobody reads, so that no
// line becomes a hot spot for the whole chip), so "at most q * (kCw + kCa) outstanding"
// proves that the iteration q steps back has landed, and (shared columns
// only) a barrier after each wave's own wait makes the activation chunk
// complete for all.
// Outputs: the KS partial results of a row tile meet in LDS and are added in
// the fixed order 0..KS-1 (deterministic).
// ---------------------------------------------------------------------------
template <class WF, int CB, int MP, int RT, int KS>
struct MfmaGeom {
    static_assert(CB % 8 == 0, "chunks hold whole 144-byte groups of 8 blocks");
    static_assert(MP == 4 || MP == 8 || MP == 16 || MP == 17 || MP == 24 || MP == 32, "padded column count");
    static constexpr int kW = RT * KS;                           // waves per workgroup
    static_assert(kW == 4 || kW == 8 || kW == 12 || kW == 16, "4, 8, 12 or 16 waves");
    static constexpr int kNT = (MP + 15) / 16;                   // 16-column MFMA tiles
    // weights: 16 rows x CB blocks
    static constexpr int kWSlotsUsed = CB * WF::kBlockBytes / 16;
    static constexpr int kWRowSlots = kWSlotsUsed | 1;           // odd stride in slots
    static constexpr int kCw = (16 * kWRowSlots + 63) / 64;      // copy instructions per wave
    static constexpr int kWBufBytes = kCw * 1024;                // per wave, per buffer
    // activations: KS parts x MP columns x CB blocks of 36 bytes
    static constexpr int kASlotsUsed = CB * 36 / 16;
    static constexpr int kAColSlots = kASlotsUsed | 1;           // odd stride in slots
    static constexpr int kAPartSlots = MP * kAColSlots;
    static constexpr int kASlots = KS * kAPartSlots;
    // One row tile per workgroup (RT = 1): each wave copies its own part's
    // columns into a private region, so no wave waits for another inside the
    // loop.  Otherwise the W waves share the copies of the KS parts.
    static constexpr bool kPriv = RT == 1;
    static constexpr int kCa = kPriv ? (kAPartSlots + 63) / 64                    // copy instructions
                                     : (kASlots + kW * 64 - 1) / (kW * 64);      // per wave
    static constexpr int kAPartBytes = kPriv ? kCa * 1024 : kAPartSlots * 16;   // part stride
    static constexpr int kABufBytes = kCa * kW * 1024;           // per workgroup, per buffer
    static constexpr int kCopies = kCw + kCa;                    // per wave, per iteration
    static constexpr int kStageBytes = kW * kWBufBytes + kABufBytes;
};

// LDS: DEPTH stages; after the loop they hold the KS partial sums.
template <class WF, int CB, int MP, int RT, int KS, int DEPTH>
constexpr size_t mfma_lds_bytes() {
    using G = MfmaGeom<WF, CB, MP, RT, KS>;
    const size_t main = (size_t)DEPTH * G::kStageBytes;
    const size_t red = (size_t)G::kW * (G::kNT * 4 + (MP == 17)) * 64 * 4;   // partial sums of the KS parts
    return main > red ? main : red;
}

// Copy addresses.  A weight copy of chunk ch is a scalar base (row tile n0,
// block ch * CB) plus a per-lane offset woff[j] fixed for the row tile: lane
// slot q = j * 64 + lane is 16-byte slot c of row r of the tile (q = r *
// kWRowSlots + c), with rows past N and slots past the chunk clamped onto
// real data (that the compute skips).  An activation copy of iteration it is
// a scalar base (block it * KS * CB) plus a per-lane offset aoff[j] fixed for
// the launch: slot s = (wave * kCa + j) * 64 + lane of the shared buffer is
// part p, column m, slot c (clamped the same way; with private parts, slot
// j * 64 + lane of the wave's own part).  Chunks hold whole groups
// of 8 blocks (K % 256 == 0) and every offset fits 32 bits (K <= 2^26), so the
// loop issues each copy with no address arithmetic.
template <class WF, int CB, int MP, int RT, int KS>
__device__ __forceinline__ void weight_offsets(uint32_t row_bytes, int rmax, int lane,
                                               uint32_t (&woff)[MfmaGeom<WF, CB, MP, RT, KS>::kCw]) {
    using G = MfmaGeom<WF, CB, MP, RT, KS>;
#pragma unroll
    for (int j = 0; j < G::kCw; ++j) {
        const int q = j * kWave + lane;
        const int r = q / G::kWRowSlots;
        const int c = q - r * G::kWRowSlots;
        int rr = r < 16 ? r : 15;
        rr = rr < rmax ? rr : rmax;
        const int cc = c < G::kWSlotsUsed ? c : G::kWSlotsUsed - 1;
        woff[j] = (uint32_t)rr * row_bytes + (uint32_t)cc * 16;
    }
}

template <class WF, int CB, int MP, int RT, int KS>
__device__ __forceinline__ void act_offsets(int nblk, int M, int wave, int lane,
                                            uint32_t (&aoff)[MfmaGeom<WF, CB, MP, RT, KS>::kCa]) {
    using G = MfmaGeom<WF, CB, MP, RT, KS>;
#pragma unroll
    for (int j = 0; j < G::kCa; ++j) {
        const int s = (wave * G::kCa + j) * kWave + lane;
        int p = G::kPriv ? wave : s / G::kAPartSlots;
        const int e = G::kPriv ? j * kWave + lane : s - p * G::kAPartSlots;
        const int m = e / G::kAColSlots;
        const int c = e - m * G::kAColSlots;
        p = p < KS ? p : KS - 1;
        const int mc = m < M ? m : M - 1;
        const int cc = c < G::kASlotsUsed ? c : G::kASlotsUsed - 1;
        aoff[j] = ((uint32_t)mc * nblk + (uint32_t)p * CB) * kQ81Bytes + (uint32_t)cc * 16;
    }
}

// This wave's weight copies of chunk ch (past the last chunk: the last one
// again, which the compute skips).
template <class WF, int CB, int L>
__device__ __forceinline__ void copy_weights(const uint8_t* __restrict__ Wq, size_t row_bytes, int n0c, int nchunks,
                                             int ch, const uint32_t* woff, uint8_t* buf) {
    const int chc = ch < nchunks ? ch : nchunks - 1;   // wave-uniform
    const uint8_t* src = Wq + (size_t)n0c * row_bytes + (size_t)chc * (CB * WF::kBlockBytes);
#pragma unroll
    for (int j = 0; j < L; ++j)
        __builtin_amdgcn_global_load_lds(src + woff[j], (lds_void_t*)(buf + j * 1024), 16, 0, kAuxNonTemporal);
}

// This wave's share (instructions wave*kCa .. wave*kCa + kCa - 1) of the
// activation copies of iteration it.  In an iteration with fewer than KS
// chunks left, the parts without a chunk (never read) re-read their chunk of
// the iteration before, or, in a first and only iteration, the last 16 bytes
// of the columns.
template <int CB, int KS, int L>
__device__ __forceinline__ void copy_acts(const uint8_t* __restrict__ Xq, uint32_t xlast, int nchunks, int it,
                                          int wave, const uint32_t* aoff, uint8_t* abuf) {
    constexpr uint32_t kIterBytes = KS * CB * kQ81Bytes;
    const uint32_t base = (uint32_t)it * kIterBytes;
    if ((it + 1) * KS <= nchunks) {   // wave-uniform
#pragma unroll
        for (int j = 0; j < L; ++j)
            __builtin_amdgcn_global_load_lds(Xq + base + aoff[j], (lds_void_t*)(abuf + (wave * L + j) * 1024),
                                             16, 0, 0);
    } else {
#pragma unroll
        for (int j = 0; j < L; ++j) {
            uint32_t o = base + aoff[j];
            if (o > xlast) o = it > 0 ? o - kIterBytes : xlast;
            __builtin_amdgcn_global_load_lds(Xq + o, (lds_void_t*)(abuf + (wave * L + j) * 1024), 16, 0, 0);
        }
    }
}

// Waits until at most q iterations' copies of this wave are outstanding
// (q <= DEPTH - 1; the count is an immediate, so each q has its own wait).
template <int COPIES, int DEPTH>
__device__ __forceinline__ void wait_iterations_ahead(int q) {
    if (DEPTH == 1 || q == 0) wait_vmcnt<0>();
    else if (q == 1) wait_vmcnt<COPIES>();
    else if (DEPTH > 3 && q == 2) wait_vmcnt<(DEPTH > 3 ? 2 * COPIES : 0)>();
    else if (DEPTH > 4 && q == 3) wait_vmcnt<(DEPTH > 4 ? 3 * COPIES : 0)>();
    else wait_vmcnt<(DEPTH > 1 ? (DEPTH - 1) * COPIES : 0)>();
}

template <class WF, int CB, int MP, int RT, int KS, int DEPTH>
__global__ void __launch_bounds__(64 * RT * KS)
k_qmfma(const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Xq, float* __restrict__ Y,
        int N, int K, int M) {
    using G = MfmaGeom<WF, CB, MP, RT, KS>;
    constexpr bool TAIL = MP == 17;                // column 16 on the vector unit (below)
    constexpr int NT = TAIL ? 1 : G::kNT;          // 16-column matrix-core tiles
    constexpr int GB = RT * KS >= 12 ? 4 : 8;   // blocks per operand group
    static_assert(DEPTH >= 1 && DEPTH <= 5, "pipeline depth");
    static_assert(G::kCopies * (DEPTH - 1) <= 63, "wait count exceeds the vmcnt field");
    extern __shared__ u32x4 mfma_lds[];
    uint8_t* const lds = reinterpret_cast<uint8_t*>(mfma_lds);
    const int lane = lane_id();
    const int wave = wave_in_block();
    const int tile = wave / KS;                // this wave's row tile in the group
    const int part = wave - tile * KS;         // this wave's part of K
    const int g = lane >> 4, rn = lane & 15;
    const int nblk = K >> 5;
    const size_t row_bytes = (size_t)nblk * WF::kBlockBytes;
    const int nchunks = (nblk + CB - 1) / CB;
    const int iters = (nchunks + KS - 1) / KS;
    const int ngroups = (N + 16 * RT - 1) / (16 * RT);
    // A-operand column of this lane in column tile t: 16t + rn, or, for the
    // MFMA rows past MP (MP = 4, 8, 24), a column of the same tile re-read
    // (16t + rn % (MP - 16t)); those results are dropped
    auto acol = [&](int t) { return 16 * t + rn < MP ? 16 * t + rn : 16 * t + rn % (MP - 16 * t); };
    auto wbuf = [&](int d) { return lds + d * G::kStageBytes + wave * G::kWBufBytes; };
    auto abuf = [&](int d) { return lds + d * G::kStageBytes + G::kW * G::kWBufBytes; };
    const uint32_t dwidth = g == 0 ? 16u : 0u;   // lane group 0 feeds d4 to k-slot 0 of the scale products

    const uint32_t xlast = (uint32_t)M * nblk * kQ81Bytes - 16;   // the columns' last 16 bytes
    uint32_t aoff[G::kCa];
    act_offsets<WF, CB, MP, RT, KS>(nblk, M, wave, lane, aoff);

    for (int grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {   // workgroup-uniform
        const int n0 = (grp * RT + tile) * 16;
        const int n0c = n0 < N ? n0 : N - 1;   // tiles past N re-read row N - 1
        uint32_t woff[G::kCw];
        weight_offsets<WF, CB, MP, RT, KS>((uint32_t)row_bytes, N - 1 - n0c, lane, woff);
        lds_barrier();   // the previous group's reads of every buffer are done
#pragma unroll
        for (int d = 0; d < DEPTH - 1; ++d)
            if (d < iters) {
                copy_weights<WF, CB, G::kCw>(Wq, row_bytes, n0c, nchunks, d * KS + part, woff, wbuf(d));
                copy_acts<CB, KS, G::kCa>(Xq, xlast, nchunks, d, wave, aoff, abuf(d));
            }

        f32x4 acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        float tacc = 0.0f;   // the 17th column (TAIL): this lane's share of row rn

        int slot = 0;
        for (int it = 0; it < iters; ++it) {
            // shared columns: every wave is done with the buffer the next
            // copies overwrite (private buffers: the wave's own reads of it
            // have returned, since their results were used)
            if constexpr (!G::kPriv) lds_barrier();
            const int ahead = it + DEPTH - 1;
            if (ahead < iters) {
                int aslot = slot + DEPTH - 1;
                if (aslot >= DEPTH) aslot -= DEPTH;
                copy_weights<WF, CB, G::kCw>(Wq, row_bytes, n0c, nchunks, ahead * KS + part, woff, wbuf(aslot));
                copy_acts<CB, KS, G::kCa>(Xq, xlast, nchunks, ahead, wave, aoff, abuf(aslot));
            }
            const int left = iters - 1 - it;
            wait_iterations_ahead<G::kCopies, DEPTH>(left < DEPTH - 1 ? left : DEPTH - 1);
            if constexpr (!G::kPriv) lds_barrier();   // every wave's copies of this iteration have landed

            const int ch = it * KS + part;
            if (ch < nchunks) {   // wave-uniform
                const int cb = nblk - ch * CB < CB ? nblk - ch * CB : CB;   // a multiple of 8
                const uint8_t* rowp = wbuf(slot) + rn * G::kWRowSlots * 16;
                const uint8_t* ap = abuf(slot) + part * G::kAPartBytes;
                // Groups of GB blocks (8, or 4 in workgroups of 12 or more
                // waves, whose 128-170 VGPRs would not hold 8) in three
                // phases, so that the matrix-core operations of a group are
                // independent of one another and of the scaling (each block
                // has its own result registers): operands, then every MFMA,
                // then the fp32 scaling.
                for (int o = 0; o < cb; o += GB) {
                    long bop[GB];
                    uint32_t h4[GB];
                    float dw[GB];
#pragma unroll
                    for (int p = 0; p < GB / 2; ++p) {   // block pairs o + 2p, o + 2p + 1
                        const uint32_t* wp =
                            reinterpret_cast<const uint32_t*>(rowp + ((o >> 1) + p) * 2 * WF::kBlockBytes);
                        WF::decode(wp, g, bop + 2 * p, dw + 2 * p);
                        WF::scale_bits(wp, dwidth, h4 + 2 * p);
                    }
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        long aop[GB];
                        uint32_t a8[GB];
#pragma unroll
                        for (int i = 0; i < GB; ++i) {
                            // A: code dwords g and 4 + g of column acol(t), block o + i,
                            // and the block's binary16 d8 (the low half of its first dword)
                            const uint32_t* ab = reinterpret_cast<const uint32_t*>(
                                ap + (acol(t) * G::kAColSlots * 16 + (o + i) * kQ81Bytes));
                            aop[i] = (long)((uint64_t)ab[1 + g] | ((uint64_t)ab[5 + g] << 32));
                            a8[i] = ab[0] & 0xFFFFu;
                        }
                        i32x4 dsum[GB];
#pragma unroll
                        for (int i = 0; i < GB; ++i)
                            dsum[i] = WF::kOffset ? __builtin_amdgcn_mfma_i32_16x16x32_i8(aop[i], kNeg8,
                                                                                         i32x4{0, 0, 0, 0}, 0, 0, 0)
                                                  : i32x4{0, 0, 0, 0};
#pragma unroll
                        for (int i = 0; i < GB; ++i)
                            dsum[i] = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop[i], bop[i], dsum[i], 0, 0, 0);
                        f32x4 sc[GB];
#pragma unroll
                        for (int i = 0; i < GB; ++i) sc[i] = scale_outer(a8[i], h4[i]);
#pragma unroll
                        for (int i = 0; i < GB; ++i)
#pragma unroll
                            for (int r = 0; r < 4; ++r) acc[t][r] = fmaf((float)dsum[i][r], sc[i][r], acc[t][r]);
                    }
                    if constexpr (TAIL) {
                        // 17 columns: the 17th on the vector unit instead of a second,
                        // mostly empty matrix-core tile.  The lane's B operand holds its
                        // row's codes at 8 of the block's 32 k-slots; two v_dot4 with the
                        // matching q8 codes give an exact partial block sum, which the
                        // lane scales by d4 d8 (the other 24 k-slots are the other three
                        // lane groups', added after the loop).
#pragma unroll
                        for (int i = 0; i < GB; ++i) {
                            uint32_t wl = (uint32_t)(uint64_t)bop[i], wh = (uint32_t)((uint64_t)bop[i] >> 32);
                            if constexpr (WF::kOffset) {   // codes 0..15 -> q - 8 as int8, byte by byte
                                wl = (wl + 0x78787878u) ^ 0x80808080u;
                                wh = (wh + 0x78787878u) ^ 0x80808080u;
                            }
                            const uint32_t* ab = reinterpret_cast<const uint32_t*>(
                                ap + (16 * G::kAColSlots * 16 + (o + i) * kQ81Bytes));
                            const int sdot = dot4_i8(wh, ab[5 + g], dot4_i8(wl, ab[1 + g], 0));
                            tacc = fmaf((float)sdot, dw[i] * half_lo_to_f32(ab[0]), tacc);
                        }
                    }
                }
            }
            slot = slot + 1 == DEPTH ? 0 : slot + 1;
        }

        if constexpr (TAIL) {   // the four lane groups' shares of each row, in a fixed order
            tacc += __shfl_xor(tacc, 16);
            tacc += __shfl_xor(tacc, 32);
        }
        // combine the KS parts of each row tile (fixed order) and store
        if constexpr (KS > 1) {
            lds_barrier();   // every wave is done reading the buffers: reuse them
            float* red = reinterpret_cast<float*>(lds);
            float* const tred = red + G::kW * NT * 4 * 64;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) red[((wave * NT + t) * 4 + r) * 64 + lane] = acc[t][r];
            if constexpr (TAIL) tred[wave * 64 + lane] = tacc;
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
                if constexpr (TAIL) {
                    for (int s2 = 1; s2 < KS; ++s2) tacc += tred[(wave + s2) * 64 + lane];
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
                if constexpr (TAIL) {
                    if (g == 0) Y[(size_t)16 * N + n] = tacc;
                }
            }
        }
    }
}

template <class WF, int CB, int MP, int RT, int KS, int DEPTH>
hipError_t launch_mfma_cfg(const void* Wq, const void* Xq, float* Y, int N, int K, int M, int grid, hipStream_t s) {
    const size_t lds = mfma_lds_bytes<WF, CB, MP, RT, KS, DEPTH>();
    if (lds > device_max_lds_per_block()) return hipErrorInvalidValue;
    if ((K >> 5) % CB != 0 || K > (1 << 26)) return hipErrorInvalidValue;   // whole chunks, 32-bit offsets
    const int groups = (N + 16 * RT - 1) / (16 * RT);
    const int g = grid ? grid : groups;
    hipLaunchKernelGGL((k_qmfma<WF, CB, MP, RT, KS, DEPTH>), dim3(g), dim3(64 * RT * KS), lds, s,
                       (const uint8_t*)Wq, (const uint8_t*)Xq, Y, N, K, M);
    return hipGetLastError();
}

template <class WF, int CB, int MP, int RT, int KS, int DEPTH>
constexpr bool mfma_builds() {
    // the stages fit the LDS of one workgroup, the wait counts fit the vmcnt
    // field, and the workgroups whose waves would exceed their registers (128
    // per lane at 16 waves, 170 at 12) and spill are not built: 12 and 16
    // waves up to 24 columns, 16 parts of K up to 16, and Q8_0 (wider
    // weight operands) at 16 waves up to 16
    return mfma_lds_bytes<WF, CB, MP, RT, KS, DEPTH>() <= 160 * 1024 &&
           MfmaGeom<WF, CB, MP, RT, KS>::kCopies * (DEPTH - 1) <= 63 && (RT * KS < 12 || MP <= 24) &&
           (KS < 16 || MP <= 16) && (RT * KS < 16 || MP <= 16 || WF::kBlockBytes == 18);
}

// The built configurations for one padded column count MP.
template <class WF, int MP>
hipError_t launch_mfma_mp(int RT, int KS, int DEPTH, int CB, const void* Wq, const void* Xq, float* Y, int N, int K,
                          int M, int grid, hipStream_t s) {
#define DG_MF(RR, SS, DD, CC)                                                          \
    if constexpr (mfma_builds<WF, CC, MP, RR, SS, DD>()) {                             \
        if (RT == RR && KS == SS && DEPTH == DD && CB == CC)                           \
            return launch_mfma_cfg<WF, CC, MP, RR, SS, DD>(Wq, Xq, Y, N, K, M, grid, s); \
    }
    DG_MF(1, 16, 1, 8) DG_MF(2, 8, 1, 8) DG_MF(4, 4, 2, 8)                       // 16 waves
    DG_MF(1, 12, 1, 8) DG_MF(3, 4, 1, 8)                                          // 12 waves
    DG_MF(1, 8, 1, 8) DG_MF(1, 8, 2, 8) DG_MF(2, 4, 2, 8) DG_MF(4, 2, 2, 8)      // 8 waves
    DG_MF(8, 1, 2, 8)
    DG_MF(4, 1, 2, 8) DG_MF(4, 1, 3, 8) DG_MF(2, 2, 2, 8) DG_MF(1, 4, 2, 8)      // 4 waves
    DG_MF(1, 4, 3, 8) DG_MF(1, 4, 4, 8) DG_MF(1, 4, 5, 8) DG_MF(2, 2, 3, 8) DG_MF(2, 2, 4, 8)
#undef DG_MF
    return hipErrorInvalidValue;
}

// unroll = RT * 10000 + KS * 100 + DEPTH * 10 + CB / 8 selects a configuration
// for sweeps (0: the default for the shape); the padded column count follows M.
template <class WF>
hipError_t launch_qmfma(int M, int unroll, const void* Wq, const void* Xq, float* Y, int N, int K, int grid,
                        hipStream_t s) {
    int RT, KS, DEPTH, CB;
    if (unroll) {
        RT = unroll / 10000;
        KS = (unroll / 100) % 100;
        DEPTH = (unroll / 10) % 10;
        CB = (unroll % 10) * 8;
    } else {
        // Measured on MI355X (decoder shapes, M = 2..24), both formats.  Up to
        // 512 row tiles: one tile per workgroup, K split over 8 waves up to 8
        // columns (4 for Q4_0 rows up to 4096) and beyond 16 on rows up to
        // 8192 (one chunk deep there, as the chunks of 24 columns fill the
        // LDS), over 12 waves one deep beyond 16 on longer Q4_0 rows, else
        // over 4 waves two deep.  More row tiles: tiles share each
        // activation chunk.  17 columns run one 16-column tile plus the 17th
        // column on the vector unit (MP = 17), over 8 waves two deep up to
        // 512 row tiles (Q4_0; Q8_0 as above) and over two tiles of two waves
        // beyond: 4096 x 14336 Q4_0 15.8 against 16.8 us with a second
        // matrix-core tile, 14336 x 4096 Q8_0 19.0 against 20.7 us.
        const int tiles = (N + 15) / 16;
        CB = 8;
        if (tiles <= 512) {
            RT = 1;
            const bool wide = M > 16 && K <= 8192;
            const bool few = M <= 8 && (K > 4096 || WF::kBlockBytes == 34);
            KS = (few || wide) ? 8 : 4;
            DEPTH = wide ? 1 : 2;
            if (M > 16 && K > 8192 && WF::kBlockBytes == 18) { KS = 12; DEPTH = 1; }   // 17..24 columns, long rows
            if (M == 17 && WF::kBlockBytes == 18) { KS = 8; DEPTH = 2; }         // 16 + 1 columns
        } else if (WF::kBlockBytes == 34) {
            // Q8_0: its weight buffers are twice those of Q4_0, so fewer row
            // tiles share a workgroup's LDS.
            DEPTH = 2;
            if (M <= 17) { RT = 2; KS = 2; }
            else { RT = 4; KS = 1; }
        } else {
            DEPTH = 2;
            if (M <= 4) { RT = 2; KS = 4; }
            else { RT = 2; KS = 2; }
        }
    }
    if (M <= 4) return launch_mfma_mp<WF, 4>(RT, KS, DEPTH, CB, Wq, Xq, Y, N, K, M, grid, s);
    if (M <= 8) return launch_mfma_mp<WF, 8>(RT, KS, DEPTH, CB, Wq, Xq, Y, N, K, M, grid, s);
    if (M <= 16) return launch_mfma_mp<WF, 16>(RT, KS, DEPTH, CB, Wq, Xq, Y, N, K, M, grid, s);
    if (M == 17) return launch_mfma_mp<WF, 17>(RT, KS, DEPTH, CB, Wq, Xq, Y, N, K, M, grid, s);
    return launch_mfma_mp<WF, 24>(RT, KS, DEPTH, CB, Wq, Xq, Y, N, K, M, grid, s);
}

}  // namespace

hipError_t launch_q4_mfma(int M, int unroll, const void* Wq, const void* Xq, float* Y, int N, int K, int grid,
                          hipStream_t s) {
    return launch_qmfma<FmtQ4_0>(M, unroll, Wq, Xq, Y, N, K, grid, s);
}

hipError_t launch_q8_mfma(int M, int unroll, const void* Wq, const void* Xq, float* Y, int N, int K, int grid,
                          hipStream_t s) {
    return launch_qmfma<FmtQ8_0>(M, unroll, Wq, Xq, Y, N, K, grid, s);
}

}  // namespace dg
