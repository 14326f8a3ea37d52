// gemv_qmfma_res.hip -- Q4_0 / Q8_0 x Q8_1 for a few activation columns on
// the int8 matrix cores, with the activation columns resident in LDS (the
// small-batch kernel of "The kernel that waited for itself").
//
// The arithmetic is that of the streaming matrix-core kernel: per weight
// block and per tile of 16 rows x 16 columns, v_mfma_i32_16x16x32_i8 gives
// the exact int32 block sums (A = 16 columns of q8 codes, B = 16 rows of
// codes, Q4_0's -8 offset as a second MFMA against a constant -8 operand),
// and each sum is scaled in fp32 by d8 * d4 (the 16 x 16 products from one
// f16 MFMA of the raw binary16 scales, exact) and added in block order.
//
// What differs is the data flow, chosen from counters of the streaming kernel
// (one or two waves per SIMD, two workgroup barriers per 8-block chunk, a
// quarter of the vector instructions spent on copy addresses):
//  * every workgroup copies all M activation columns (raw Q8_1 blocks) into
//    LDS once and keeps them for every row tile it computes; workgroups are persistent
//    and take row groups b, b + grid, ...;
//  * a workgroup is RT x KS waves: RT row tiles of 16 rows, each row's K split
//    into KS equal parts.  Wave (t, p) owns part p of tile t; it walks its
//    (row group, 8-block chunk) items in order and streams the chunk's 16 row
//    spans (16 x 144 bytes for Q4_0, 16 x 272 for Q8_0) with 16-byte loads
//    straight into registers, P items ahead of the one it computes.  To
//    compute, it writes the chunk into a private LDS buffer (rows at an odd
//    number of 16-byte slots) and reads back the MFMA operands: LDS
//    operations of one wave complete in order, so no barrier is needed;
//  * the KS partial sums of a row tile meet in LDS after the tile's last
//    chunk and are added in the fixed order 0..KS-1 (deterministic), which is
//    the only place the waves of a workgroup synchronise.
#include "dg_internal.h"
#include "mfma_formats.h"

namespace dg {
namespace {

using namespace q4;
using namespace mfma;

constexpr int kCB = 8;   // blocks per chunk

template <class WF>
struct ResGeom {
    static constexpr int kG = kCB * WF::kBlockBytes / 16;   // 16-byte granules per row span (9 or 17, odd)
    static constexpr int kL = (16 * kG + kWave - 1) / kWave;  // loads per lane per chunk (3 or 5)
    static constexpr int kBufBytes = kL * 1024;             // per-wave transpose buffer
};

// LDS bytes of one workgroup: the activation columns (cstr bytes each), one
// transpose buffer per wave, and the partial sums of the KS - 1 upper parts
// of each row tile.
template <class WF>
__host__ __device__ constexpr size_t res_lds_bytes(int M, int cstr, int NT, int RT, int KS) {
    return (size_t)M * cstr + (size_t)RT * KS * ResGeom<WF>::kBufBytes + (size_t)RT * (KS - 1) * NT * 1024;
}

// Bytes per activation column in LDS: the column's 36-byte blocks rounded up
// to an odd number of 16-byte slots, so that the 16 columns a lane group
// reads fall in different banks.
__host__ __device__ constexpr int res_col_bytes(int nblk) { return ((nblk * 36 / 16) | 1) * 16; }

// Loads one chunk: the 16 row spans of kCB blocks from block blk0 of the
// rows n0 .. n0 + 15, as kL 16-byte loads per lane.  Lane slot q = j*64 + lane
// is granule c = q % kG of row r = q / kG (rq[j] = r, cq[j] = 16 c, fixed per
// lane); slots past the 16 spans re-read the last granule (their LDS slots are
// never read) and rows past N re-read row N - 1 (their results are dropped).
// The chunk's base is wave-uniform, so each load is one scalar base plus one
// 32-bit offset (row_bytes < 2^24).
template <class WF>
__device__ __forceinline__ void load_chunk(const uint8_t* __restrict__ Wq, uint32_t row_bytes, int n0, int N,
                                           int blk0, const int (&rq)[ResGeom<WF>::kL],
                                           const uint32_t (&cq)[ResGeom<WF>::kL], u32x4 (&st)[ResGeom<WF>::kL]) {
    using G = ResGeom<WF>;
    const uint8_t* base = Wq + (size_t)n0 * row_bytes + (size_t)blk0 * WF::kBlockBytes;
    const int rmax = N - 1 - n0;   // >= 0: every row group starts below N
#pragma unroll
    for (int j = 0; j < G::kL; ++j) {
        const int rr = rq[j] < rmax ? rq[j] : rmax;
        st[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (__umul24(rr, row_bytes) + cq[j])));
    }
}

template <class WF, int NT, int RT, int KS, int P>
__global__ void __launch_bounds__(64 * RT * KS)
k_qres(const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Xq, float* __restrict__ Y, int N, int K,
       int M) {
    using G = ResGeom<WF>;
    constexpr int W = RT * KS;
    constexpr int MP = 16 * NT;
    static_assert(P >= 1 && P <= 3, "chunks in flight");
    extern __shared__ u32x4 res_lds[];
    uint8_t* const lds = reinterpret_cast<uint8_t*>(res_lds);
    const int lane = lane_id();
    const int wave = wave_in_block();
    const int tile = wave / KS;
    const int part = wave - tile * KS;
    const int g = lane >> 4, rn = lane & 15;
    const int nblk = K >> 5;
    const int SB = nblk / KS;        // blocks per part, a multiple of kCB
    const int nch = SB / kCB;        // chunks per part
    const size_t row_bytes = (size_t)nblk * WF::kBlockBytes;
    const int cstr = res_col_bytes(nblk);
    const int ngroups = (N + 16 * RT - 1) / (16 * RT);
    uint8_t* const acts = lds;
    uint8_t* const tbuf = lds + (size_t)M * cstr + wave * G::kBufBytes;
    float* const red = reinterpret_cast<float*>(lds + (size_t)M * cstr + W * G::kBufBytes);
    const uint32_t dwidth = g == 0 ? 16u : 0u;   // lane group 0 feeds d4 to k-slot 0 of the scale products

    // this workgroup's row groups, and its items (row group, chunk) in order
    const int mygroups = (int)blockIdx.x < ngroups ? (ngroups - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
    const int items = mygroups * nch;
    auto item_n0 = [&](int i) { return ((int)blockIdx.x + (i / nch) * (int)gridDim.x) * RT * 16 + tile * 16; };
    auto item_blk0 = [&](int i) { return part * SB + (i - (i / nch) * nch) * kCB; };
    // a tile past N (the last group, RT > 1) computes row N - 1 and drops it
    auto clamp_n0 = [&](int n0) { return n0 < N ? n0 : N - 1; };

    // per-lane granule of each chunk load
    int rq[G::kL];
    uint32_t cq[G::kL];
#pragma unroll
    for (int j = 0; j < G::kL; ++j) {
        const int q0 = j * kWave + lane;
        const int q = q0 < 16 * G::kG ? q0 : 16 * G::kG - 1;
        rq[j] = q / G::kG;
        cq[j] = (uint32_t)(q - rq[j] * G::kG) * 16;
    }
    const uint32_t rb32 = (uint32_t)row_bytes;

    // the first P chunks, then the activation columns (ordinary 16-byte loads,
    // mostly served by L2: every workgroup reads the same columns), so that
    // both latencies overlap
    u32x4 st[P][G::kL];
#pragma unroll
    for (int s = 0; s < P; ++s) {
        const int i = s < items ? s : (items > 0 ? items - 1 : 0);
        if (items > 0) load_chunk<WF>(Wq, rb32, clamp_n0(item_n0(i)), N, item_blk0(i), rq, cq, st[s]);
    }

    const int gpc = nblk * 36 / 16;   // granules per column
    const int cslots = cstr / 16;
    const int aslots = M * cslots;
    constexpr int kAB = 8;            // activation granules per thread per batch
    for (int s0 = 0; s0 < aslots; s0 += kAB * 64 * W) {
        u32x4 a[kAB];
#pragma unroll
        for (int u = 0; u < kAB; ++u) {
            const int s = s0 + u * 64 * W + (int)threadIdx.x;
            const int m = s / cslots;
            const int c = s - m * cslots;
            const int mc = m < M ? m : M - 1;
            const int cc = c < gpc ? c : gpc - 1;
            a[u] = *reinterpret_cast<const u32x4*>(Xq + ((size_t)mc * nblk * 36 + (size_t)cc * 16));
        }
#pragma unroll
        for (int u = 0; u < kAB; ++u) {
            const int s = s0 + u * 64 * W + (int)threadIdx.x;
            if (s < aslots) *reinterpret_cast<u32x4*>(acts + (size_t)s * 16) = a[u];
        }
    }

    lds_barrier();   // every column is in LDS

    int acol[NT];   // the activation column this lane feeds to tile t (padded columns re-read M - 1)
#pragma unroll
    for (int t = 0; t < NT; ++t) acol[t] = 16 * t + rn < M ? 16 * t + rn : M - 1;

    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // one item: the chunk in st -> LDS, refill st with item i + P, compute
    auto step = [&](int i, u32x4 (&sti)[G::kL], bool refill) {
#pragma unroll
        for (int j = 0; j < G::kL; ++j) *reinterpret_cast<u32x4*>(tbuf + j * 1024 + lane * 16) = sti[j];
        if (refill) {
            const int i2 = i + P;
            load_chunk<WF>(Wq, rb32, clamp_n0(item_n0(i2)), N, item_blk0(i2), rq, cq, sti);
        }
        const uint8_t* rowp = tbuf + rn * G::kG * 16;
        // two halves of four blocks: operands, then the 8 MFMAs of a column
        // tile (independent of one another), then its fp32 scaling
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            constexpr int kH = kCB / 2;
            const int blk0 = item_blk0(i) + h * kH;
            long bop[kH];
            uint32_t h4[kH];
#pragma unroll
            for (int p = 0; p < kH / 2; ++p) {
                const uint32_t* wp = reinterpret_cast<const uint32_t*>(rowp + (h * kH / 2 + p) * 2 * WF::kBlockBytes);
                float dunused[2];
                WF::decode(wp, g, bop + 2 * p, dunused);
                WF::scale_bits(wp, dwidth, h4 + 2 * p);
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint8_t* ap = acts + (size_t)acol[t] * cstr + (size_t)blk0 * kQ81Bytes;
                long aop[kH];
                uint32_t a8[kH];   // the block's binary16 d8
#pragma unroll
                for (int b = 0; b < kH; ++b) {
                    const uint32_t* ab = reinterpret_cast<const uint32_t*>(ap + b * kQ81Bytes);
                    aop[b] = (long)((uint64_t)ab[1 + g] | ((uint64_t)ab[5 + g] << 32));
                    a8[b] = ab[0] & 0xFFFFu;
                }
                i32x4 dsum[kH];
#pragma unroll
                for (int b = 0; b < kH; ++b)
                    dsum[b] = WF::kOffset
                                  ? __builtin_amdgcn_mfma_i32_16x16x32_i8(aop[b], kNeg8, i32x4{0, 0, 0, 0}, 0, 0, 0)
                                  : i32x4{0, 0, 0, 0};
#pragma unroll
                for (int b = 0; b < kH; ++b)
                    dsum[b] = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop[b], bop[b], dsum[b], 0, 0, 0);
                f32x4 sc[kH];
#pragma unroll
                for (int b = 0; b < kH; ++b) sc[b] = scale_outer(a8[b], h4[b]);
#pragma unroll
                for (int b = 0; b < kH; ++b)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[t][r] = fmaf((float)dsum[b][r], sc[b][r], acc[t][r]);
            }
        }
        if (i - (i / nch) * nch == nch - 1) {   // the tile's last chunk: combine the parts, store
            const int n = item_n0(i) + rn;
            if constexpr (KS > 1) {
                if (part != 0) {
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        *reinterpret_cast<f32x4*>(red + (((tile * (KS - 1) + part - 1) * NT + t) * 64 + lane) * 4) =
                            acc[t];
                }
                lds_barrier();
                if (part == 0) {
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        for (int p2 = 1; p2 < KS; ++p2)
                            acc[t] += *reinterpret_cast<const f32x4*>(
                                red + (((tile * (KS - 1) + p2 - 1) * NT + t) * 64 + lane) * 4);
                }
                lds_barrier();
            }
            if (part == 0 && n < N) {
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int m = 16 * t + 4 * g + r;
                        if (m < M) Y[(size_t)m * N + n] = acc[t][r];
                    }
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };

    int i = 0;
    for (; i + 2 * P <= items; i += P) {   // steady state: every item refills its stage
#pragma unroll
        for (int s = 0; s < P; ++s) step(i + s, st[s], true);
    }
    for (; i < items; i += P) {            // the last items: refill only while items remain
#pragma unroll
        for (int s = 0; s < P; ++s)
            if (i + s < items) step(i + s, st[s], i + s + P < items);
    }
}

template <class WF, int NT, int RT, int KS, int P>
hipError_t launch_res_cfg(const void* Wq, const void* Xq, float* Y, int N, int K, int M, int grid, hipStream_t s) {
    const int nblk = K / 32;
    if (nblk % (KS * kCB) != 0) return hipErrorInvalidValue;
    const size_t lds = res_lds_bytes<WF>(M, res_col_bytes(nblk), NT, RT, KS);
    const size_t cap = device_max_lds_per_block();
    if (lds > cap) return hipErrorInvalidValue;
    const int groups = (N + 16 * RT - 1) / (16 * RT);
    int g = grid;
    if (!g) {
        // persistent: as many workgroups as fit the CUs at once, never more than row groups
        const int per_cu = (int)(cap / lds) > 0 ? (int)(cap / lds) : 1;
        const int fit = device_cu_count() * (per_cu < 16 / (RT * KS) * 2 ? per_cu : 16 / (RT * KS) * 2);
        g = groups < fit ? groups : fit;
    }
    hipLaunchKernelGGL((k_qres<WF, NT, RT, KS, P>), dim3(g), dim3(64 * RT * KS), lds, s, (const uint8_t*)Wq,
                       (const uint8_t*)Xq, Y, N, K, M);
    return hipGetLastError();
}

// 16-wave workgroups (128 VGPRs per lane) with two column tiles are built
// only for Q4_0 with one row tile: Q8_0's 5-load chunks, or several row
// tiles' offsets, would spill.
template <class WF, int NT, int RT, int KS>
constexpr bool res_builds() {
    return !(NT == 2 && RT * KS == 16 && (WF::kBlockBytes == 34 || RT > 1));
}

template <class WF, int NT>
hipError_t launch_res_nt(int RT, int KS, int P, const void* Wq, const void* Xq, float* Y, int N, int K, int M,
                         int grid, hipStream_t s) {
#define DG_RES(RR, SS, PP)                                                                  \
    if constexpr (res_builds<WF, NT, RR, SS>()) {                                            \
        if (RT == RR && KS == SS && P == PP)                                                \
            return launch_res_cfg<WF, NT, RR, SS, PP>(Wq, Xq, Y, N, K, M, grid, s);           \
    }
    DG_RES(1, 16, 2) DG_RES(2, 8, 2) DG_RES(4, 4, 2)                  // 16 waves
    DG_RES(1, 8, 2) DG_RES(2, 4, 2) DG_RES(4, 2, 2) DG_RES(8, 1, 2)   // 8 waves
    DG_RES(1, 4, 2) DG_RES(2, 2, 2) DG_RES(4, 1, 2)                   // 4 waves
    DG_RES(1, 8, 3) DG_RES(2, 4, 3) DG_RES(1, 4, 3)
#undef DG_RES
    return hipErrorInvalidValue;
}

// unroll = RT * 10000 + KS * 100 + P * 10 (row tiles and K parts per
// workgroup, chunks in flight per wave); 0 = the default for the shape.
template <class WF>
hipError_t launch_res(int M, int unroll, const void* Wq, const void* Xq, float* Y, int N, int K, int grid,
                      hipStream_t s) {
    int RT, KS, P;
    if (unroll) {
        RT = unroll / 10000;
        KS = (unroll / 100) % 100;
        P = (unroll / 10) % 10;
    } else {
        // Measured on MI355X (decoder shapes, M = 2..24): with many row tiles
        // (14336 rows) four tiles per workgroup, K in two parts for Q4_0 and
        // whole for Q8_0 (its chunks are twice as large); otherwise one tile
        // per workgroup with K in eight parts, or four when the columns need
        // the LDS.
        const int tiles = (N + 15) / 16;
        P = 2;
        if (tiles > 512) { RT = 4; KS = WF::kBlockBytes == 34 ? 1 : 2; }
        else { RT = 1; KS = 8; }
        const int nblk = K / 32, NT = M <= 16 ? 1 : 2;
        if (nblk % (KS * kCB) != 0 ||
            res_lds_bytes<WF>(M, res_col_bytes(nblk), NT, RT, KS) > device_max_lds_per_block()) {
            RT = 1;
            KS = 4;
        }
    }
    if (M < 1 || M > 32) return hipErrorInvalidValue;
    if (M <= 16) return launch_res_nt<WF, 1>(RT, KS, P, Wq, Xq, Y, N, K, M, grid, s);
    return launch_res_nt<WF, 2>(RT, KS, P, Wq, Xq, Y, N, K, M, grid, s);
}

}  // namespace

hipError_t launch_q4_res(int M, int unroll, const void* Wq, const void* Xq, float* Y, int N, int K, int grid,
                         hipStream_t s) {
    return launch_res<FmtQ4_0>(M, unroll, Wq, Xq, Y, N, K, grid, s);
}

hipError_t launch_q8_res(int M, int unroll, const void* Wq, const void* Xq, float* Y, int N, int K, int grid,
                         hipStream_t s) {
    return launch_res<FmtQ8_0>(M, unroll, Wq, Xq, Y, N, K, grid, s);
}

}  // namespace dg
