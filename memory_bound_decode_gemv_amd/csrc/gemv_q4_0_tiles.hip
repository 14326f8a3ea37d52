// gemv_q4_0_tiles.hip -- Q4_0 x Q8_1 for 1..24 activation columns from Q4_0
// weights rearranged into 16-row tiles, and that rearrangement.
//
// Why a second weight layout.  In the row-major block format every 16-row
// tile of the matrix-core kernels is 16 row segments of 144 bytes per 8
// blocks, two cache lines each and 8064 bytes apart at K = 14336; a wave can
// only turn them into MFMA operands through LDS, and those reads, copies and
// waits bound the small-batch kernel well below HBM speed.  The small-batch
// page ("The kernel that waited for itself", what remains open: the VALU
// floor) names a different weight format as the next step, and the
// bitsandbytes issue on 4-bit decode (its analysis of the naive kernel) asks
// for a layout in which consecutive lanes read consecutive 128-bit chunks
// before unpacking.  The tiled layout holds the same bytes (every block's
// binary16 scale and its 16 code bytes, untouched), ordered so that one
// 16-byte load per lane IS the B operand of four consecutive blocks:
//
//   tile t (rows 16t..16t+15) x group s (blocks 8s..8s+7): 2304 bytes at
//   (t * K/256 + s) * 2304:
//     bytes    0..1023: lane l (l = 16g + n) holds, in dword j, code bytes
//                       4g..4g+3 of row 16t+n, block 8s+j;
//     bytes 1024..2047: the same for blocks 8s+4..8s+7;
//     bytes 2048..2303: row n's eight binary16 scales (blocks 8s..8s+7) at
//                       2048 + 16n, block 8s+i in half i%2 of dword i/2.
//   Rows past N (the last tile's padding) hold codes 0x88 and scale 0, so
//   they add exact zeros.
//
// The matrix-core arithmetic is that of the row-major kernels: per block, one
// v_mfma_i32_16x16x32_i8 of the 16 columns' q8 codes against the 16 rows'
// 4-bit codes, a second against the constant -8 (the offset of q - 8), and
// the d8 * d4 products from one v_mfma_f32_16x16x16_f16 (exact in fp32); the
// int32 block sums are converted and scaled in fp32.  Lane group g carries
// k-slots 4g..4g+3 (low nibbles of code dword g) and 16+4g..16+4g+3 (high
// nibbles), with the matching activation code dwords g and 4 + g.
//
// Data flow.  A workgroup of RT x KW waves covers RT row tiles over one range
// of K (KP ranges per row group, one per workgroup); wave (rt, kw) streams
// tile rt over the kw-th part of the range, D groups of 8 blocks in flight
// (three 16-byte non-temporal loads per lane and group, straight into the
// operand registers: no LDS and no reshuffling for the weights).  The M
// activation columns of the range are copied once into LDS (DMA, columns at
// an odd stride of 16-byte slots so that the 16 columns of a lane group read
// different banks), while the first weight groups are in flight.  The KW
// parts of a tile meet in LDS in the fixed order 0..KW-1.  With KP > 1, each
// workgroup writes its partial tile sums to a workspace and takes a ticket
// from a per-row-group counter; the workgroup that takes the last ticket adds
// the KP partials in the fixed order 0..KP-1, stores Y and resets the counter
// to zero for the next call.  Results therefore do not depend on timing.
// Workgroup i of a row group takes range i % KP: with the hardware's
// round-robin placement, the workgroups on one XCD read the same activation
// range, so each XCD's L2 holds only its part of the columns.
#include "dg_internal.h"
#include "mfma_formats.h"

namespace dg {
namespace {

using namespace q4;
using namespace mfma;

constexpr int kGroupBlocks = 8;      // blocks per group of a tile
constexpr int kGroupBytes = 2304;    // 16 rows x 8 blocks x 18 bytes
constexpr int kCodeBytes = 2048;     // the group's code bytes; 256 bytes of scales follow
constexpr int kGroupSlots = 18;      // 16-byte slots of one column's Q8_1 blocks per group (8 x 36 / 16)

// ---------------------------------------------------------------------------
// Rearrangement: one thread per 16-byte slot of the tiled layout (144 per
// group).  Source reads are 2-byte loads (block fields sit at even offsets).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
k_q4_tiles_pack(const uint8_t* __restrict__ Wq, uint8_t* __restrict__ Wt, int N, int S, int64_t slots) {
    const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= slots) return;
    const int64_t ts = u / 144;                 // tile * S + group
    const int k = (int)(u - ts * 144);
    const int64_t t = ts / S;
    const int s = (int)(ts - t * S);
    const size_t row_bytes = (size_t)S * kGroupBlocks * 18;
    uint32_t d[4];
    if (k < 128) {
        const int h = k >> 6, l = k & 63, g = l >> 4, n = l & 15;
        const int64_t row = t * 16 + n;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (row < N) {
                const uint16_t* p = reinterpret_cast<const uint16_t*>(
                    Wq + (size_t)row * row_bytes + (size_t)(kGroupBlocks * s + 4 * h + j) * 18 + 2 + 4 * g);
                d[j] = (uint32_t)p[0] | ((uint32_t)p[1] << 16);
            } else {
                d[j] = 0x88888888u;
            }
        }
    } else {
        const int n = k - 128;
        const int64_t row = t * 16 + n;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t lo = 0, hi = 0;
            if (row < N) {
                const uint8_t* r = Wq + (size_t)row * row_bytes + (size_t)(kGroupBlocks * s + 2 * j) * 18;
                lo = *reinterpret_cast<const uint16_t*>(r);
                hi = *reinterpret_cast<const uint16_t*>(r + 18);
            }
            d[j] = lo | (hi << 16);
        }
    }
    *reinterpret_cast<u32x4*>(Wt + (size_t)ts * kGroupBytes + (size_t)k * 16) = u32x4{d[0], d[1], d[2], d[3]};
}

// Three 16-byte loads per lane: the codes of blocks 0..3 and 4..7 of the
// group (this lane's B operands) and its row's eight scales.
__device__ __forceinline__ void load_group(const uint8_t* __restrict__ g0, int lane, int rn, u32x4 (&w)[3]) {
    w[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(g0 + lane * 16));
    w[1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(g0 + 1024 + lane * 16));
    w[2] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(g0 + kCodeBytes + rn * 16));
}

// Marks a group's registers as written here (an empty asm): arithmetic on
// them cannot move above this point, and its loads are waited for here.
__device__ __forceinline__ void bind_group(u32x4 (&w)[3]) {
    asm volatile("" : "+v"(w[0]), "+v"(w[1]), "+v"(w[2])::"memory");
}

template <int NT>
__device__ __forceinline__ void store_tile(const f32x4 (&acc)[NT], float* __restrict__ Y, int N, int M, int t,
                                           int g, int rn) {
    const int n = t * 16 + rn;
    if (n >= N) return;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = tt * 16 + g * 4 + r;
            if (m < M) Y[(size_t)m * N + n] = acc[tt][r];
        }
}

// One group of 8 blocks: operands, matrix-core products, fp32 scaling into
// acc.  blk is the group's first block within the LDS copy of the columns;
// width is 16 in lane group 0 (it feeds d4 to k-slot 0 of the scale
// products), 0 elsewhere and for a group that must add exact zeros.
template <int NT, int GB>
__device__ __forceinline__ void tiles_group(const u32x4 (&w)[3], const uint8_t* lds, const uint32_t (&acol)[NT],
                                            uint32_t blk, int g, uint32_t width, f32x4 (&acc)[NT]) {
    const uint32_t code[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
    const uint32_t scl[4] = {w[2].x, w[2].y, w[2].z, w[2].w};
#pragma unroll
    for (int o = 0; o < kGroupBlocks; o += GB) {
        long bop[GB];
        uint32_t h4[GB];
#pragma unroll
        for (int b = 0; b < GB; ++b) {
            const uint32_t c = code[o + b];
            bop[b] = (long)((uint64_t)(c & kNib) | ((uint64_t)((c >> 4) & kNib) << 32));
            h4[b] = __builtin_amdgcn_ubfe(scl[(o + b) >> 1], ((o + b) & 1) * 16, width);
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            long aop[GB];
            uint32_t a8[GB];
#pragma unroll
            for (int b = 0; b < GB; ++b) {
                const uint32_t* ab = reinterpret_cast<const uint32_t*>(lds + acol[tt] + (blk + o + b) * kQ81Bytes);
                aop[b] = (long)((uint64_t)ab[1 + g] | ((uint64_t)ab[5 + g] << 32));
                a8[b] = ab[0] & 0xFFFFu;
            }
            i32x4 dsum[GB];
#pragma unroll
            for (int b = 0; b < GB; ++b)
                dsum[b] = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop[b], kNeg8, i32x4{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
            for (int b = 0; b < GB; ++b)
                dsum[b] = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop[b], bop[b], dsum[b], 0, 0, 0);
            f32x4 sc[GB];
#pragma unroll
            for (int b = 0; b < GB; ++b) sc[b] = scale_outer(a8[b], h4[b]);
#pragma unroll
            for (int b = 0; b < GB; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[tt][r] = fmaf((float)dsum[b][r], sc[b][r], acc[tt][r]);
        }
    }
}

// ---------------------------------------------------------------------------
// The GEMV.  MP = 16 (M <= 16) or 32 (17..24 columns: two 16-column tiles,
// the second one's rows past M re-reading column M - 1, results dropped).
// ---------------------------------------------------------------------------
template <int MP, int RT, int KW, int D>
__global__ void __launch_bounds__(64 * RT * KW)
k_q4_tiles(const uint8_t* __restrict__ Wt, const uint8_t* __restrict__ Xq, float* __restrict__ Y,
           uint32_t* __restrict__ tickets, f32x4* __restrict__ part, int N, int K, int M, int KP, int spw,
           int cs_slots, uint32_t cs_magic) {
    constexpr int NT = MP / 16;
    constexpr int W = RT * KW;
    constexpr int GB = 2;   // blocks per operand batch
    extern __shared__ u32x4 tiles_lds[];
    __shared__ int last_ticket;
    uint8_t* const lds = reinterpret_cast<uint8_t*>(tiles_lds);
    const int lane = lane_id();
    const int wave = wave_in_block();
    const int rt = wave / KW, kw = wave - rt * KW;
    const int g = lane >> 4, rn = lane & 15;
    const int S = K >> 8;
    const int nblk = K >> 5;
    const int T = (N + 15) >> 4;
    const int grp = (int)blockIdx.x / KP;
    const int kp = (int)blockIdx.x - grp * KP;
    const int s0 = kp * spw;                       // first group of the workgroup's range
    const int ns = min(spw, S - s0);               // groups in the range (>= 1)
    const int spk = (ns + KW - 1) / KW;
    const int w0 = kw * spk;                       // the wave's part: groups w0 .. w0 + cnt - 1 of the range
    const int cnt = max(0, min(spk, ns - w0));     // wave-uniform
    const int t = grp * RT + rt;
    const int tc = t < T ? t : T - 1;
    const uint8_t* const wbase = Wt + ((size_t)tc * S + s0 + (cnt > 0 ? w0 : 0)) * kGroupBytes;
    const int last = cnt > 0 ? cnt - 1 : 0;

    // (1) the first D groups of this wave's weights (past its part: its last
    // group again, never used), then (2) the activation columns of the range
    u32x4 wb[D][3];
#pragma unroll
    for (int d = 0; d < D; ++d) load_group(wbase + (size_t)(d < cnt ? d : last) * kGroupBytes, lane, rn, wb[d]);
    {
        const int used = ns * kGroupSlots;
        const int copies = (M * cs_slots + kWave - 1) / kWave;
        const uint8_t* const xr = Xq + (size_t)s0 * kGroupBlocks * kQ81Bytes;
        for (int j = wave; j < copies; j += W) {
            const uint32_t q = (uint32_t)(j * kWave + lane);
            const uint32_t m = __umulhi(q, cs_magic);          // q / cs_slots
            const uint32_t c = q - m * (uint32_t)cs_slots;
            const bool ok = m < (uint32_t)M && c < (uint32_t)used;
            const uint8_t* src = xr + (ok ? (size_t)m * nblk * kQ81Bytes + (size_t)c * 16 : 0);
            __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(lds + j * 1024), 16, 0, 0);
        }
    }
    // This wave's copies (and first weights) have landed, then every other
    // wave's.  The wait is the builtin, not inline asm, so that the compiler's
    // own wait counting knows nothing is outstanding past this point (after
    // an asm wait it assumed the copies pending and waited for every load at
    // the top of each round).
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt, lgkmcnt at their maximum: no wait
    lds_barrier();

    // A operand addresses: column 16 tt + rn of each 16-column tile (past M:
    // column M - 1 again, results dropped)
    uint32_t acol[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        const int m = 16 * tt + rn < M ? 16 * tt + rn : M - 1;
        acol[tt] = (uint32_t)m * (uint32_t)cs_slots * 16u;
    }
    const uint32_t dwidth = g == 0 ? 16u : 0u;   // lane group 0 feeds d4 to k-slot 0 of the scale products
    f32x4 acc[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // D groups per round; the loads of the next round are issued right after
    // each group's products, with no branch between them, so the compiler's
    // waits count exactly the D - 1 groups still in flight.  The last round
    // is peeled (no loads).
    const int rounds = (cnt + D - 1) / D;
    for (int rd = 0; rd + 1 < rounds; ++rd) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int i = rd * D + d;
            tiles_group<NT, GB>(wb[d], lds, acol, (uint32_t)(w0 + i) * kGroupBlocks, g, dwidth, acc);
            const int nx = i + D;
            load_group(wbase + (size_t)(nx < cnt ? nx : last) * kGroupBytes, lane, rn, wb[d]);
            // Keep the loads here and the next group's arithmetic behind them:
            // binding that group's registers ("bind values, not memory", the
            // third finding of "The kernel that waited for itself") stops the
            // scheduler from interleaving the groups, which made it wait for
            // every group in flight at the top of each round.
            bind_group(wb[(d + 1) % D]);
        }
    }
    if (rounds > 0) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int i = (rounds - 1) * D + d;
            if (d > 0) bind_group(wb[d]);
            const bool valid = i < cnt;   // past the part: the last group again, adding zeros
            tiles_group<NT, GB>(wb[d], lds, acol, (uint32_t)(w0 + (valid ? i : last)) * kGroupBlocks, g,
                                valid ? dwidth : 0u, acc);
        }
    }

    // the KW parts of each tile, added in the order 0..KW-1
    if constexpr (KW > 1) {
        lds_barrier();   // every wave is done with the activation copies
        f32x4* red = reinterpret_cast<f32x4*>(lds);
        if (kw > 0) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) red[(wave * NT + tt) * kWave + lane] = acc[tt];
        }
        lds_barrier();
        if (kw == 0) {
            for (int k2 = 1; k2 < KW; ++k2)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    const f32x4 v = red[((wave + k2) * NT + tt) * kWave + lane];
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[tt][r] += v[r];
                }
        }
    }
    if (KP == 1) {
        if (kw == 0 && t < T) store_tile<NT>(acc, Y, N, M, t, g, rn);
        return;
    }

    // KP ranges: partial tile sums to the workspace, then a ticket.  Every
    // access to the workspace is an agent-scope atomic (device-coherent loads
    // and stores, sc1 on gfx950), and each wave waits for its stores to
    // complete before the workgroup takes its ticket; the workgroup that draws
    // the last ticket issues its loads only after the ticket has returned.
    // Agent-scope release and acquire fences (an L2 write-back and an L2
    // invalidate on this chip, both of whole caches) measured 15-140 us per
    // call, and are not needed when every shared access is atomic.
    float* const mine = reinterpret_cast<float*>(part + (((size_t)grp * KP + kp) * RT + rt) * NT * kWave);
    if (kw == 0) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                __hip_atomic_store(mine + (tt * kWave + lane) * 4 + r, acc[tt][r], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's partial sums are stored
    __syncthreads();
    if (threadIdx.x == 0)
        last_ticket = __hip_atomic_fetch_add(tickets + grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                      (uint32_t)(KP - 1);
    __syncthreads();
    if (!last_ticket) return;   // workgroup-uniform
    if (kw == 0 && t < T) {
        f32x4 sum[NT];
        for (int k2 = 0; k2 < KP; ++k2) {
            const float* const src =
                reinterpret_cast<const float*>(part + (((size_t)grp * KP + k2) * RT + rt) * NT * kWave);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                f32x4 v = acc[tt];
                if (k2 != kp) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] = __hip_atomic_load(src + (tt * kWave + lane) * 4 + r, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
                }
                if (k2 == 0) sum[tt] = v;
                else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) sum[tt][r] += v[r];
                }
            }
        }
        store_tile<NT>(sum, Y, N, M, t, g, rn);
    }
    if (threadIdx.x == 0) __hip_atomic_store(tickets + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A resolved configuration of the tiled kernel.
struct TilesPlan {
    int RT, KW, D, KP;   // row tiles and K parts per workgroup, groups in flight per wave, K ranges
    int spw;             // groups per range
    int cs_slots;        // LDS column stride, 16-byte slots (odd)
    size_t lds;          // dynamic LDS per workgroup
    int groups;          // row groups
};

constexpr int kTilesMaxKP = 16;
// The ticket counters sit at the start of the workspace, one per row group,
// at the same place for every shape: a call leaves all of them zero, so
// calls of different shapes can share one workspace (partial sums, whose
// place depends on the shape, follow them and never cover a counter).
constexpr int kTicketSlots = 16384;
constexpr size_t kTicketBytes = kTicketSlots * 4;
constexpr size_t kTilesMaxLds = 160 * 1024 - 256;   // a gfx950 workgroup's LDS, less the ticket flag

// The built (RT, KW, D) configurations (launch_tiles_mp lists the same).
bool tiles_built(int RT, int KW, int D) {
    static const int kBuilt[][3] = {{1, 4, 2}, {1, 4, 4}, {1, 8, 2}, {1, 8, 4}, {1, 16, 2}, {2, 4, 2}, {2, 4, 4},
                                    {2, 2, 4}, {2, 8, 2}, {4, 1, 4}, {4, 2, 2}, {4, 2, 4}, {4, 4, 2}, {4, 4, 4}};
    for (const auto& c : kBuilt)
        if (c[0] == RT && c[1] == KW && c[2] == D) return true;
    return false;
}

bool tiles_plan(int N, int K, int M, int RT, int KW, int D, int KP, TilesPlan& p) {
    const int S = K >> 8;
    if (S < 1 || KP < 1 || KP > kTilesMaxKP || !tiles_built(RT, KW, D)) return false;
    p.RT = RT;
    p.KW = KW;
    p.D = D;
    p.spw = (S + KP - 1) / KP;
    p.KP = (S + p.spw - 1) / p.spw;   // no empty range
    p.cs_slots = kGroupSlots * p.spw + 1;
    const int NT = M > 16 ? 2 : 1;
    const size_t act = (size_t)((M * p.cs_slots + kWave - 1) / kWave) * 1024;
    const size_t red = (size_t)RT * KW * NT * kWave * 16;
    p.lds = act > red ? act : red;
    p.groups = ((N + 15) / 16 + RT - 1) / RT;
    if (p.KP > 1 && p.groups > kTicketSlots) return false;   // one ticket counter per row group
    // LDS of one workgroup; the quotient by the column stride (a multiply-high
    // by ceil(2^32 / stride)) is exact for strides below 2^14 and slots below 2^18
    return p.lds <= kTilesMaxLds && p.cs_slots < (1 << 14) && M * p.cs_slots + kWave < (1 << 18);
}

// Default configuration, from a sweep of every built configuration on MI355X
// over the four decoder-layer shapes at M = 1, 4, 8, 16, 17, 24 (K split 1, 2
// or 4 ways).  K is split over workgroups only when the columns of a whole
// row would not fit a workgroup's LDS (the ticket exchange costs 1.5-2.5 us
// per call): then the ranges are as long as fit, and four row tiles per
// workgroup keep the workgroup count near the CU count.  Otherwise one row
// tile per workgroup (four from 512 row tiles on, which shares each column
// copy between them), with K split over 8 waves, or over 4 waves for K <=
// 4096 up to 16 columns on 256..511 row tiles; two groups in flight per wave.
// Measured (us): 4096x4096 M = 16 / 24 5.60 / 7.17; 14336x4096 9.62 / 14.19;
// 1024x4096 4.78 / 6.29; 4096x14336 M = 8 / 16 / 24 10.61 / 12.21 / 18.25.
void tiles_default(int N, int K, int M, int& RT, int& KW, int& D, int& KP) {
    const int T = (N + 15) / 16;
    const int S = K >> 8;
    const size_t fit = 150 * 1024;   // the columns of one range in LDS
    D = 2;
    KP = 1;
    while (KP < kTilesMaxKP && KP < S && (size_t)M * ((S + KP - 1) / KP) * kGroupSlots * 16 > fit) KP *= 2;
    if (KP > 1) {
        RT = KP >= 4 ? 4 : 2;
        KW = 4;
    } else if (T >= 512) {
        RT = 4;
        KW = 2;
    } else {
        RT = 1;
        KW = (K <= 4096 && M <= 16 && T >= 256) ? 4 : 8;
    }
}

template <int MP, int RT, int KW, int D>
hipError_t launch_tiles_cfg(const TilesPlan& p, const void* Wt, const void* Xq, float* Y, void* ws, int N, int K,
                            int M, hipStream_t s) {
    uint32_t* tickets = reinterpret_cast<uint32_t*>(ws);
    f32x4* part = reinterpret_cast<f32x4*>(reinterpret_cast<uint8_t*>(ws) + kTicketBytes);
    const uint32_t magic = (uint32_t)((((uint64_t)1 << 32) + (uint64_t)p.cs_slots - 1) / (uint64_t)p.cs_slots);
    hipLaunchKernelGGL((k_q4_tiles<MP, RT, KW, D>), dim3(p.groups * p.KP), dim3(64 * RT * KW), p.lds, s,
                       (const uint8_t*)Wt, (const uint8_t*)Xq, Y, tickets, part, N, K, M, p.KP, p.spw, p.cs_slots,
                       magic);
    return hipGetLastError();
}

template <int MP>
hipError_t launch_tiles_mp(const TilesPlan& p, const void* Wt, const void* Xq, float* Y, void* ws, int N, int K,
                           int M, hipStream_t s) {
#define DG_TL(RR, WW, DD) \
    if (p.RT == RR && p.KW == WW && p.D == DD) return launch_tiles_cfg<MP, RR, WW, DD>(p, Wt, Xq, Y, ws, N, K, M, s);
    DG_TL(1, 4, 2) DG_TL(1, 4, 4) DG_TL(1, 8, 2) DG_TL(1, 8, 4) DG_TL(1, 16, 2)
    DG_TL(2, 4, 2) DG_TL(2, 4, 4) DG_TL(2, 2, 4) DG_TL(2, 8, 2)
    DG_TL(4, 1, 4) DG_TL(4, 2, 2) DG_TL(4, 2, 4) DG_TL(4, 4, 2) DG_TL(4, 4, 4)
#undef DG_TL
    return hipErrorInvalidValue;
}

}  // namespace

size_t q4_tiles_bytes(int64_t N, int64_t K) { return (size_t)((N + 15) / 16) * (size_t)(K / 256) * kGroupBytes; }

hipError_t launch_q4_tiles_pack(const void* Wq, void* Wt, int64_t N, int64_t K, hipStream_t s) {
    const int S = (int)(K / 256);
    const int64_t slots = (N + 15) / 16 * S * 144;
    if (slots == 0) return hipSuccess;
    hipLaunchKernelGGL(k_q4_tiles_pack, dim3((unsigned)((slots + 255) / 256)), dim3(256), 0, s, (const uint8_t*)Wq,
                       (uint8_t*)Wt, (int)N, S, slots);
    return hipGetLastError();
}

// The workspace a configuration needs: the ticket counters (64 KiB), then KP x
// groups x RT x NT x 1 KiB of partial tile sums; none when KP = 1.
static size_t tiles_ws_bytes(const TilesPlan& p, int M) {
    if (p.KP == 1) return 0;
    const size_t nt = M > 16 ? 2 : 1;
    return kTicketBytes + (size_t)p.KP * p.groups * p.RT * nt * 1024;
}

// unroll = KP * 1000000 + RT * 10000 + KW * 100 + D (0: the default).
static bool tiles_resolve(int N, int K, int M, int unroll, TilesPlan& p) {
    int RT, KW, D, KP;
    if (unroll) {
        KP = unroll / 1000000;
        RT = (unroll / 10000) % 100;
        KW = (unroll / 100) % 100;
        D = unroll % 100;
    } else {
        tiles_default(N, K, M, RT, KW, D, KP);
    }
    return tiles_plan(N, K, M, RT, KW, D, KP, p);
}

bool q4_tiles_config(int N, int K, int M, int unroll, size_t* ws_bytes) {
    TilesPlan p;
    if (N <= 0 || K <= 0 || M <= 0 || M > 24 || !tiles_resolve(N, K, M, unroll, p)) return false;
    *ws_bytes = tiles_ws_bytes(p, M);
    return true;
}

hipError_t launch_q4_tiles(int M, int unroll, const void* Wt, const void* Xq, float* Y, void* ws, int N, int K,
                           hipStream_t s) {
    TilesPlan p;
    if (!tiles_resolve(N, K, M, unroll, p) || p.lds > device_max_lds_per_block()) return hipErrorInvalidValue;
    if (M <= 16) return launch_tiles_mp<16>(p, Wt, Xq, Y, ws, N, K, M, s);
    return launch_tiles_mp<32>(p, Wt, Xq, Y, ws, N, K, M, s);
}

}  // namespace dg
