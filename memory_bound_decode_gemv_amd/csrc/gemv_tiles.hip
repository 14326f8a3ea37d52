// gemv_tiles.hip -- Q4_0 or Q8_0 x Q8_1 for 1..24 activation columns from
// weights rearranged into 16-row tiles, and those rearrangements.
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
// before unpacking.  The tiled layout holds the blocks' information byte for
// byte (every binary16 scale untouched; every 4-bit code q stored as q XOR 8,
// the two's-complement nibble of q - 8), ordered so that one 16-byte load
// per lane IS the B operand of four consecutive blocks:
//
//   tile t (rows 16t..16t+15) x group s (blocks 8s..8s+7): 2304 bytes at
//   (t * K/256 + s) * 2304:
//     bytes    0..1023: lane l (l = 16g + n) holds, in dword j, code bytes
//                       4g..4g+3 of row 16t+n, block 8s+j (nibbles XOR 8);
//     bytes 1024..2047: the same for blocks 8s+4..8s+7;
//     bytes 2048..2303: row n's eight binary16 scales (blocks 8s..8s+7) at
//                       2048 + 16n, block 8s+i in half i%2 of dword i/2.
//   Rows past N (the last tile's padding) hold code nibbles 0 (q - 8 = 0)
//   and scale 0, so they add exact zeros.
//
// Q8_0 (34-byte blocks: binary16 d, 32 int8 codes) is tiled the same way,
// codes unchanged: a group is 4352 bytes, four KiB of codes (KiB h: lane l
// = 16g + n holds code dwords g and 4 + g of row n, blocks 2h and 2h + 1),
// then the 256 bytes of scales; a lane's codes are its B operands as loaded.
//
// The matrix-core arithmetic keeps the exact integer block sums of the
// row-major kernels: per block, one v_mfma_i32_16x16x32_i8 of the 16
// columns' q8 codes against 16 (q - 8) of the 16 rows (the signed nibbles
// masked in place, no offset term), and the d8 * d4 products from one
// v_mfma_f32_16x16x16_f16 (exact in fp32); the int32 block sums are
// converted and scaled in fp32.  Lane group g carries k-slots 4g..4g+3 (low
// nibbles of code dword g) and 16+4g..16+4g+3 (high nibbles), with the
// matching activation code dwords g and 4 + g.
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
constexpr int kGroupSlots = 18;      // 16-byte slots of one column's Q8_1 blocks per group (8 x 36 / 16)
constexpr uint32_t kHiNib = 0xF0F0F0F0u;

// Tiled weight formats.  A group (16 rows x 8 blocks) is kCodeLoads KiB of
// codes in lane order, then 256 bytes of scales (16 per row); a lane loads
// kCodeLoads + 1 16-byte vectors per group.  bops gives the lane's B operand
// dwords of block i for its low k-slots (activation code dword g) and high
// k-slots (dword 4 + g); kUnscale divides out the factor the integer operands
// and the scale products (4 d8 d4) carry.
struct TilesQ4_0 {
    static constexpr int kCodeLoads = 2;
    static constexpr int kGroupBytes = 2304;     // 16 rows x 8 blocks x 18 bytes
    static constexpr float kUnscale = 1.0f / 64.0f;   // 16 (q - 8) codes, 4 d8 d4
    __device__ __forceinline__ static void bops(const u32x4* w, int i, uint32_t& lo, uint32_t& hi) {
        const u32x4 v = w[i >> 2];
        const uint32_t c = (i & 3) == 0 ? v.x : (i & 3) == 1 ? v.y : (i & 3) == 2 ? v.z : v.w;
        lo = (c << 4) & kHiNib;   // signed nibbles (codes q XOR 8) in the high half of each byte: 16 (q - 8)
        hi = c & kHiNib;
    }
};
struct TilesQ8_0 {
    static constexpr int kCodeLoads = 4;
    static constexpr int kGroupBytes = 4352;     // 16 rows x 8 blocks x 34 bytes
    static constexpr float kUnscale = 1.0f / 4.0f;    // codes as they are, 4 d8 d4
    __device__ __forceinline__ static void bops(const u32x4* w, int i, uint32_t& lo, uint32_t& hi) {
        const u32x4 v = w[i >> 1];
        lo = (i & 1) ? v.z : v.x;
        hi = (i & 1) ? v.w : v.y;
    }
};

// ---------------------------------------------------------------------------
// Rearrangement: one thread per 16-byte slot of the tiled layout (144 per
// group).  Source reads are 2-byte loads (block fields sit at even offsets).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
k_q4_tiles_pack(const uint8_t* __restrict__ Wq, uint8_t* __restrict__ Wt, int N, int S, int64_t slots) {
    constexpr int kGroupBytes = TilesQ4_0::kGroupBytes;
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
                d[j] = ((uint32_t)p[0] | ((uint32_t)p[1] << 16)) ^ 0x88888888u;   // q -> q - 8, signed nibbles
            } else {
                d[j] = 0u;   // padding rows: q - 8 = 0
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

// Q8_0: 272 slots per group (256 of codes, 16 of scales).
__global__ void __launch_bounds__(256)
k_q8_tiles_pack(const uint8_t* __restrict__ Wq, uint8_t* __restrict__ Wt, int N, int S, int64_t slots) {
    constexpr int kGroupBytes = TilesQ8_0::kGroupBytes;
    const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= slots) return;
    const int64_t ts = u / 272;                 // tile * S + group
    const int k = (int)(u - ts * 272);
    const int64_t t = ts / S;
    const int s = (int)(ts - t * S);
    const size_t row_bytes = (size_t)S * kGroupBlocks * 34;
    uint32_t d[4] = {0u, 0u, 0u, 0u};
    if (k < 256) {
        const int h = k >> 6, l = k & 63, g = l >> 4, n = l & 15;
        const int64_t row = t * 16 + n;
        if (row < N) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {   // blocks 2h, 2h + 1: code dwords g, 4 + g
                const int b = kGroupBlocks * s + 2 * h + (j >> 1);
                const uint16_t* p = reinterpret_cast<const uint16_t*>(
                    Wq + (size_t)row * row_bytes + (size_t)b * 34 + 2 + 4 * (g + 4 * (j & 1)));
                d[j] = (uint32_t)p[0] | ((uint32_t)p[1] << 16);
            }
        }
    } else {
        const int n = k - 256;
        const int64_t row = t * 16 + n;
        if (row < N) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint8_t* r = Wq + (size_t)row * row_bytes + (size_t)(kGroupBlocks * s + 2 * j) * 34;
                d[j] = (uint32_t)*reinterpret_cast<const uint16_t*>(r) |
                       ((uint32_t)*reinterpret_cast<const uint16_t*>(r + 34) << 16);
            }
        }
    }
    *reinterpret_cast<u32x4*>(Wt + (size_t)ts * kGroupBytes + (size_t)k * 16) = u32x4{d[0], d[1], d[2], d[3]};
}

// One group of a lane's weights: kCodeLoads 16-byte loads of codes (its B
// operands) and one of its row's eight scales.
template <class TF>
__device__ __forceinline__ void load_group(const uint8_t* __restrict__ g0, int lane, int rn,
                                           u32x4 (&w)[TF::kCodeLoads + 1]) {
#pragma unroll
    for (int c = 0; c < TF::kCodeLoads; ++c)
        w[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(g0 + c * 1024 + lane * 16));
    w[TF::kCodeLoads] =
        __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(g0 + TF::kCodeLoads * 1024 + rn * 16));
}

// Column tiles of a launch with MP padded columns: a full tile of 16 columns
// (MP >= 16) and a pair tile of 8 columns from c0 = MP - 8 (MP = 8 or 24).
// The pair tile computes two blocks per matrix-core instruction: a
// v_mfma_i32_16x16x64_i8 (as fast as the 32-deep one on gfx950) whose 64
// k-slots hold both blocks, A rows 0..7 carrying the 8 columns' codes of the
// first block (zeros in the second block's k-slots, read from a zero column
// in LDS) and rows 8..15 those of the second: output row m' is the block sum
// of column c0 + m' % 8 and block i + m' / 8.  Per output that is half the
// instructions of a 16-column tile with eight columns unused.
template <int MP>
struct TileSet {
    static constexpr int kFull = MP >= 16 ? 1 : 0;
    static constexpr int kPair = (MP == 8 || MP == 24) ? 1 : 0;
    // f32x4 accumulators per lane: the full tile's even and odd blocks apart
    // (so that every column is summed in the same order as the pair tile's:
    // even blocks, odd blocks, then the two sums), then the pair tile's
    static constexpr int kNA = 2 * kFull + kPair;
    static constexpr int kPairAcc = 2 * kFull;
    static constexpr int kC0 = MP - 8;          // first column of the pair tile
};

// Per-lane LDS byte offsets of the A operands within the column copy.
struct ALanes {
    uint32_t full;   // the full tile: column rn
    uint32_t p01;    // pair tile, first block's k-slots: column c0 + rn (rn < 8), else the zero column
    uint32_t p23;    // pair tile, second block's k-slots: column c0 + rn - 8 (rn >= 8), else the zero column
    uint32_t ps;     // pair tile, d8: this row's column, one block further for rn >= 8
    uint32_t sel;    // byte selector: that d8 into the low (rn < 8) or high half of a dword
};

// One group of 8 blocks: operands, matrix-core products, fp32 scaling into
// acc, which gathers 1 / TF::kUnscale times the sums (divided out at the
// store):
//  * B (weights), Q4_0: the tiled codes are signed nibbles (q - 8), so
//    masking the high nibbles of a code dword, and of the dword shifted left
//    by 4, gives 16 (q - 8) as int8 for the lane's 8 k-slots: one MFMA per
//    block (per two blocks in the pair tile) gives 16 times the exact block
//    sums (|16 S| < 2^20), with no offset term; Q8_0: the codes as loaded;
//  * the scale products come from one v_mfma_f32_16x16x16_f16 per block (per
//    two blocks in the pair tile) in which B is the lane's raw pair of scale
//    dwords (the d4 of four blocks, one per k-slot, repeated in all four lane
//    groups) and A carries each output row's d8 at the k-slot of its block
//    in every lane group, zeros elsewhere: each output is 4 d8 d4, exact in
//    fp32 (binary16 products are exact, and so are sums of four equal ones).
// blk is the group's first block within the LDS copy of the columns.
template <class TF, int MP>
__device__ __forceinline__ void tiles_group(const u32x4 (&w)[TF::kCodeLoads + 1], const uint8_t* lds,
                                            const ALanes& al, uint32_t blk, int g,
                                            f32x4 (&acc)[TileSet<MP>::kNA]) {
    using TS = TileSet<MP>;
    const u32x4 sv = w[TF::kCodeLoads];
    const f16x4 d4q[2] = {__builtin_bit_cast(f16x4, u32x2{sv.x, sv.y}),    // blocks 0..3
                          __builtin_bit_cast(f16x4, u32x2{sv.z, sv.w})};   // blocks 4..7
    uint32_t blo[8], bhi[8];   // B operand dwords of the lane's low and high k-slots
#pragma unroll
    for (int i = 0; i < kGroupBlocks; ++i) TF::bops(w, i, blo[i], bhi[i]);
    if constexpr (TS::kFull) {
#pragma unroll
        for (int i = 0; i < kGroupBlocks; ++i) {
            const uint32_t* ab = reinterpret_cast<const uint32_t*>(lds + al.full + (blk + i) * kQ81Bytes);
            const long aop = (long)((uint64_t)ab[1 + g] | ((uint64_t)ab[5 + g] << 32));
            const long bop = (long)((uint64_t)blo[i] | ((uint64_t)bhi[i] << 32));
            const uint32_t h = (i & 1) ? ab[0] << 16 : ab[0] & 0xFFFFu;   // d8, in the half of k-slot i % 4
            const f16x4 a8 = __builtin_bit_cast(f16x4, (i & 2) ? u32x2{0u, h} : u32x2{h, 0u});
            const i32x4 dsum = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, bop, i32x4{0, 0, 0, 0}, 0, 0, 0);
            const f32x4 sc = __builtin_amdgcn_mfma_f32_16x16x16f16(a8, d4q[i >> 2], f32x4{0.0f, 0.0f, 0.0f, 0.0f},
                                                                   0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i & 1][r] = fmaf((float)dsum[r], sc[r], acc[i & 1][r]);
        }
    }
    if constexpr (TS::kPair) {
#pragma unroll
        for (int i = 0; i < kGroupBlocks; i += 2) {
            const uint32_t* x01 = reinterpret_cast<const uint32_t*>(lds + al.p01 + (blk + i) * kQ81Bytes);
            const uint32_t* x23 = reinterpret_cast<const uint32_t*>(lds + al.p23 + (blk + i + 1) * kQ81Bytes);
            const i32x4 aop = {(int)x01[1 + g], (int)x01[5 + g], (int)x23[1 + g], (int)x23[5 + g]};
            const i32x4 bop = {(int)blo[i], (int)bhi[i], (int)blo[i + 1], (int)bhi[i + 1]};
            const uint32_t d8 = *reinterpret_cast<const uint32_t*>(lds + al.ps + (blk + i) * kQ81Bytes);
            const uint32_t h = __builtin_amdgcn_perm(0u, d8, al.sel);   // k-slot i % 4 + (row >= 8)
            const f16x4 a8 = __builtin_bit_cast(f16x4, (i & 2) ? u32x2{0u, h} : u32x2{h, 0u});
            const i32x4 dsum = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop, bop, i32x4{0, 0, 0, 0}, 0, 0, 0);
            const f32x4 sc = __builtin_amdgcn_mfma_f32_16x16x16f16(a8, d4q[i >> 2], f32x4{0.0f, 0.0f, 0.0f, 0.0f},
                                                                   0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[TS::kPairAcc][r] = fmaf((float)dsum[r], sc[r], acc[TS::kPairAcc][r]);
        }
    }
}

// Marks a group's registers as written here (an empty asm): arithmetic on
// them cannot move above this point, and its loads are waited for here.
template <int L>
__device__ __forceinline__ void bind_group(u32x4 (&w)[L]) {
    static_assert(L == 3 || L == 5, "three or five loads per group");
    if constexpr (L == 3) asm volatile("" : "+v"(w[0]), "+v"(w[1]), "+v"(w[2])::"memory");
    else asm volatile("" : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(w[4])::"memory");
}

// Stores the tile's outputs (unscaled).  The full tile adds its even- and
// odd-block sums; the pair tile's sit in lane groups g and g + 2 (output rows
// m' and m' + 8).  All 64 lanes of the wave call this.
template <class TF, int MP>
__device__ __forceinline__ void store_tile(const f32x4 (&acc)[TileSet<MP>::kNA], float* __restrict__ Y, int N, int M,
                                           int t, int g, int rn) {
    constexpr float kUnscale = TF::kUnscale;
    using TS = TileSet<MP>;
    const int n = t * 16 + rn;
    f32x4 pr = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (TS::kPair) {
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[r] = acc[TS::kPairAcc][r] + __shfl_xor(acc[TS::kPairAcc][r], 32);
    }
    if (n >= N) return;
    if constexpr (TS::kFull) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = g * 4 + r;
            if (m < M) Y[(size_t)m * N + n] = (acc[0][r] + acc[1][r]) * kUnscale;
        }
    }
    if constexpr (TS::kPair) {
        if (g < 2) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = TS::kC0 + g * 4 + r;
                if (m < M) Y[(size_t)m * N + n] = pr[r] * kUnscale;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// The GEMV.  MP = 8 (M <= 8: one pair tile), 16 (one full tile) or 24 (a
// full tile and a pair tile); columns past M re-read column M - 1, their
// results dropped.
// ---------------------------------------------------------------------------
template <class TF, int MP, int RT, int KW, int D>
__global__ void __launch_bounds__(64 * RT * KW)
k_tiles(const uint8_t* __restrict__ Wt, const uint8_t* __restrict__ Xq, float* __restrict__ Y,
           uint32_t* __restrict__ tickets, f32x4* __restrict__ part, int N, int K, int M, int KP, int spw,
           int cs_slots, uint32_t cs_magic, int CS, int groups, int pre) {
    using TS = TileSet<MP>;
    constexpr int NA = TS::kNA;
    constexpr int W = RT * KW;
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
    int grp, kp, cs = 0;
    if (CS == 1) {
        grp = (int)blockIdx.x / KP;
        kp = (int)blockIdx.x - grp * KP;
    } else {
        // Column slices: the CS workgroups of a (row group, K range) unit take
        // Mh = ceil(M / CS) columns each and sit 8 workgroup ids apart, so the
        // round-robin placement puts them on one XCD, whose L2 serves their
        // shared weight rows once.  Units are padded to whole blocks of 8.
        const int b = (int)blockIdx.x;
        const int hi = b >> 3;
        cs = hi % CS;
        const int u = (hi / CS) * 8 + (b & 7);
        if (u >= groups * KP) return;   // workgroup-uniform, before any barrier
        grp = u / KP;
        kp = u - grp * KP;
        const int Mh = (M + CS - 1) / CS;
        const int mc0 = cs * Mh;
        Xq += (size_t)mc0 * (size_t)(K >> 5) * kQ81Bytes;
        Y += (size_t)mc0 * (size_t)N;
        M = min(Mh, M - mc0);
    }
    const int s0 = kp * spw;                       // first group of the workgroup's range
    const int ns = min(spw, S - s0);               // groups in the range (>= 1)
    const int spk = (ns + KW - 1) / KW;
    const int w0 = kw * spk;                       // the wave's part: groups w0 .. w0 + cnt - 1 of the range
    const int cnt = max(0, min(spk, ns - w0));     // wave-uniform
    const int t = grp * RT + rt;
    const int tc = t < T ? t : T - 1;
    constexpr int kGroupBytes = TF::kGroupBytes;
    constexpr int L = TF::kCodeLoads + 1;   // 16-byte loads per lane and group
    const uint8_t* const wbase = Wt + ((size_t)tc * S + s0 + (cnt > 0 ? w0 : 0)) * kGroupBytes;
    const int last = cnt > 0 ? cnt - 1 : 0;

    // (1) the activation columns of the range, copied into LDS by DMA, and a
    // wait for them; then (2) the first D groups of this wave's weights (past
    // its part: its last group again, never used).  The wait is the builtin
    // (not inline asm) and waits for everything: only then does the
    // compiler's own wait counting know that no copy into LDS is outstanding.
    // With copies possibly outstanding it treats the counter as out of order
    // and waits for every load before each use (measured: vmcnt(0) at the top
    // of every round of the loop).  Waiting for the copies before the first
    // weight loads leaves those loads to the compiler's exact counting, so the
    // first group's products start when that group has arrived; with the
    // weights issued before the wait (pre = 0, kept for measurements) they
    // start when all D have.  Measured 2-16% faster on most shapes.
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
        if constexpr (TS::kPair) {   // the zero column after the copies (its used slots)
            u32x4* const z = reinterpret_cast<u32x4*>(lds + copies * 1024);
            for (int e = wave * kWave + lane; e < used; e += W * kWave) z[e] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    u32x4 wb[D][L];
    if (pre) {
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the copies only
        lds_barrier();                        // every other wave's copies have landed too
#pragma unroll
        for (int d = 0; d < D; ++d)
            load_group<TF>(wbase + (size_t)(d < cnt ? d : last) * kGroupBytes, lane, rn, wb[d]);
    } else {
#pragma unroll
        for (int d = 0; d < D; ++d)
            load_group<TF>(wbase + (size_t)(d < cnt ? d : last) * kGroupBytes, lane, rn, wb[d]);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt, lgkmcnt at their maximum: no wait
        lds_barrier();   // every other wave's copies have landed too
    }

    // A operand offsets (columns past M: column M - 1 again, results dropped)
    ALanes al;
    {
        const uint32_t stride = (uint32_t)cs_slots * 16u;
        const uint32_t zero = (uint32_t)((M * cs_slots + kWave - 1) / kWave) * 1024u;   // the zero column
        al.full = (uint32_t)(rn < M ? rn : M - 1) * stride;
        const int c = TS::kC0 + (rn & 7);
        const uint32_t pc = (uint32_t)(c < M ? c : M - 1) * stride;
        const bool hi = rn >= 8;
        al.p01 = hi ? zero : pc;
        al.p23 = hi ? pc : zero;
        al.ps = pc + (hi ? (uint32_t)kQ81Bytes : 0u);
        al.sel = hi ? 0x01000C0Cu : 0x0C0C0100u;
    }
    f32x4 acc[NA];
#pragma unroll
    for (int a = 0; a < NA; ++a) acc[a] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // D groups per round; the loads of the next round are issued right after
    // each group's products, with no branch between them, so the compiler's
    // waits count exactly the D - 1 groups still in flight.  The last round
    // is peeled (no loads).
    const int rounds = (cnt + D - 1) / D;
    for (int rd = 0; rd + 1 < rounds; ++rd) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int i = rd * D + d;
            tiles_group<TF, MP>(wb[d], lds, al, (uint32_t)(w0 + i) * kGroupBlocks, g, acc);
            const int nx = i + D;
            load_group<TF>(wbase + (size_t)(nx < cnt ? nx : last) * kGroupBytes, lane, rn, wb[d]);
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
            if (i < cnt)   // wave-uniform; no loads follow, so the branch costs no wait
                tiles_group<TF, MP>(wb[d], lds, al, (uint32_t)(w0 + i) * kGroupBlocks, g, acc);
        }
    }

    // the KW parts of each tile, added in the order 0..KW-1
    if constexpr (KW > 1) {
        lds_barrier();   // every wave is done with the activation copies
        f32x4* red = reinterpret_cast<f32x4*>(lds);
        if (kw > 0) {
#pragma unroll
            for (int a = 0; a < NA; ++a) red[(wave * NA + a) * kWave + lane] = acc[a];
        }
        lds_barrier();
        if (kw == 0) {
            for (int k2 = 1; k2 < KW; ++k2)
#pragma unroll
                for (int a = 0; a < NA; ++a) {
                    const f32x4 v = red[((wave + k2) * NA + a) * kWave + lane];
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[a][r] += v[r];
                }
        }
    }
    if (KP == 1) {
        if (kw == 0 && t < T) store_tile<TF, MP>(acc, Y, N, M, t, g, rn);
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
    const int slot = grp * CS + cs;   // this slice's ticket counter and partial sums
    float* const mine = reinterpret_cast<float*>(part + (((size_t)slot * KP + kp) * RT + rt) * NA * kWave);
    if (kw == 0) {
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                __hip_atomic_store(mine + (a * kWave + lane) * 4 + r, acc[a][r], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's partial sums are stored
    __syncthreads();
    if (threadIdx.x == 0)
        last_ticket = __hip_atomic_fetch_add(tickets + slot, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                      (uint32_t)(KP - 1);
    __syncthreads();
    if (!last_ticket) return;   // workgroup-uniform
    if (kw == 0 && t < T) {
        f32x4 sum[NA];
        for (int k2 = 0; k2 < KP; ++k2) {
            const float* const src =
                reinterpret_cast<const float*>(part + (((size_t)slot * KP + k2) * RT + rt) * NA * kWave);
#pragma unroll
            for (int a = 0; a < NA; ++a) {
                f32x4 v = acc[a];
                if (k2 != kp) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] = __hip_atomic_load(src + (a * kWave + lane) * 4 + r, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
                }
                if (k2 == 0) sum[a] = v;
                else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) sum[a][r] += v[r];
                }
            }
        }
        store_tile<TF, MP>(sum, Y, N, M, t, g, rn);
    }
    if (threadIdx.x == 0) __hip_atomic_store(tickets + slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// f32x4 accumulators per lane for M columns (TileSet<MP>::kNA).
int tiles_accumulators(int M) { return M <= 8 ? 1 : M <= 16 ? 2 : 3; }

// A resolved configuration of the tiled kernel.
struct TilesPlan {
    int RT, KW, D, KP;   // row tiles and K parts per workgroup, groups in flight per wave, K ranges
    int CS;              // column slices per row group and K range
    int pre;
    int Mh;              // columns per workgroup: ceil(M / CS)
    int spw;             // groups per range
    int cs_slots;        // LDS column stride, 16-byte slots (odd)
    size_t lds;          // dynamic LDS per workgroup
    int groups;          // row groups
};

constexpr int kTilesMaxKP = 16;
constexpr int kTilesMaxCS = 8;
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

bool tiles_plan(int N, int K, int M, int RT, int KW, int D, int KP, int CS, TilesPlan& p) {
    const int S = K >> 8;
    if (S < 1 || KP < 1 || KP > kTilesMaxKP || !tiles_built(RT, KW, D)) return false;
    if (CS < 1 || CS > kTilesMaxCS) return false;
    p.RT = RT;
    p.KW = KW;
    p.D = D;
    p.CS = CS;
    p.Mh = (M + CS - 1) / CS;
    if ((CS - 1) * p.Mh >= M) return false;   // every slice has columns
    M = p.Mh;                                 // a workgroup's columns
    p.spw = (S + KP - 1) / KP;
    p.KP = (S + p.spw - 1) / p.spw;   // no empty range
    p.cs_slots = kGroupSlots * p.spw + 1;
    const int NA = tiles_accumulators(M);
    const bool pair = M <= 8 || M > 16;
    const size_t act = (size_t)((M * p.cs_slots + kWave - 1) / kWave) * 1024 + (pair ? (size_t)p.cs_slots * 16 : 0);
    const size_t red = (size_t)RT * KW * NA * kWave * 16;
    p.lds = act > red ? act : red;
    p.groups = ((N + 15) / 16 + RT - 1) / RT;
    if (p.KP > 1 && p.groups * CS > kTicketSlots) return false;   // one ticket counter per row group and slice
    // LDS of one workgroup; the quotient by the column stride (a multiply-high
    // by ceil(2^32 / stride)) is exact for strides below 2^14 and slots below 2^18
    return p.lds <= kTilesMaxLds && p.cs_slots < (1 << 14) && M * p.cs_slots + kWave < (1 << 18);
}

// Default configuration, from sweeps of every built configuration on MI355X
// over the four decoder-layer shapes (1024, 4096 and 14336 rows of 4096
// columns, 4096 rows of 14336) at M = 1..24, with K split 1..4 ways, the
// columns in 2..8 slices, and both.
//
// Column slices first.  Below 128 row tiles one workgroup per row group
// leaves most of the chip idle: M / 2 slices, at most 4, of 8 waves over K.
// Below 512 row tiles and past 8 columns, 2 slices.  Where the columns of
// whole rows do not fit a workgroup's LDS, 2 slices (Q4_0: 3 when 2 do not
// fit) in place of a K split: the slices of a row group read each weight
// byte once from HBM and again from their XCD's L2, and exchange nothing.
// More slices than that on the larger shapes were 40-100% slower (3 to 8
// slices) with the same HBM traffic: every slice still moves every weight
// byte of its rows into its CU, and the waves are latency-bound.  A slice
// whose columns take more than half the LDS (one workgroup per CU) gets two
// row tiles per workgroup over 8 K parts (Q8_0: 4), or four over 4 for 3
// slices; other slices two row tiles over 4 parts (below 128 row tiles one
// over 8).  When even the slices do not fit, K is split over workgroups as
// well (the ticket exchange costs 1.5-2.5 us per call), in 2 column slices:
// ranges as long as fit, four row tiles per workgroup over 2 waves (two over
// 4 when a row group has only two workgroups).  Without slices or a split:
// from 512 row tiles on, four row tiles over K in 2 parts to 8 columns and in
// 4 beyond (Q8_0: two over 4 parts to 16 columns, four over 2 beyond);
// below 512, one row tile over K in 8 parts.  Two groups in flight per wave.
void tiles_default(bool q8, int N, int K, int M, int& RT, int& KW, int& D, int& KP, int& CS) {
    const int T = (N + 15) / 16;
    const int S = K >> 8;
    D = 2;
    KP = 1;
    int want = T < 128 ? std::min(4, std::max(1, M / 2)) : (T < 512 && M > 8) ? 2 : 1;
    while (want > 1 && (want - 1) * ((M + want - 1) / want) >= M) --want;   // no empty slice
    const int cand[3] = {want, std::max(want, 2), q8 ? 0 : std::max(want, 3)};
    TilesPlan p;
    CS = 0;
    for (int c : cand)
        if (c > 0 && tiles_plan(N, K, M, 1, 4, 2, 1, c, p)) {
            CS = c;
            break;
        }
    if (CS > 1) {
        if (p.lds > kTilesMaxLds / 2) {
            RT = CS == 3 ? 4 : 2;
            KW = CS == 3 || q8 ? 4 : 8;
        } else if (T < 128) {
            RT = 1;
            KW = 8;
        } else {
            RT = 2;
            KW = 4;
        }
        return;
    }
    if (CS == 1) {
        if (T >= 512) {
            RT = q8 && M > 16 ? 4 : q8 ? 2 : 4;
            KW = q8 ? (M > 16 ? 2 : 4) : (M <= 8 ? 2 : 4);
        } else {
            RT = 1;
            KW = 8;
        }
        return;
    }
    CS = M >= 2 ? 2 : 1;
    const int Mh = (M + CS - 1) / CS;
    const size_t fit = 150 * 1024;   // the columns of one range in LDS
    while (KP < kTilesMaxKP && KP < S && (size_t)Mh * ((S + KP - 1) / KP) * kGroupSlots * 16 > fit) KP *= 2;
    RT = KP * CS >= 4 ? 4 : 2;
    KW = KP * CS >= 4 ? 2 : 4;
}

template <class TF, int MP, int RT, int KW, int D>
hipError_t launch_tiles_cfg(const TilesPlan& p, const void* Wt, const void* Xq, float* Y, void* ws, int N, int K,
                            int M, hipStream_t s) {
    uint32_t* tickets = reinterpret_cast<uint32_t*>(ws);
    f32x4* part = reinterpret_cast<f32x4*>(reinterpret_cast<uint8_t*>(ws) + kTicketBytes);
    const uint32_t magic = (uint32_t)((((uint64_t)1 << 32) + (uint64_t)p.cs_slots - 1) / (uint64_t)p.cs_slots);
    const int grid = p.CS == 1 ? p.groups * p.KP : (p.groups * p.KP + 7) / 8 * 8 * p.CS;
    hipLaunchKernelGGL((k_tiles<TF, MP, RT, KW, D>), dim3(grid), dim3(64 * RT * KW), p.lds, s, (const uint8_t*)Wt,
                       (const uint8_t*)Xq, Y, tickets, part, N, K, M, p.KP, p.spw, p.cs_slots, magic, p.CS,
                       p.groups, p.pre);
    return hipGetLastError();
}

// Instantiations that would spill (a 16-wave workgroup has 128 VGPRs per
// lane; Q8_0 holds five loads per group, and 24 columns three accumulators)
// are not built; asking for one is an argument error.
template <class TF, int MP, int RT, int KW, int D>
constexpr bool tiles_instantiated() {
    return !(TF::kCodeLoads == 4 && MP == 24 && RT * KW == 16 && D == 4);
}

template <class TF, int MP>
hipError_t launch_tiles_mp(const TilesPlan& p, const void* Wt, const void* Xq, float* Y, void* ws, int N, int K,
                           int M, hipStream_t s) {
#define DG_TL(RR, WW, DD)                                                              \
    if constexpr (tiles_instantiated<TF, MP, RR, WW, DD>())                            \
        if (p.RT == RR && p.KW == WW && p.D == DD)                                     \
            return launch_tiles_cfg<TF, MP, RR, WW, DD>(p, Wt, Xq, Y, ws, N, K, M, s);
    DG_TL(1, 4, 2) DG_TL(1, 4, 4) DG_TL(1, 8, 2) DG_TL(1, 8, 4) DG_TL(1, 16, 2)
    DG_TL(2, 4, 2) DG_TL(2, 4, 4) DG_TL(2, 2, 4) DG_TL(2, 8, 2)
    DG_TL(4, 1, 4) DG_TL(4, 2, 2) DG_TL(4, 2, 4) DG_TL(4, 4, 2) DG_TL(4, 4, 4)
#undef DG_TL
    return hipErrorInvalidValue;
}

template <class TF>
hipError_t launch_tiles_fmt(const TilesPlan& p, const void* Wt, const void* Xq, float* Y, void* ws, int N, int K,
                            int M, hipStream_t s) {
    if (p.Mh <= 8) return launch_tiles_mp<TF, 8>(p, Wt, Xq, Y, ws, N, K, M, s);
    if (p.Mh <= 16) return launch_tiles_mp<TF, 16>(p, Wt, Xq, Y, ws, N, K, M, s);
    return launch_tiles_mp<TF, 24>(p, Wt, Xq, Y, ws, N, K, M, s);
}

}  // namespace

size_t tiles_bytes(bool q8, int64_t N, int64_t K) {
    return (size_t)((N + 15) / 16) * (size_t)(K / 256) * (q8 ? TilesQ8_0::kGroupBytes : TilesQ4_0::kGroupBytes);
}

hipError_t launch_tiles_pack(bool q8, const void* Wq, void* Wt, int64_t N, int64_t K, hipStream_t s) {
    const int S = (int)(K / 256);
    const int64_t slots = (N + 15) / 16 * S * (q8 ? 272 : 144);
    if (slots == 0) return hipSuccess;
    hipLaunchKernelGGL(q8 ? k_q8_tiles_pack : k_q4_tiles_pack, dim3((unsigned)((slots + 255) / 256)), dim3(256), 0,
                       s, (const uint8_t*)Wq, (uint8_t*)Wt, (int)N, S, slots);
    return hipGetLastError();
}

// The workspace a configuration needs: the ticket counters (64 KiB), then KP x
// groups x CS x RT x NA x 1 KiB of partial tile sums; none when KP = 1.
static size_t tiles_ws_bytes(const TilesPlan& p) {
    if (p.KP == 1) return 0;
    return kTicketBytes + (size_t)p.KP * p.groups * p.CS * p.RT * tiles_accumulators(p.Mh) * 1024;
}

// unroll = CS * 100000000 + KP * 1000000 + RT * 10000 + KW * 100 + D (0: the
// default; CS 0 means 1).
static bool tiles_resolve(bool q8, int N, int K, int M, int unroll, TilesPlan& p) {
    int RT, KW, D, KP, CS;
    if (unroll) {
        CS = unroll / 100000000;
        CS = CS ? CS : 1;
        KP = (unroll / 1000000) % 100;
        RT = (unroll / 10000) % 100;
        KW = (unroll / 100) % 100;
        D = unroll % 100;
    } else {
        tiles_default(q8, N, K, M, RT, KW, D, KP, CS);
    }
    const int late = D >= 10;   // D + 10: the other prologue order (measurements only)
    if (late) D -= 10;
    const bool ok = tiles_plan(N, K, M, RT, KW, D, KP, CS, p);
    p.pre = !late;
    return ok;
}

bool tiles_config(bool q8, int N, int K, int M, int unroll, size_t* ws_bytes) {
    TilesPlan p;
    if (N <= 0 || K <= 0 || M <= 0 || M > 24 || !tiles_resolve(q8, N, K, M, unroll, p)) return false;
    *ws_bytes = tiles_ws_bytes(p);
    return true;
}

hipError_t launch_tiles(bool q8, int M, int unroll, const void* Wt, const void* Xq, float* Y, void* ws, int N, int K,
                        hipStream_t s) {
    TilesPlan p;
    if (!tiles_resolve(q8, N, K, M, unroll, p) || p.lds > device_max_lds_per_block()) return hipErrorInvalidValue;
    return q8 ? launch_tiles_fmt<TilesQ8_0>(p, Wt, Xq, Y, ws, N, K, M, s)
              : launch_tiles_fmt<TilesQ4_0>(p, Wt, Xq, Y, ws, N, K, M, s);
}

}  // namespace dg
