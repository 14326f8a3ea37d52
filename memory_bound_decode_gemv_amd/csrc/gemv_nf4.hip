// gemv_nf4.hip -- NF4 x bfloat16 GEMV for one activation column, and the NF4
// quantiser.
//
// The lookup-table 4-bit M = 1 GEMV of the bitsandbytes issue on 70B 4-bit
// decode: each weight is a 4-bit index into a 16-entry float table, scaled by
// its block's absmax, against bfloat16 activations, in float arithmetic.
// Layout (codes: two per byte, the first weight in the high nibble; absmax:
// float32 per block of B weights) as documented in include/decodegemv.h.
//
// The page's kernel dequantises every weight through a float table in shared
// memory.  On gfx950 the per-weight work is what would bound this kernel, so
// here every code BYTE -- two weights -- is one lookup:
//   * each workgroup builds in LDS a 256-entry table indexed by the code
//     byte; an entry holds the two weights' table values as binary16 pairs,
//     each value scaled by a power of two 2^st (largest |table| near 2^14)
//     and split into a high part (rounded to binary16) and a low part (the
//     rest, rounded to binary16): 22 significant bits, within about 2^-23 of
//     the float value;
//   * each lane converts its 32 activations of a unit to binary16 once,
//     scaled by a power of two 2^sx that puts their largest near 2^14: a
//     bfloat16 value (8 significant bits) converts exactly unless it lies
//     some 2^28 below that largest;
//   * two v_dot2_f32_f16 multiply the pair with the two activations (one
//     dword of binary16 x) and add into fp32 -- the products are exact -- and
//     the unit's sum is scaled back by 2^-st, 2^-sx and its absmax: the float
//     GEMV up to fp32 rounding;
//   * the table is replicated TC times (copy = lane % TC) so that the 8-byte
//     lookups of 16 (TC = 16) or 32 lanes fall in distinct banks; with 32
//     copies an entry spans 256 bytes and one byte permute per code byte
//     forms the lookup address.
// The K of a row is split over the S = K/2048 waves of a workgroup: wave w
// owns weights 2048w .. 2048w + 2047 of every row the workgroup takes, a lane
// 32 of them -- 16 code bytes, one 16-byte load (the wave's 64 lanes read 1 KiB
// of consecutive bytes), and its block's absmax -- so a lane holds only 32
// activations and the kernel keeps many waves per CU.  Each wave streams its
// slice of successive rows with AHEAD rows of loads in flight, straight to
// registers: with nothing but plain loads in flight the compiler's own vmcnt
// waits are exact (LDS-DMA copies in flight would make it wait for all of
// them before every table lookup).  The waves' per-row partials meet in LDS
// every 64 rows and are added in unit order, so results do not depend on the
// launch shape.
#include "dg_internal.h"
#include "q4_common.h"

namespace dg {
namespace {

using namespace q4;

constexpr int kUnitWeights = 2048;    // weights per unit: 64 lanes x 32
constexpr int kUnitCodes = 1024;      // code bytes per unit
constexpr int kMaxUnits = 16;         // K <= 32768: one wave per unit, 1024 threads

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);   // round to nearest even
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }

// 2^e as a float, e clamped to the normal range.
__device__ __forceinline__ float pow2f(int e) {
    e = e < -126 ? -126 : (e > 127 ? 127 : e);
    return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
}

// The power of two that brings a biased binary32/bfloat16 exponent field to 14.
__device__ __forceinline__ int scale_exp(uint32_t biased) { return 14 - ((int)biased - 127); }


// Loads a lane's 16 code bytes of one unit of row r and their block's absmax
// (for r >= N, the same fixed bytes in every lane: an instruction that moves
// no new data, so that no branch ever surrounds a load and the compiler's
// in-order vmcnt accounting stays exact).
__device__ __forceinline__ void load_unit(const uint8_t* __restrict__ codes, const float* __restrict__ absmax,
                                          int r, int N, int K, int nab, bool lane_valid, int code_off, int ab_off,
                                          u32x4& c, float& a) {
    const bool live = lane_valid && r < N;
    c = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(live ? codes + (size_t)r * (K >> 1) + code_off : codes));
    a = __builtin_nontemporal_load(live ? absmax + (size_t)r * nab + ab_off : absmax);
}

// A lane's 16 code bytes against its 32 activations: NA independent partial
// sums (byte i to sum i % NA), added in a fixed order.  tab_lane is the
// lane's copy of the pair table (entry v at tab_lane[v * TC]).  With 32
// copies an entry is 256 bytes, so the byte offset of entry v in the lane's
// copy is v << 8 plus the copy's 8 * (lane % 32): one byte permute forms it
// from the code word (byte v into bits 8..15, the copy offset into bits
// 0..7), where fewer copies need a byte extract and a shift-add.
template <int TC, int NA>
__device__ __forceinline__ float unit_dot(const u32x4& c, const uint32_t (&xr)[16], const uint2* tab_lane,
                                          const uint2* tab0, uint32_t copy_off) {
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    float p[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) p[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        uint2 e;
        if constexpr (TC == 32) {
            // D = bytes {copy_off.b0, code byte i & 3, 0, 0} (selector 4 + k picks byte k of
            // the first operand, 0 byte 0 of the second, 0x0C a zero byte)
            const uint32_t off = __builtin_amdgcn_perm(cw[i >> 2], copy_off, 0x0C0C0000u | ((4u + (i & 3)) << 8));
            e = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(tab0) + off);
        } else {
            const uint32_t v = (cw[i >> 2] >> (8 * (i & 3))) & 0xFFu;
            e = tab_lane[v * TC];
        }
        p[i % NA] = dot2_f16(e.x, xr[i], p[i % NA]);
        p[i % NA] = dot2_f16(e.y, xr[i], p[i % NA]);
    }
    float s = p[0];
#pragma unroll
    for (int j = 1; j < NA; ++j) s += p[j];
    return s;
}

// One workgroup of S waves takes rows b, b + grid, b + 2*grid, ...; wave w
// owns unit w (weights 2048w .. 2048w + 2047) of every one of them, so a lane
// keeps only its 32 activations of that unit.  Each wave reduces a row's unit
// over its lanes (DPP) and lane k keeps the k-th row of a batch of 64; after
// the batch the waves' partials meet in LDS and wave 0 adds them in unit
// order and stores the 64 results.
template <int TC, int NA, int AHEAD>
__global__ void __launch_bounds__(1024)
k_nf4(const uint8_t* __restrict__ codes, const float* __restrict__ absmax, const float* __restrict__ table,
      const uint16_t* __restrict__ x, float* __restrict__ y, int N, int K, int B) {
    static_assert(TC == 8 || TC == 16 || TC == 32, "table copies");
    static_assert(AHEAD >= 2 && AHEAD <= 8 && (kWave % AHEAD) == 0, "rows in flight");
    __shared__ uint2 ptab[256 * TC];
    __shared__ float red[16][kWave];
    __shared__ float tl[16];
    const int lane = lane_id();
    const int wave = wave_in_block();           // = the unit
    const int S = blockDim.x / kWave;
    const int grid = gridDim.x;
    const int nab = K / B;
    const int k0 = wave * kUnitWeights + lane * 32;
    const bool lane_valid = k0 < K;
    const int code_off = wave * kUnitCodes + lane * 16;
    const int ab_off = wave * (kUnitWeights / B) + (lane * 32) / B;

    // the activations are requested first, then the first AHEAD rows of
    // weights; building the pair table and converting x wait only for the
    // older loads, so the weight stream starts at once
    u32x4 xraw[4];
    {
        const u32x4* src = reinterpret_cast<const u32x4*>(x + (lane_valid ? k0 : 0));
#pragma unroll
        for (int q = 0; q < 4; ++q) xraw[q] = src[q];
    }
    const int b = blockIdx.x;
    const int nrows = b < N ? (N - 1 - b) / grid + 1 : 0;   // rows of this workgroup (uniform)
    // rows in flight: q[j] holds row k + j of the workgroup's sequence
    u32x4 qc[AHEAD];
    float qa[AHEAD];
#pragma unroll
    for (int j = 0; j < AHEAD; ++j)
        load_unit(codes, absmax, b + j * grid, N, K, nab, lane_valid, code_off, ab_off, qc[j], qa[j]);

    // the byte-pair table: entry v = (weights 2j, 2j+1 with codes v >> 4 and v & 15).
    // The 16 values are read with uniform (scalar) loads, which do not count
    // in vmcnt, and passed on through LDS: a per-thread indexed read of the
    // table here would be a vector load behind the weight loads, and waiting
    // for it would wait for them too.
    uint32_t tmax = 0;
    float tv = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const float v = table[j];
        tmax = max(tmax, __builtin_bit_cast(uint32_t, v) & 0x7FFFFFFFu);
        tv = threadIdx.x == (unsigned)j ? v : tv;
    }
    if (threadIdx.x < 16) tl[threadIdx.x] = tv;
    lds_barrier();
    const int st = min(scale_exp(tmax >> 23), 126);   // 2^st and 2^-st both normal
    {
        const float ts = pow2f(st);
        for (int i = threadIdx.x; i < 256 * TC; i += blockDim.x) {
            const int v = i / TC;
            const float a = tl[v >> 4] * ts, b2 = tl[v & 15] * ts;
            const uint32_t ha = f32_to_f16_bits(a), hb = f32_to_f16_bits(b2);
            const uint32_t la = f32_to_f16_bits(a - f16_bits_to_f32(ha));
            const uint32_t lb = f32_to_f16_bits(b2 - f16_bits_to_f32(hb));
            ptab[i] = uint2{ha | (hb << 16), la | (lb << 16)};   // the first weight in the low half, as x[2j]
        }
    }
    // the lane's activations as binary16 scaled by 2^sx; bx = 2^-sx, bt = 2^-st
    uint32_t xr[16];
    float bx;
    {
        uint32_t raw[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            raw[4 * q + 0] = lane_valid ? xraw[q].x : 0u;   // lanes past the row: 0 times any table value
            raw[4 * q + 1] = lane_valid ? xraw[q].y : 0u;
            raw[4 * q + 2] = lane_valid ? xraw[q].z : 0u;
            raw[4 * q + 3] = lane_valid ? xraw[q].w : 0u;
        }
        uint32_t emax = 0;   // largest bfloat16 exponent field of the 32 values
#pragma unroll
        for (int i = 0; i < 16; ++i) emax = max(emax, max((raw[i] >> 7) & 0xFFu, (raw[i] >> 23) & 0xFFu));
        const int sx = min(scale_exp(emax), 126);
        const float xs = pow2f(sx);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float lo = __builtin_bit_cast(float, raw[i] << 16) * xs;
            const float hi = __builtin_bit_cast(float, raw[i] & 0xFFFF0000u) * xs;
            xr[i] = f32_to_f16_bits(lo) | (f32_to_f16_bits(hi) << 16);
        }
        bx = pow2f(-sx);
    }
    const float bt = pow2f(-st);
    lds_barrier();   // the pair table is complete

    const uint2* const tab_lane = ptab + (lane % TC);
    const uint32_t copy_off = (uint32_t)(lane % TC) * 8u;
    // Rows in batches of 64: the inner loop holds nothing but loads, lookups
    // and reductions (rows past the workgroup's last re-read a fixed address
    // and are dropped), and the batch's results are stored after it.  With a
    // store or an early exit inside the loop the compiler's vmcnt analysis
    // merged unequal histories at the loop head and drained every load there
    // (vmcnt(0) once per AHEAD rows); without them its waits are exact.
    const int nrows_pad = (nrows + AHEAD - 1) / AHEAD * AHEAD;   // uniform
    for (int kb = 0; kb < nrows_pad; kb += kWave) {
        const int kend = kb + kWave < nrows_pad ? kb + kWave : nrows_pad;
        float part = 0.0f;
        for (int k0r = kb; k0r < kend; k0r += AHEAD) {
#pragma unroll
            for (int j = 0; j < AHEAD; ++j) {
                const int k = k0r + j;
                const float s = unit_dot<TC, NA>(qc[j], xr, tab_lane, ptab, copy_off);
                const float a = lane_valid ? qa[j] : 0.0f;
                load_unit(codes, absmax, b + (k + AHEAD) * grid, N, K, nab, lane_valid, code_off, ab_off, qc[j],
                          qa[j]);
                const float r = wave_sum_f32(s * bt * bx * a);   // this unit of row k, wave-uniform
                if (lane == (k & (kWave - 1))) part = r;
            }
        }
        const bool mine = kb + lane < nrows;   // lane i holds row kb + i of the workgroup's sequence
        if (S == 1) {
            if (mine) y[b + (int64_t)(kb + lane) * grid] = part;
        } else {
            red[wave][lane] = part;
            lds_barrier();
            if (wave == 0 && mine) {
                float t = red[0][lane];
                for (int w = 1; w < S; ++w) t += red[w][lane];
                y[b + (int64_t)(kb + lane) * grid] = t;
            }
            lds_barrier();
        }
    }
}

// ---------------------------------------------------------------------------
// NF4 on the vector unit in float arithmetic, rows reduced four at a time
// (the default).
//
// A code byte is still one lookup (one byte permute forms the address, one
// 8-byte LDS read returns both weights), but the entry holds the two table
// values as binary32, and the lane multiplies them with its activations
// (bfloat16 widened to binary32, exact) by two v_fmac_f32: the products and
// sums are the float GEMV's, with nothing approximated.  This is also the
// faster form on gfx950: v_dot2_f32_f16 issues at half the rate of
// v_fmac_f32 (timed here: with the weight stream cached, k_nf4's two dot2 per
// code byte put its arithmetic alone at about 20 us for 28672 x 8192), so the
// binary16 split of k_nf4 -- two dot2, four multiplies per byte -- costs twice
// the cycles of two fmac.  Beyond that, two changes remove most of k_nf4's
// per-row work:
//   * the lookups are free of bank conflicts: entry v of copy c sits at byte
//     256v + 8c, so the lanes that the LDS serves together (c = lane % 32)
//     hit distinct banks whatever their codes.  With 8 copies, k_nf4 at
//     28672 x 8192 stalled on bank conflicts for 3.5 times its busy LDS
//     cycles;
//   * a wave's lane sums of four rows are reduced together: a
//     v_permlane32_swap and an add fold rows (0, 1) and (2, 3) into half
//     waves, a v_permlane16_swap and an add fold those into 16-lane rows
//     (rows 0, 2, 1, 3), and four DPP row_shr adds finish the four at once
//     in lanes 15, 31, 47 and 63: ten instructions for four rows, where a
//     whole-wave reduction takes about a dozen per row.
// The 64 KiB table is built once per workgroup, so a workgroup holds G row
// groups of S = ceil(K/2048) waves (wave u of a group owns weights
// 2048u .. 2048u + 2047 of each of its rows, as in k_nf4); group g of
// workgroup b takes rows bG + g, bG + g + gridG, ....  The unit sums of a
// row meet in LDS every 64 rows and are added in unit order, so results do
// not depend on the launch shape.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float f32_of(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t bits_of(float f) { return __builtin_bit_cast(uint32_t, f); }

// Sums over the wave of four per-lane values: the sum of p0 ends in lane
// 15, of p2 in lane 31, of p1 in lane 47, of p3 in lane 63.
__device__ __forceinline__ float sum_four_rows(float p0, float p1, float p2, float p3) {
    // halves: p0' = (p0.lo, p1.lo), p1' = (p0.hi, p1.hi)
    const auto a = __builtin_amdgcn_permlane32_swap(bits_of(p0), bits_of(p1), false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(bits_of(p2), bits_of(p3), false, false);
    const float q01 = f32_of(a[0]) + f32_of(a[1]);   // lanes 0..31: row 0, 32..63: row 1
    const float q23 = f32_of(b[0]) + f32_of(b[1]);   // row 2, row 3
    // 16-lane rows: q01' = (q01.r0, q23.r0, q01.r2, q23.r2), q23' = (q01.r1, q23.r1, q01.r3, q23.r3)
    const auto c = __builtin_amdgcn_permlane16_swap(bits_of(q01), bits_of(q23), false, false);
    float r = f32_of(c[0]) + f32_of(c[1]);           // 16-lane rows hold rows 0, 2, 1, 3
    r += dpp_mov_f32<kDppRowShr1, 0xF>(r);
    r += dpp_mov_f32<kDppRowShr2, 0xF>(r);
    r += dpp_mov_f32<kDppRowShr4, 0xF>(r);
    r += dpp_mov_f32<kDppRowShr8, 0xF>(r);
    return r;
}

// A lane's 16 code bytes and absmax of row r: every load is in bounds and
// unconditional (lanes past K read inside their row, rows past N read row
// 0) and the values that do not belong to the result are dropped.
// The row's base is wave-uniform and the lane's offset a 32-bit constant, so
// the loads take the scalar-base form: no vector instruction forms an address.
__device__ __forceinline__ void load_row_unit(const uint8_t* __restrict__ codes, const float* __restrict__ absmax,
                                              int r, int row_bytes, int nab, uint32_t code_off, uint32_t ab_off,
                                              u32x4& c, float& a) {
    const uint8_t* crow = codes + (size_t)r * (size_t)row_bytes;
    const float* arow = absmax + (size_t)r * (size_t)nab;
    c = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(crow + code_off));
    a = __builtin_nontemporal_load(arow + ab_off);
}

// A lane's 16 code bytes against its 32 activations in binary32: NA
// independent sums (byte i to sum i % NA), added in a fixed order.  Entry v
// of the lane's table copy is at byte 256v + copy_off; one byte permute
// forms that offset from the code word (byte v into bits 8..15, the copy
// offset into bits 0..7).
template <int NA>
__device__ __forceinline__ float unit_dot_f32(const u32x4& c, const float (&xf)[32], const uint8_t* tab,
                                              uint32_t copy_off) {
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    float2 e[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t off = __builtin_amdgcn_perm(cw[i >> 2], copy_off, 0x0C0C0000u | ((4u + (i & 3)) << 8));
        e[i] = *reinterpret_cast<const float2*>(tab + off);
    }
    // One wait for all 16 reads (the empty asm takes them all), instead of a
    // wait before each entry's first use: on this path the instructions a
    // SIMD issues, waits included, are what bounds the kernel.
    asm volatile("" ::"v"(e[0]), "v"(e[1]), "v"(e[2]), "v"(e[3]), "v"(e[4]), "v"(e[5]), "v"(e[6]), "v"(e[7]),
                 "v"(e[8]), "v"(e[9]), "v"(e[10]), "v"(e[11]), "v"(e[12]), "v"(e[13]), "v"(e[14]), "v"(e[15]));
    float p[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) p[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        p[i % NA] = fmaf(e[i].x, xf[2 * i], p[i % NA]);       // weight 2i: the high nibble
        p[i % NA] = fmaf(e[i].y, xf[2 * i + 1], p[i % NA]);
    }
    float s = p[0];
#pragma unroll
    for (int j = 1; j < NA; ++j) s += p[j];
    return s;
}

template <int AHEAD, int NA>
__global__ void __launch_bounds__(1024)
k_nf4_rows(const uint8_t* __restrict__ codes, const float* __restrict__ absmax, const float* __restrict__ table,
           const uint16_t* __restrict__ x, float* __restrict__ y, int N, int K, int B, int S) {
    static_assert(AHEAD == 4 || AHEAD == 8, "rows in flight: whole groups of four");
    __shared__ float2 ftab[256 * 32];   // entry v of copy c at [32v + c]
    __shared__ float red[16][kWave];    // [wave][row of the batch]
    __shared__ float tl[16];
    const int lane = lane_id();
    const int wave = wave_in_block();
    const int G = blockDim.x / (S * kWave);
    const int unit = wave % S;
    const int grp = wave / S;
    const int nab = K / B;
    const int row_bytes = K >> 1;
    const int k0 = unit * kUnitWeights + lane * 32;
    const bool lane_valid = k0 < K;
    const int kl = lane_valid ? k0 : 0;   // lanes past K: weights 0..31 of the row
    const uint32_t code_off = (uint32_t)(kl >> 1);
    const uint32_t ab_off = (uint32_t)(kl / B);

    u32x4 xraw[4];
    {
        const u32x4* src = reinterpret_cast<const u32x4*>(x + kl);
#pragma unroll
        for (int q = 0; q < 4; ++q) xraw[q] = src[q];
    }
    const int nstreams = gridDim.x * G;
    const int stream = blockIdx.x * G + grp;
    const int first = blockIdx.x * G;
    const int nrows = stream < N ? (N - 1 - stream) / nstreams + 1 : 0;
    const int nrows_wg = first < N ? (N - 1 - first) / nstreams + 1 : 0;   // the longest stream: uniform
    // row k of this stream, or row 0 past its end (read and dropped)
    auto row_at = [&](int k) -> int { return k < nrows ? stream + k * nstreams : 0; };
    u32x4 qc[AHEAD];
    float qa[AHEAD];
#pragma unroll
    for (int j = 0; j < AHEAD; ++j) load_row_unit(codes, absmax, row_at(j), row_bytes, nab, code_off, ab_off, qc[j], qa[j]);

    // The 16 table values are read with uniform (scalar) loads, which do not
    // count in vmcnt, and passed on through LDS: a per-thread indexed read of
    // the table here would be a vector load behind the weight loads, and
    // waiting for it would wait for them too.
    float tv = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const float v = table[j];
        tv = threadIdx.x == (unsigned)j ? v : tv;
    }
    if (threadIdx.x < 16) tl[threadIdx.x] = tv;
    lds_barrier();
    if ((blockDim.x & 255) == 0) {
        // entry v = thread % 256 into copies thread / 256, + blockDim / 256, ...; the
        // lanes of a write (consecutive v) reach copies (c + v) % 32: distinct banks
        const int v = threadIdx.x & 255;
        const float2 e = float2{tl[v >> 4], tl[v & 15]};
        for (int c = threadIdx.x >> 8; c < 32; c += blockDim.x >> 8) ftab[v * 32 + ((c + v) & 31)] = e;
    } else {
        for (int i = threadIdx.x; i < 256 * 32; i += blockDim.x) ftab[i] = float2{tl[i >> 9], tl[(i >> 5) & 15]};
    }
    // the lane's activations in binary32 (lanes past K: 0 times any table value)
    float xf[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t w[4] = {xraw[q].x, xraw[q].y, xraw[q].z, xraw[q].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            xf[8 * q + 2 * h] = lane_valid ? f32_of(w[h] << 16) : 0.0f;
            xf[8 * q + 2 * h + 1] = lane_valid ? f32_of(w[h] & 0xFFFF0000u) : 0.0f;
        }
    }
    lds_barrier();   // the table is complete

    const uint8_t* const tab = reinterpret_cast<const uint8_t*>(ftab);
    const uint32_t copy_off = (uint32_t)(lane & 31) * 8u;
    const int h = lane >> 4;
    const int row_of_lane = ((h & 1) << 1) | (h >> 1);   // lanes 15, 31, 47, 63 end rows 0, 2, 1, 3
    float* const mine = red[wave];
    const int nrows_pad = (nrows_wg + AHEAD - 1) / AHEAD * AHEAD;   // uniform
    for (int kb = 0; kb < nrows_pad; kb += kWave) {
        const int kend = kb + kWave < nrows_pad ? kb + kWave : nrows_pad;
        for (int kr = kb; kr < kend; kr += AHEAD) {
            float p[AHEAD];
#pragma unroll
            for (int j = 0; j < AHEAD; ++j) {
                p[j] = unit_dot_f32<NA>(qc[j], xf, tab, copy_off) * (lane_valid ? qa[j] : 0.0f);
                load_row_unit(codes, absmax, row_at(kr + j + AHEAD), row_bytes, nab, code_off, ab_off, qc[j],
                              qa[j]);
                // one row's lookups at a time: the row's sum is formed here (the empty
                // asm takes it), not sunk to the reduction with every row's 16
                // looked-up entries held in registers until then
                asm volatile("" : "+v"(p[j]));
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int q = 0; q < AHEAD / 4; ++q) {
                const float r = sum_four_rows(p[4 * q], p[4 * q + 1], p[4 * q + 2], p[4 * q + 3]);
                if ((lane & 15) == 15) mine[kr - kb + 4 * q + row_of_lane] = r;
            }
        }
        lds_barrier();
        if (unit == 0 && kb + lane < nrows) {
            float t = red[grp * S][lane];
            for (int u = 1; u < S; ++u) t += red[grp * S + u][lane];
            y[stream + (int64_t)(kb + lane) * nstreams] = t;
        }
        lds_barrier();
    }
}

// ---------------------------------------------------------------------------
// NF4 on the matrix cores (K = 2048, 4096 or 8192).
//
// The same products, with the per-byte work moved from the vector unit to
// v_mfma_f32_16x16x32_f16.  A workgroup of 16 waves takes tiles of 16 rows;
// wave w owns part w of K (K/16 weights, whole blocks of B), so a tile is 16
// rows x K/16 weights per wave, in k-steps of 32 weights of one block:
//   each lane group g covers weights 8g..8g+7 of a k-step of row j (4 code
//     bytes), in two MFMAs of two bytes each.  A byte's table entry is its
//     two weights' high binary16 parts and their remainders (two dwords, as
//     one 8-byte LDS read lands them); two entries side by side are the
//     lane's B operand, so B holds (hi, hi, lo, lo) of two weights twice
//     over, and A holds the matching activations twice: x pair, x pair,
//     next x pair, next x pair (x is stored in LDS with every binary16 pair
//     duplicated, so one 16-byte read is the operand).  The MFMA's sum over
//     its 32 k-slots is then the exact hi*x + lo*x over 16 weights;
//   every row of A is the same, so every row of D is the same and lane
//     (g, j) holds row j's sum in each of its four D registers;
//   after the B/32 k-steps of a block, the block's D is scaled by the row's
//     absmax and added to the lane's running sum (fp32); four D accumulators
//     alternate so that consecutive MFMAs do not wait for each other.
// Loads: lane (g, j) reads 16 consecutive code bytes of row j per instruction
// -- k-step 4c + g, all four lane groups' bytes -- and four permlane swaps
// (v_permlane16_swap, v_permlane32_swap: a 4 x 4 transpose across the lane
// groups) hand each lane group its own dword of the four k-steps.  The next
// tile's codes and absmax values are loaded while this tile computes.  The
// 16 parts of a tile meet in LDS and are added in part order (deterministic).
// Arithmetic: products exact (binary16 x binary16), sums in fp32 inside the
// MFMA and in the running sum; x is scaled by one power of two for the whole
// of K (exact unless a value lies some 2^28 below the largest).
// ---------------------------------------------------------------------------
constexpr int kMW = 16;   // waves per workgroup = parts of K

__device__ __forceinline__ float u32_as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_mov_u32<kDppRowShr1, 0xF>(v));
    v = max(v, dpp_mov_u32<kDppRowShr2, 0xF>(v));
    v = max(v, dpp_mov_u32<kDppRowShr4, 0xF>(v));
    v = max(v, dpp_mov_u32<kDppRowShr8, 0xF>(v));
    v = max(v, dpp_mov_u32<kDppRowBcast15, 0xA>(v));
    v = max(v, dpp_mov_u32<kDppRowBcast31, 0xC>(v));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4m __attribute__((ext_vector_type(4)));

// 4 x 4 transpose of dwords across the four 16-lane groups: in, lane group g
// holds v[0..3] of its own k-step; out, lane group g holds dword g of k-steps
// 0..3 (v[s] = dword g of k-step s).
__device__ __forceinline__ void xpose4(uint32_t (&v)[4]) {
    // rows (lane groups) 0<->1 and 2<->3 exchange: v0' = (v0.r0, v1.r0, v0.r2, v1.r2),
    // v1' = (v0.r1, v1.r1, v0.r3, v1.r3); likewise v2, v3
    const auto a = __builtin_amdgcn_permlane16_swap(v[0], v[1], false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(v[2], v[3], false, false);
    // halves exchange: (a0, b0) -> k-steps 0 and 2; (a1, b1) -> k-steps 1 and 3
    const auto c = __builtin_amdgcn_permlane32_swap(a[0], b[0], false, false);
    const auto d = __builtin_amdgcn_permlane32_swap(a[1], b[1], false, false);
    v[0] = c[0];
    v[2] = c[1];
    v[1] = d[0];
    v[3] = d[1];
}

template <int KSP, int BPK>   // k-steps per part (K / 512), k-steps per block (B / 32)
__global__ void __launch_bounds__(kMW * kWave)
k_nf4_mfma(const uint8_t* __restrict__ codes, const float* __restrict__ absmax, const float* __restrict__ table,
           const uint16_t* __restrict__ x, float* __restrict__ y, int N, int K, int B) {
    static_assert(KSP == 4 || KSP == 8 || KSP == 16, "K = 2048, 4096 or 8192");
    static_assert(BPK >= 1 && BPK <= KSP, "whole blocks per part");
    constexpr int NB = KSP / BPK;           // blocks per part
    constexpr int NC = KSP / 4;             // 16-byte code loads per lane per tile
    constexpr int NAL = NB >= 4 ? NB / 4 : NB;   // absmax loads per lane per tile
    __shared__ uint2 ptab[256 * 32];        // the byte-pair table, 32 copies (64 KiB)
    __shared__ uint32_t xh[8192];           // x as scaled binary16 pairs, each pair twice
    __shared__ float red[2][kMW][16];       // the parts of a tile (double-buffered)
    __shared__ float tl[16];
    __shared__ uint32_t emax_w[kMW];
    const int lane = lane_id();
    const int wave = wave_in_block();
    const int g = lane >> 4, j = lane & 15;
    const int ntiles = (N + 15) / 16;
    const int nab = K / B;                  // absmax values per row
    const int pbyte = wave * KSP * 16;      // first code byte of this part in a row
    const int pblk = wave * NB;             // first block of this part

    // code and absmax loads of tile t (rows past N re-read row N - 1)
    auto load_tile = [&](int t, u32x4 (&c)[NC], float (&am)[NB]) {
        const int r = min(t * 16 + j, N - 1);
        const uint8_t* rowc = codes + (size_t)r * (K >> 1) + pbyte + 16 * g;
#pragma unroll
        for (int q = 0; q < NC; ++q) c[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowc + 64 * q));
        const float* rowa = absmax + (size_t)r * nab + pblk;
        if constexpr (NB >= 4) {
#pragma unroll
            for (int q = 0; q < NAL; ++q) {
                // elements pass through u32_as_f32 by value: a bit cast applied to a
                // vector element lvalue (v.y) reads element 0 on this compiler
                const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowa + 4 * q));
                am[4 * q + 0] = u32_as_f32(v.x);
                am[4 * q + 1] = u32_as_f32(v.y);
                am[4 * q + 2] = u32_as_f32(v.z);
                am[4 * q + 3] = u32_as_f32(v.w);
            }
        } else {
#pragma unroll
            for (int q = 0; q < NB; ++q) am[q] = __builtin_nontemporal_load(rowa + q);
        }
    };

    // x first (one 16-byte load per thread covers K = 8192), then the first tile
    const int nxv = K / 8;                   // 16-byte vectors of x
    u32x4 xv = reinterpret_cast<const u32x4*>(x)[(int)threadIdx.x < nxv ? (int)threadIdx.x : 0];
    int t = blockIdx.x;
    u32x4 cc[NC];
    float am[NB];
    if (t < ntiles) load_tile(t, cc, am);

    // the byte-pair table (as in k_nf4), 32 copies
    uint32_t tmax = 0;
    float tv = 0.0f;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const float v = table[q];
        tmax = max(tmax, __builtin_bit_cast(uint32_t, v) & 0x7FFFFFFFu);
        tv = threadIdx.x == (unsigned)q ? v : tv;
    }
    if (threadIdx.x < 16) tl[threadIdx.x] = tv;
    // the largest bfloat16 exponent field of x, over the workgroup
    uint32_t em = 0;
    if ((int)threadIdx.x < nxv) {
        const uint32_t w4[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) em = max(em, max((w4[q] >> 7) & 0xFFu, (w4[q] >> 23) & 0xFFu));
    }
    em = wave_max_u32(em);
    if (lane == 0) emax_w[wave] = em;
    lds_barrier();
    const int st = min(scale_exp(tmax >> 23), 126);
    {
        const float ts = pow2f(st);
        for (int i = threadIdx.x; i < 256 * 32; i += kMW * kWave) {
            const int v = i >> 5;
            const float a = tl[v >> 4] * ts, b2 = tl[v & 15] * ts;
            const uint32_t ha = f32_to_f16_bits(a), hb = f32_to_f16_bits(b2);
            const uint32_t la = f32_to_f16_bits(a - f16_bits_to_f32(ha));
            const uint32_t lb = f32_to_f16_bits(b2 - f16_bits_to_f32(hb));
            ptab[i] = uint2{ha | (hb << 16), la | (lb << 16)};   // the first weight in the low half
        }
    }
    uint32_t emx = 0;
#pragma unroll
    for (int w = 0; w < kMW; ++w) emx = max(emx, emax_w[w]);
    const int sx = min(scale_exp(emx), 126);
    if ((int)threadIdx.x < nxv) {
        const float xs = pow2f(sx);
        const uint32_t w4[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float lo = __builtin_bit_cast(float, w4[q] << 16) * xs;
            const float hi = __builtin_bit_cast(float, w4[q] & 0xFFFF0000u) * xs;
            const uint32_t pr = f32_to_f16_bits(lo) | (f32_to_f16_bits(hi) << 16);
            xh[8 * threadIdx.x + 2 * q] = pr;
            xh[8 * threadIdx.x + 2 * q + 1] = pr;
        }
    }
    const float bt = pow2f(-st), bx = pow2f(-sx);
    lds_barrier();   // table and x complete

    const uint32_t copy_off = (uint32_t)(lane & 31) * 8u;
    const uint8_t* const tab0 = reinterpret_cast<const uint8_t*>(ptab);
    const uint32_t* const xpart = xh + wave * KSP * 32 + 8 * g;   // this part's x (doubled), lane group g's
    int par = 0;
    for (; t < ntiles; t += gridDim.x) {   // workgroup-uniform
        u32x4 cur[NC];
        float amc[NB];
#pragma unroll
        for (int q = 0; q < NC; ++q) cur[q] = cc[q];
#pragma unroll
        for (int q = 0; q < NB; ++q) amc[q] = am[q];
        if (t + (int)gridDim.x < ntiles) load_tile(t + gridDim.x, cc, am);

        float acc = 0.0f;
        f32x4m d[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) d[u] = f32x4m{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int q = 0; q < NC; ++q) {
            uint32_t v[4] = {cur[q].x, cur[q].y, cur[q].z, cur[q].w};
            xpose4(v);   // v[s'] = this lane group's code dword of k-step 4q + s'
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const int ks = 4 * q + s2;
                uint2 e[4];
#pragma unroll
                for (int b4 = 0; b4 < 4; ++b4) {
                    const uint32_t off = __builtin_amdgcn_perm(v[s2], copy_off, 0x0C0C0000u | ((4u + b4) << 8));
                    e[b4] = *reinterpret_cast<const uint2*>(tab0 + off);
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {   // bytes 2h, 2h + 1 of the lane's four
                    const u32x4 bop = u32x4{e[2 * h].x, e[2 * h].y, e[2 * h + 1].x, e[2 * h + 1].y};
                    const u32x4 aop = *reinterpret_cast<const u32x4*>(xpart + ks * 32 + 4 * h);
                    f32x4m& dd = d[2 * (ks & 1) + h];
                    dd = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, aop),
                                                                __builtin_bit_cast(f16x8, bop), dd, 0, 0, 0);
                }
                if ((ks + 1) % BPK == 0) {   // the block is complete: scale by its absmax
                    float bs;
                    if constexpr (BPK == 1) {
                        bs = d[2 * (ks & 1)][0] + d[2 * (ks & 1) + 1][0];
                        d[2 * (ks & 1)] = f32x4m{0.0f, 0.0f, 0.0f, 0.0f};
                        d[2 * (ks & 1) + 1] = f32x4m{0.0f, 0.0f, 0.0f, 0.0f};
                    } else {
                        bs = (d[0][0] + d[1][0]) + (d[2][0] + d[3][0]);
#pragma unroll
                        for (int u = 0; u < 4; ++u) d[u] = f32x4m{0.0f, 0.0f, 0.0f, 0.0f};
                    }
                    acc = fmaf(bs, amc[ks / BPK], acc);
                }
            }
        }
        if (lane < 16) red[par][wave][j] = acc * bt * bx;
        lds_barrier();
        if (wave == 0 && lane < 16 && t * 16 + j < N) {
            float sum = red[par][0][j];
#pragma unroll
            for (int w = 1; w < kMW; ++w) sum += red[par][w][j];
            y[t * 16 + j] = sum;
        }
        par ^= 1;
    }
}

// One thread per block of B weights: absmax, then the nearest table level of
// each w / absmax (binary32, correctly rounded division), a tie going to the
// lower level; two codes per byte, the first weight in the high nibble.
__global__ void k_quantize_nf4(const float* __restrict__ w, uint8_t* __restrict__ codes, float* __restrict__ absmax,
                               const float* __restrict__ table, int64_t nblocks, int B) {
    const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (blk >= nblocks) return;
    float mid[15];
#pragma unroll
    for (int j = 0; j < 15; ++j) mid[j] = bind_f32(table[j] + table[j + 1]) * 0.5f;
    const float* xb = w + blk * B;
    float amax = 0.0f;
    for (int i = 0; i < B; ++i) amax = fmaxf(amax, fabsf(xb[i]));
    absmax[blk] = amax;
    uint8_t* cb = codes + blk * (B / 2);
    for (int i = 0; i < B; i += 2) {
        int c[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float r = amax != 0.0f ? xb[i + h] / amax : 0.0f;
            int q = 0;
#pragma unroll
            for (int j = 0; j < 15; ++j) q += r > mid[j] ? 1 : 0;
            c[h] = q;
        }
        cb[i / 2] = (uint8_t)((c[0] << 4) | c[1]);
    }
}

hipError_t launch_nf4_mfma(const uint8_t* c8, const float* absmax, const float* table, const uint16_t* x16, float* y,
                           int N, int K, int B, int grid, hipStream_t s) {
    const int ksp = K / 512, bpk = B / 32;
    if (K != 512 * ksp || (ksp != 4 && ksp != 8 && ksp != 16) || bpk > ksp || ksp / bpk > 8)
        return hipErrorInvalidValue;   // at most 8 absmax blocks per part (registers)
    const int ntiles = (N + 15) / 16;
    if (!grid) grid = ntiles < device_cu_count() ? ntiles : device_cu_count();   // one workgroup per CU (LDS)
#define DG_NF4M(KK, BB)                                                                                       \
    if (ksp == KK && bpk == BB) {                                                                             \
        hipLaunchKernelGGL((k_nf4_mfma<KK, BB>), dim3(grid), dim3(kMW * kWave), 0, s, c8, absmax, table, x16, y, \
                           N, K, B);                                                                          \
        return hipGetLastError();                                                                             \
    }
    DG_NF4M(4, 1) DG_NF4M(4, 2) DG_NF4M(4, 4)
    DG_NF4M(8, 1) DG_NF4M(8, 2) DG_NF4M(8, 4) DG_NF4M(8, 8)
    DG_NF4M(16, 2) DG_NF4M(16, 4) DG_NF4M(16, 8)   // K = 8192 with B = 32 would spill
#undef DG_NF4M
    return hipErrorInvalidValue;
}

}  // namespace

// block 0: the fewest row groups that make at least eight waves (G =
// ceil(8 / S) below eight units, 8..16 waves); rows in flight 0: eight for
// K of 4097..8192, else four; grid 0: one workgroup per CU.  Measured on MI355X over the
// decoder shapes and the 70B MLP pair (K = 4096, 8192, 14336, 28672), each
// launch timed against the others in turn on one device: K = 14336 with two
// row groups (14 waves) instead of one took 9.0 instead of 9.9 us, and K =
// 8192 with eight rows in flight 23.5 instead of 24.7 us at 28672 rows,
// while eight rows in flight lost 5-18% at the other K.  A second workgroup
// per CU (LDS allows two) or more waves per workgroup gain nothing or lose,
// and a grid past one round of workgroups loses up to a third.
static hipError_t launch_nf4_rows(const uint8_t* c8, const float* absmax, const float* table, const uint16_t* x16,
                                  float* y, int N, int K, int B, int grid, int block, int unroll, hipStream_t s) {
    const int S = (K + kUnitWeights - 1) / kUnitWeights;
    if (S > kMaxUnits) return hipErrorInvalidValue;
    const int G = block ? block / (S * kWave) : (S < 8 ? (8 + S - 1) / S : 1);
    if (block && (block % (S * kWave) != 0 || block > 1024)) return hipErrorInvalidValue;
    if (G < 1) return hipErrorInvalidValue;
    // unroll: rows in flight (4, 8) + 100 * independent partial sums per lane (1, 2, 4)
    const int na = unroll / 100 ? unroll / 100 : 1;
    const int ahead = unroll % 100 ? unroll % 100 : (S == 3 || S == 4 ? 8 : 4);
    if (!grid) {
        const int need = (N + G - 1) / G;
        grid = need < 256 ? need : 256;
    }
    const dim3 b3(G * S * kWave);
#define DG_NF4R(HH, AA)                                                                                     \
    if (ahead == HH && na == AA) {                                                                          \
        hipLaunchKernelGGL((k_nf4_rows<HH, AA>), dim3(grid), b3, 0, s, c8, absmax, table, x16, y, N, K, B, S); \
        return hipGetLastError();                                                                           \
    }
    DG_NF4R(4, 1) DG_NF4R(4, 2) DG_NF4R(4, 4) DG_NF4R(8, 1) DG_NF4R(8, 2)
#undef DG_NF4R
    return hipErrorInvalidValue;
}

hipError_t launch_gemv_nf4(const void* codes, const float* absmax, const float* table, const void* x, float* y,
                           int N, int K, int B, const dg_launch* cfg, hipStream_t s) {
    const int variant = cfg ? cfg->variant : 0;
    if (variant == 0 || variant == DG_VARIANT_NF4_ROWS)   // the default
        return launch_nf4_rows((const uint8_t*)codes, absmax, table, (const uint16_t*)x, y, N, K, B,
                               cfg ? cfg->grid : 0, cfg ? cfg->block : 0, cfg ? cfg->unroll : 0, s);
    if (variant == DG_VARIANT_NF4_MFMA) {
        if (cfg->block || cfg->unroll) return hipErrorInvalidValue;   // fixed: 16 waves, one table
        return launch_nf4_mfma((const uint8_t*)codes, absmax, table, (const uint16_t*)x, y, N, K, B, cfg->grid, s);
    }
    if (variant != DG_VARIANT_NF4_UNITS) return hipErrorInvalidValue;
    const int S = (K + kUnitWeights - 1) / kUnitWeights;   // waves per workgroup: one per unit
    if (S > kMaxUnits) return hipErrorInvalidValue;
    if (cfg->block && cfg->block != S * kWave) return hipErrorInvalidValue;   // fixed by K
    // unroll: table copies (8, 16 or 32) + 100 * independent partial sums (1, 2)
    //         + 1000 * rows in flight per wave (4 or 8)
    const int u = cfg->unroll;
    const int copies = u % 100 ? u % 100 : 8;
    const int na = (u / 100) % 10 ? (u / 100) % 10 : 1;
    const int ahead = u / 1000 ? u / 1000 : 4;
    if ((copies != 8 && copies != 16 && copies != 32) || (na != 1 && na != 2) || (ahead != 4 && ahead != 8))
        return hipErrorInvalidValue;
    int grid = cfg->grid;
    if (!grid) {
        // about 4096 waves in multiples of 256 workgroups, between 256 and
        // 1024 workgroups (the fastest of grids 256..2048 measured on MI355X
        // at K = 4096, 8192, 14336 and 28672); never more workgroups than rows
        int g = (4096 / S) & ~255;
        g = g < 256 ? 256 : (g > 1024 ? 1024 : g);
        grid = N < g ? N : g;
    }
    const uint8_t* c8 = (const uint8_t*)codes;
    const uint16_t* x16 = (const uint16_t*)x;
#define DG_NF4(TT, AA, HH)                                                                                    \
    if (copies == TT && na == AA && ahead == HH) {                                                            \
        hipLaunchKernelGGL((k_nf4<TT, AA, HH>), dim3(grid), dim3(S * kWave), 0, s, c8, absmax, table, x16, y, N, \
                           K, B);                                                                             \
        return hipGetLastError();                                                                             \
    }
    DG_NF4(16, 1, 4) DG_NF4(16, 2, 4) DG_NF4(8, 1, 4) DG_NF4(8, 2, 4)
    DG_NF4(16, 1, 8) DG_NF4(16, 2, 8) DG_NF4(8, 1, 8) DG_NF4(8, 2, 8)
    DG_NF4(32, 1, 4) DG_NF4(32, 2, 4) DG_NF4(32, 1, 8) DG_NF4(32, 2, 8)
#undef DG_NF4
    return hipErrorInvalidValue;
}

hipError_t launch_quantize_nf4(const float* w, void* codes, float* absmax, const float* table, int64_t N,
                               int64_t K, int B, hipStream_t s) {
    const int64_t nblocks = N * (K / B);
    if (nblocks == 0) return hipSuccess;
    hipLaunchKernelGGL(k_quantize_nf4, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, s, w,
                       (uint8_t*)codes, absmax, table, nblocks, B);
    return hipGetLastError();
}

}  // namespace dg
