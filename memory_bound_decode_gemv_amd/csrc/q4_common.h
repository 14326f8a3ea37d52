// q4_common.h -- device helpers shared by the Q4_0 x Q8_1 kernels: block and
// block-pair decoding, the v_dot4 block sums, and the LDS-DMA primitives
// (global_load_lds with explicit vmcnt waits).  Device code only.
#pragma once

#include "dg_device.h"

namespace dg {
namespace q4 {


constexpr uint32_t kNib = 0x0F0F0F0Fu;
constexpr int kPairBytes = 36;   // two Q4_0 blocks
constexpr int kQ81Bytes = 36;    // one Q8_1 block

// One column's activations for one block pair: codes of block a and block b
// (element 4i..4i+3 in dword i), scales as fp32, and c = -8 * sum(q8).
struct ActPair {
    uint32_t qa[8];
    uint32_t qb[8];
    float da, db;
    int ca, cb;
};

__device__ __forceinline__ int block_code_sum(const uint32_t* q) {
    int s = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s = dot4_i8(q[i], 0x01010101u, s);
    return s;
}

// Reads the Q8_1 blocks 2p and 2p+1 of a column (72 bytes, 8-byte aligned
// when the column start is) from global memory, as stored.  Kept apart from
// the decoding so that a kernel can issue every activation load, then its
// first weight copies, and only then wait: decoding one pair before loading
// the next would cost one memory round trip per pair before the weight
// stream starts.
__device__ __forceinline__ void load_act_raw(const uint8_t* col, int p, uint32_t v[18]) {
    const uint32_t* b = reinterpret_cast<const uint32_t*>(col + (size_t)p * (2 * kQ81Bytes));
#pragma unroll
    for (int i = 0; i < 18; ++i) v[i] = b[i];
}

// The pair load_act_raw read.  valid == false marks a lane past the end of
// the row (its loads re-read the row's last pair): only the two scales are
// zeroed, which makes its contribution exactly 0 in every kernel (the integer
// block sums are multiplied by them), and no load depends on the flag, so the
// compiler cannot move the loads into a branch behind later copies.
__device__ __forceinline__ void decode_act_pair(const uint32_t v[18], bool valid, ActPair& a) {
    a.da = valid ? half_lo_to_f32(v[0]) : 0.0f;
    a.db = valid ? half_lo_to_f32(v[9]) : 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a.qa[i] = v[1 + i];
        a.qb[i] = v[10 + i];
    }
    a.ca = -8 * block_code_sum(a.qa);
    a.cb = -8 * block_code_sum(a.qb);
}

__device__ __forceinline__ void load_act_pair(const uint8_t* col, int p, ActPair& a) {
    uint32_t v[18];
    load_act_raw(col, p, v);
    decode_act_pair(v, true, a);
}

// Loads the 9 dwords of block pair p of a weight row (non-temporal).
__device__ __forceinline__ void load_weight_pair(const uint8_t* row, int p, uint32_t w[9]) {
    const uint32_t* b = reinterpret_cast<const uint32_t*>(row + (size_t)p * kPairBytes);
    const u32x4 lo = __builtin_nontemporal_load(reinterpret_cast<const u32x4_a4*>(b));
    const u32x4 hi = __builtin_nontemporal_load(reinterpret_cast<const u32x4_a4*>(b + 4));
    w[0] = lo.x; w[1] = lo.y; w[2] = lo.z; w[3] = lo.w;
    w[4] = hi.x; w[5] = hi.y; w[6] = hi.z; w[7] = hi.w;
    w[8] = __builtin_nontemporal_load(b + 8);
}

// The unpacked codes of one weight pair: lo[i]/hi[i] of block a in 0..3,
// block b in 4..7, and the two scales.
struct WeightPair {
    uint32_t lo[8];
    uint32_t hi[8];
    float d4a, d4b;
};

__device__ __forceinline__ void unpack_weight_pair(const uint32_t w[9], WeightPair& u) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // block a: scale in bytes 0-1, codes in bytes 2..17 (straddling dwords)
        const uint32_t ca = __builtin_amdgcn_alignbit(w[i + 1], w[i], 16);
        u.lo[i] = ca & kNib;
        u.hi[i] = (ca >> 4) & kNib;
        // block b: scale in bytes 18-19, codes in bytes 20..35 (dwords 5..8)
        const uint32_t cb = w[5 + i];
        u.lo[4 + i] = cb & kNib;
        u.hi[4 + i] = (cb >> 4) & kNib;
    }
    u.d4a = half_lo_to_f32(w[0]);
    u.d4b = half_hi_to_f32(w[4]);
}

__device__ __forceinline__ float pair_dot(const WeightPair& u, const uint32_t* qa, const uint32_t* qb,
                                          float da, float db, int ca, int cb, float acc) {
    int sa = ca, sb = cb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        sa = dot4_i8(u.lo[i], qa[i], sa);       // weights 4i..4i+3
        sa = dot4_i8(u.hi[i], qa[4 + i], sa);   // weights 16+4i..16+4i+3
        sb = dot4_i8(u.lo[4 + i], qb[i], sb);
        sb = dot4_i8(u.hi[4 + i], qb[4 + i], sb);
    }
    acc = fmaf((float)sa, u.d4a * da, acc);
    acc = fmaf((float)sb, u.d4b * db, acc);
    return acc;
}

__device__ __forceinline__ int wave_in_block() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
}

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kAuxNonTemporal = 2;   // cache-policy operand of global_load_lds: nt

template <int C>
__device__ __forceinline__ void copy_row_to_lds(const uint8_t* __restrict__ row, uint8_t* buf, int nchunks,
                                                int lane) {
#pragma unroll
    for (int j = 0; j < C; ++j) {
        const int c = j * kWave + lane;
        if (c < nchunks)
            __builtin_amdgcn_global_load_lds(row + (size_t)c * 16, (lds_void_t*)(buf + j * 1024), 16, 0,
                                             kAuxNonTemporal);
    }
}

template <int N_OUTSTANDING>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N_OUTSTANDING >= 0 && N_OUTSTANDING <= 63, "wait count out of range (6-bit vmcnt)");
#define DG_WAIT(n) if constexpr (N_OUTSTANDING == n) asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory");
#define DG_WAIT8(b) DG_WAIT(b) DG_WAIT(b + 1) DG_WAIT(b + 2) DG_WAIT(b + 3) DG_WAIT(b + 4) DG_WAIT(b + 5) \
    DG_WAIT(b + 6) DG_WAIT(b + 7)
    DG_WAIT8(0) DG_WAIT8(8) DG_WAIT8(16) DG_WAIT8(24) DG_WAIT8(32) DG_WAIT8(40) DG_WAIT8(48) DG_WAIT8(56)
#undef DG_WAIT8
#undef DG_WAIT
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations
// (lgkmcnt) and meets the other waves, without draining vector-memory loads
// that are still in flight (__syncthreads would wait for vmcnt(0) as well).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Waits until at most q*C vector-memory operations are outstanding
// (0 <= q < DEPTH; larger q waits as for DEPTH - 1).
template <int C, int DEPTH, int Q = 0>
__device__ __forceinline__ void wait_ahead(int q) {
    if constexpr (Q >= DEPTH - 1) {
        wait_vmcnt<(DEPTH - 1) * C>();
    } else {
        if (q == Q) {
            wait_vmcnt<Q * C>();
            return;
        }
        wait_ahead<C, DEPTH, Q + 1>(q);
    }
}

template <int C, int DEPTH>
__device__ __forceinline__ void wait_rows_ahead(int q) {
    wait_ahead<C, DEPTH>(q);
}

// LDS bytes that hold one Q8_1 column of K elements (K % 256 == 0, so the
// column is a whole number of 16-byte slots), in whole 1 KiB copies.
__host__ __device__ constexpr int column_lds_bytes(int K) {
    return ((K / 32) * kQ81Bytes / 16 + kWave - 1) / kWave * 1024;
}

// The M = 1 kernels give every workgroup one copy of the activation column
// (in general, of any run of 16-byte slots) in LDS instead of one per wave:
// the 1 KiB copies are split over the workgroup's waves (wave w issues copies
// w, w + wpb, ...) and are issued before any weight copy, so a wave's own
// share has landed once at most its weight copies are outstanding; a barrier
// then makes every share visible.  Every copy has all 64 lanes active (lanes
// past the end re-read the first slot into the unused tail of the last KiB).
// dst is formed from the kernel's __shared__ array.
__device__ __forceinline__ void copy_slots_to_lds(const uint8_t* __restrict__ src, int slots, uint8_t* dst, int wave,
                                                  int wpb, int lane) {
    const int copies = (slots + kWave - 1) / kWave;
    for (int j = wave; j < copies; j += wpb) {
        const int c = j * kWave + lane;
        __builtin_amdgcn_global_load_lds(src + (size_t)(c < slots ? c : 0) * 16, (lds_void_t*)(dst + j * 1024), 16,
                                         0, 0);
    }
}

__device__ __forceinline__ void copy_column_to_lds(const uint8_t* __restrict__ col, int K, uint8_t* dst, int wave,
                                                   int wpb, int lane) {
    copy_slots_to_lds(col, (K / 32) * kQ81Bytes / 16, dst, wave, wpb, lane);
}

__device__ __forceinline__ void read_pair_lds(const uint8_t* buf, int p, uint32_t w[9]) {
    const uint32_t* b = reinterpret_cast<const uint32_t*>(buf + (size_t)p * kPairBytes);
#pragma unroll
    for (int i = 0; i < 9; ++i) w[i] = b[i];
}

}  // namespace q4
}  // namespace dg
