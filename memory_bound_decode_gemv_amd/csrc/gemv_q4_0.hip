// gemv_q4_0.hip -- Q4_0 weights x Q8_1 activations, M = 1..24 columns.
//
// Y[m][n] = sum_b d4(n,b) d8(m,b) sum_{j<32} (q4 - 8) q8, the quantised decode
// GEMV of "The kernel that waited for itself" (Q4_0/Q8_1 harness, small-batch
// kernel for many columns) and of the bitsandbytes issue on 4-bit M = 1 decode
// (70B MLP shape).  Design rules taken from those pages and kept here:
//  * dequantise inside the load loop, never as a separate pass (bitsandbytes
//    issue, "Path Comparison": fused 1147 us vs dequantise + matmul 7574 us);
//  * one 64-lane wavefront per row, consecutive lanes reading consecutive
//    bytes of the row (same issue, 64 threads per block and coalescing notes);
//  * loads issued as a batch before any is consumed, and register use kept low
//    enough for several waves per SIMD ("The kernel that waited for itself",
//    the 105-117 VGPR / 2 waves per SIMD wall);
//  * one kernel family for every column count, so there is no dispatch cliff
//    between 12 and 16 columns (same page, "A dip at sixteen").
//
// Arithmetic.  Each lane owns pairs of consecutive blocks (36 bytes, dword
// aligned because rows are 16-byte aligned when K % 256 == 0).  The 16 code
// bytes of a block split into low nibbles (weights 0..15) and high nibbles
// (weights 16..31) with one mask each; the unsigned codes 0..15 go straight
// into v_dot4_i32_i8 against the signed activation codes, and the -8 offset
// enters as the initial accumulator -8 * sum(q8), computed exactly once per
// activation block.  The int32 block sum is then scaled by d4 * d8 in fp32.
#include "dg_device.h"
#include "dg_internal.h"

namespace dg {
namespace {

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
// when the column start is) from global memory.
__device__ __forceinline__ void load_act_pair(const uint8_t* col, int p, ActPair& a) {
    const uint32_t* b = reinterpret_cast<const uint32_t*>(col + (size_t)p * (2 * kQ81Bytes));
    uint32_t v[18];
#pragma unroll
    for (int i = 0; i < 18; ++i) v[i] = b[i];
    a.da = half_lo_to_f32(v[0]);
    a.db = half_lo_to_f32(v[9]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a.qa[i] = v[1 + i];
        a.qb[i] = v[10 + i];
    }
    a.ca = -8 * block_code_sum(a.qa);
    a.cb = -8 * block_code_sum(a.qb);
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

// ---------------------------------------------------------------------------
// M = 1: the lane's activation pairs stay in registers for every row the wave
// handles (S * 64 pairs cover one row).  Bytes in flight are what a bandwidth
// kernel lives on, so the wave
//  * requests its first row's weights before it touches the activations
//    (their loads and the -8 * sum(q8) preparation hide under HBM latency);
//  * requests row r + stride before it computes row r (a two-row software
//    pipeline: while one row is unpacked and reduced, the next is in flight).
// The branch that guards the prefetch is wave-uniform.
// ---------------------------------------------------------------------------
template <int S>
__global__ void __launch_bounds__(256)
k_q4_m1_regs(const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Xq,
             float* __restrict__ Y, int N, int K) {
    const int lane = lane_id();
    const int wpb = blockDim.x / kWave;
    const int npairs = K >> 6;
    const size_t row_bytes = (size_t)(K >> 5) * 18;
    const int rstride = gridDim.x * wpb;
    int row = blockIdx.x * wpb + wave_in_block();
    if (row >= N) return;

    int pc[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int p = s * kWave + lane;
        pc[s] = p < npairs ? p : npairs - 1;
    }

    uint32_t w[S][9];
#pragma unroll
    for (int s = 0; s < S; ++s) load_weight_pair(Wq + (size_t)row * row_bytes, pc[s], w[s]);

    ActPair act[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        load_act_pair(Xq, pc[s], act[s]);
        if (s * kWave + lane >= npairs) {  // lanes past the end of the row contribute exactly 0
            act[s].da = 0.0f;
            act[s].db = 0.0f;
            act[s].ca = 0;
            act[s].cb = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) { act[s].qa[i] = 0; act[s].qb[i] = 0; }
        }
    }

    while (true) {
        const int next = row + rstride;
        const bool more = next < N;
        uint32_t wn[S][9];
        if (more) {
#pragma unroll
            for (int s = 0; s < S; ++s) load_weight_pair(Wq + (size_t)next * row_bytes, pc[s], wn[s]);
        }
        float acc = 0.0f;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            WeightPair u;
            unpack_weight_pair(w[s], u);
            acc = pair_dot(u, act[s].qa, act[s].qb, act[s].da, act[s].db, act[s].ca, act[s].cb, acc);
        }
        acc = wave_sum_f32(acc);
        if (lane == 0) Y[row] = acc;
        if (!more) break;
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
            for (int i = 0; i < 9; ++i) w[s][i] = wn[s][i];
        row = next;
    }
}

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
    static_assert(N_OUTSTANDING >= 0 && N_OUTSTANDING <= 31, "wait count out of range");
#define DG_WAIT(n) if constexpr (N_OUTSTANDING == n) asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory");
    DG_WAIT(0) DG_WAIT(1) DG_WAIT(2) DG_WAIT(3) DG_WAIT(4) DG_WAIT(5) DG_WAIT(6) DG_WAIT(7)
    DG_WAIT(8) DG_WAIT(9) DG_WAIT(10) DG_WAIT(11) DG_WAIT(12) DG_WAIT(13) DG_WAIT(14) DG_WAIT(15)
    DG_WAIT(16) DG_WAIT(17) DG_WAIT(18) DG_WAIT(19) DG_WAIT(20) DG_WAIT(21) DG_WAIT(22) DG_WAIT(23)
    DG_WAIT(24) DG_WAIT(25) DG_WAIT(26) DG_WAIT(27) DG_WAIT(28) DG_WAIT(29) DG_WAIT(30) DG_WAIT(31)
#undef DG_WAIT
}

// Waits until at most q*C vector-memory operations are outstanding (q < DEPTH).
template <int C, int DEPTH>
__device__ __forceinline__ void wait_rows_ahead(int q) {
    if (q == 0) wait_vmcnt<0>();
    else if (DEPTH > 2 && q == 1) wait_vmcnt<C>();
    else if (DEPTH > 3 && q == 2) wait_vmcnt<(DEPTH > 3 ? 2 * C : 0)>();
    else wait_vmcnt<(DEPTH - 1) * C>();
}

__device__ __forceinline__ void read_pair_lds(const uint8_t* buf, int p, uint32_t w[9]) {
    const uint32_t* b = reinterpret_cast<const uint32_t*>(buf + (size_t)p * kPairBytes);
#pragma unroll
    for (int i = 0; i < 9; ++i) w[i] = b[i];
}

template <int S, int C, int DEPTH>
__global__ void __launch_bounds__(256)
k_q4_m1_ldsrow(const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Xq,
               float* __restrict__ Y, int N, int K) {
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
    if (row0 >= N) return;
    // Byte offset of the wave's buffers; addresses are always formed from the
    // __shared__ array itself, so that they stay LDS addresses (ds_read) rather
    // than generic ones (flat_load).
    const int buf_off = wave * DEPTH * row_bytes;
    uint8_t* const lds_base = reinterpret_cast<uint8_t*>(lds_rows) + buf_off;

    // rows row0 + i*rstride for i = 0, 1, ...; the first DEPTH - 1 are requested now
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d) {
        const int r = row0 + d * rstride;
        if (r < N) copy_row_to_lds<C>(Wq + (size_t)r * row_bytes, lds_base + d * row_bytes, nchunks, lane);
    }

    int pc[S];
    ActPair act[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int p = s * kWave + lane;
        pc[s] = p < npairs ? p : npairs - 1;
        load_act_pair(Xq, pc[s], act[s]);
        if (p >= npairs) {   // lanes past the end of the row contribute exactly 0
            act[s].da = 0.0f;
            act[s].db = 0.0f;
            act[s].ca = 0;
            act[s].cb = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) { act[s].qa[i] = 0; act[s].qb[i] = 0; }
        }
    }

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
        acc = wave_sum_f32(acc);
        if (lane == 0) Y[row] = acc;
        slot = slot + 1 == DEPTH ? 0 : slot + 1;
    }
}

// ---------------------------------------------------------------------------
// General M: activations of a 64-pair (4096-element) chunk of K, for all M
// columns, are staged once per workgroup in LDS in structure-of-arrays form
// (quad j of pair p of column m at ((m*5 + j)*64 + p)): quads 0-1 hold block
// a's codes, 2-3 block b's, quad 4 holds (d8a, d8b, ca, cb).  Lane p of every
// wave reads pair p, so one ds_read_b128 of the wave covers 1 KiB of
// consecutive LDS.  Each wave owns R rows; each activation quad read from LDS
// serves all R rows.
// ---------------------------------------------------------------------------
constexpr int kChunkPairs = 64;
constexpr int kQuadsPerPair = 5;
constexpr int kLdsBlock = 256;   // threads per workgroup of the LDS kernel

template <int M, int R>
__global__ void __launch_bounds__(kLdsBlock)
k_q4_lds(const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Xq,
         float* __restrict__ Y, int N, int K) {
    extern __shared__ u32x4 lds[];
    const int lane = lane_id();
    const int wave = wave_in_block();
    constexpr int kWaves = kLdsBlock / kWave;
    const int npairs = K >> 6;
    const int nblk = K >> 5;
    const size_t row_bytes = (size_t)nblk * 18;
    const int ntiles = (N + kWaves * R - 1) / (kWaves * R);

    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int row0 = tile * kWaves * R + wave * R;
        float acc[R][M];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

        for (int c0 = 0; c0 < npairs; c0 += kChunkPairs) {
            // weights of this chunk: issued before the staging so that they are in flight meanwhile
            const int gp = c0 + lane;
            const bool pvalid = gp < npairs;
            const int gpc = pvalid ? gp : npairs - 1;
            uint32_t w[R][9];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int row = row0 + r < N ? row0 + r : N - 1;
                load_weight_pair(Wq + (size_t)row * row_bytes, gpc, w[r]);
            }

            __syncthreads();   // the previous chunk's readers are done
            for (int e = threadIdx.x; e < M * 2 * kChunkPairs; e += kLdsBlock) {
                const int m = e / (2 * kChunkPairs);
                const int bl = e % (2 * kChunkPairs);
                const int p = bl >> 1, half = bl & 1;
                const int gb = 2 * (c0 + p) + half;
                uint32_t q[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                float d = 0.0f;
                int c = 0;
                if (c0 + p < npairs) {
                    const uint32_t* b = reinterpret_cast<const uint32_t*>(
                        Xq + ((size_t)m * nblk + gb) * kQ81Bytes);
                    const uint32_t d0 = b[0];
#pragma unroll
                    for (int i = 0; i < 8; ++i) q[i] = b[1 + i];
                    d = half_lo_to_f32(d0);
                    c = -8 * block_code_sum(q);
                }
                u32x4* base = lds + (m * kQuadsPerPair) * kChunkPairs + p;
                base[(half * 2 + 0) * kChunkPairs] = u32x4{q[0], q[1], q[2], q[3]};
                base[(half * 2 + 1) * kChunkPairs] = u32x4{q[4], q[5], q[6], q[7]};
                uint32_t* sc = reinterpret_cast<uint32_t*>(base + 4 * kChunkPairs);
                sc[half] = __builtin_bit_cast(uint32_t, d);
                sc[2 + half] = (uint32_t)c;
            }
            __syncthreads();

            WeightPair u[R];
#pragma unroll
            for (int r = 0; r < R; ++r) unpack_weight_pair(w[r], u[r]);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const u32x4* base = lds + (m * kQuadsPerPair) * kChunkPairs + lane;
                const u32x4 a0 = base[0 * kChunkPairs];
                const u32x4 a1 = base[1 * kChunkPairs];
                const u32x4 b0 = base[2 * kChunkPairs];
                const u32x4 b1 = base[3 * kChunkPairs];
                const u32x4 sc = base[4 * kChunkPairs];
                const uint32_t qa[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                const uint32_t qb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
                const float da = __builtin_bit_cast(float, (uint32_t)sc.x);
                const float db = __builtin_bit_cast(float, (uint32_t)sc.y);
#pragma unroll
                for (int r = 0; r < R; ++r)
                    acc[r][m] = pair_dot(u[r], qa, qb, da, db, (int)sc.z, (int)sc.w, acc[r][m]);
            }
        }

#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float s = wave_sum_f32(acc[r][m]);
                if (lane == 0 && row0 + r < N) Y[(size_t)m * N + row0 + r] = s;
            }
        }
    }
}

size_t lds_bytes(int M) { return (size_t)M * kQuadsPerPair * kChunkPairs * sizeof(u32x4); }

template <int M, int R>
hipError_t launch_lds_mr(const void* Wq, const void* Xq, float* Y, int N, int K, int grid, hipStream_t s) {
    if (lds_bytes(M) > device_max_lds_per_block()) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_q4_lds<M, R>), dim3(grid), dim3(kLdsBlock), lds_bytes(M), s,
                       (const uint8_t*)Wq, (const uint8_t*)Xq, Y, N, K);
    return hipGetLastError();
}

template <int M>
hipError_t launch_lds_m(int R, const void* Wq, const void* Xq, float* Y, int N, int K, int grid, hipStream_t s) {
    if (R == 1) return launch_lds_mr<M, 1>(Wq, Xq, Y, N, K, grid, s);
    if (R == 2) return launch_lds_mr<M, 2>(Wq, Xq, Y, N, K, grid, s);
    if constexpr (M <= 4) {
        if (R == 4) return launch_lds_mr<M, 4>(Wq, Xq, Y, N, K, grid, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_lds(int M, int R, const void* Wq, const void* Xq, float* Y, int N, int K, int grid,
                      hipStream_t s) {
    switch (M) {
#define DG_M(MM) case MM: return launch_lds_m<MM>(R, Wq, Xq, Y, N, K, grid, s);
        DG_M(1) DG_M(2) DG_M(3) DG_M(4) DG_M(5) DG_M(6) DG_M(7) DG_M(8)
        DG_M(9) DG_M(10) DG_M(11) DG_M(12) DG_M(13) DG_M(14) DG_M(15) DG_M(16)
        DG_M(17) DG_M(18) DG_M(19) DG_M(20) DG_M(21) DG_M(22) DG_M(23) DG_M(24)
#undef DG_M
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_ldsrow(int K, int depth, const void* Wq, const void* Xq, float* Y, int N, int grid, int block,
                         hipStream_t s) {
    const uint8_t* w = (const uint8_t*)Wq;
    const uint8_t* x = (const uint8_t*)Xq;
    const size_t row_bytes = (size_t)(K / 32) * 18;
    const size_t lds = (size_t)(block / kWave) * depth * row_bytes;
    if (lds > device_max_lds_per_block()) return hipErrorInvalidValue;
    const int C = (int)((row_bytes + 1023) / 1024);
    const int S = (K / 64 + kWave - 1) / kWave;
#define DG_SCD(SS, CC, DD)                                                                              \
    else if (S == SS && C == CC && depth == DD)                                                         \
        hipLaunchKernelGGL((k_q4_m1_ldsrow<SS, CC, DD>), dim3(grid), dim3(block), lds, s, w, x, Y, N, K);
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

hipError_t launch_regs(int S, const void* Wq, const void* Xq, float* Y, int N, int K, int grid, int block,
                       hipStream_t s) {
    const uint8_t* w = (const uint8_t*)Wq;
    const uint8_t* x = (const uint8_t*)Xq;
    switch (S) {
        case 1: hipLaunchKernelGGL((k_q4_m1_regs<1>), dim3(grid), dim3(block), 0, s, w, x, Y, N, K); break;
        case 2: hipLaunchKernelGGL((k_q4_m1_regs<2>), dim3(grid), dim3(block), 0, s, w, x, Y, N, K); break;
        case 3: hipLaunchKernelGGL((k_q4_m1_regs<3>), dim3(grid), dim3(block), 0, s, w, x, Y, N, K); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_q4_0(const void* Wq, const void* Xq, float* Y, int N, int K, int M,
                            const dg_launch* cfg, hipStream_t s) {
    const int npairs = K / 64;
    const int S = (npairs + kWave - 1) / kWave;
    int variant = cfg && cfg->variant ? cfg->variant : 0;
    if (variant == 0) variant = (M == 1 && S <= 4) ? DG_VARIANT_Q4_LDSROW : DG_VARIANT_Q4_LDS;

    if (variant == DG_VARIANT_Q4_REGS) {
        const int block = cfg && cfg->block ? cfg->block : 256;
        if (M != 1 || S > 3 || block > 256) return hipErrorInvalidValue;   // compiled for <= 256 threads
        const int wpb = block / kWave;
        const int grid = cfg && cfg->grid ? cfg->grid : (N + wpb - 1) / wpb;
        return launch_regs(S, Wq, Xq, Y, N, K, grid, block, s);
    }
    if (variant == DG_VARIANT_Q4_LDSROW) {
        const int block = cfg && cfg->block ? cfg->block : 256;
        if (M != 1 || block > 256) return hipErrorInvalidValue;             // compiled for <= 256 threads
        // Measured on MI355X at 28672 x 8192: two row buffers per wave and at
        // most 2048 workgroups of four waves (a few rows per wave) read fastest.
        const int depth = cfg && cfg->unroll ? cfg->unroll : 2;
        const int wpb = block / kWave;
        const int rows_grid = (N + wpb - 1) / wpb;
        const int grid = cfg && cfg->grid ? cfg->grid : (rows_grid < 2048 ? rows_grid : 2048);
        return launch_ldsrow(K, depth, Wq, Xq, Y, N, grid, block, s);
    }
    if (variant == DG_VARIANT_Q4_LDS) {
        if (cfg && cfg->block && cfg->block != kLdsBlock) return hipErrorInvalidValue;
        int R = cfg && cfg->unroll ? cfg->unroll : (M <= 8 ? 2 : 1);
        const int rows_per_tile = (kLdsBlock / kWave) * R;
        const int ntiles = (N + rows_per_tile - 1) / rows_per_tile;
        const int grid = cfg && cfg->grid ? cfg->grid : ntiles;
        return launch_lds(M, R, Wq, Xq, Y, N, K, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace dg
