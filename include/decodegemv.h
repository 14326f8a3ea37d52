/*
 * decodegemv.h -- C ABI of libdecodegemv, the batch-1 / small-batch LLM decode
 * matrix-vector product y = W x for AMD Instinct MI355X (gfx950, wave64).
 *
 * Every weight byte of a decode step is read once and never reused, so a call
 * costs (bytes moved) / (HBM bandwidth); the kernels behind these calls are
 * bandwidth kernels (batch1-cdna README, opening paragraph and "FP16 GEMV"
 * section).
 *
 * Conventions shared by every call
 *  - Pointers named d_* or documented as "device" are device (HBM) pointers
 *    owned by the caller; the library never frees, retains or allocates them
 *    and allocates no device memory of its own.
 *  - Every call only enqueues work on `stream` (a hipStream_t; NULL means the
 *    null stream) and returns without synchronising.  Outputs are valid once
 *    the stream has reached that point.
 *  - Arguments are checked before anything is enqueued.  On any error the
 *    call returns a non-zero dg_status, launches nothing and writes nothing.
 *    The library never aborts or exits.
 *  - Sizes are element counts unless the name says bytes.  Empty work (a zero
 *    row or column count) returns DG_OK and launches nothing.
 *  - Thread-safety: calls carry no shared mutable state except the per-thread
 *    text of the last HIP error.
 */
#ifndef DECODEGEMV_H
#define DECODEGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DG_OK = 0,
    DG_ERR_NULL = 1,        /* a required pointer is NULL                         */
    DG_ERR_MISALIGNED = 2,  /* a pointer or leading dimension breaks its alignment */
    DG_ERR_SHAPE = 3,       /* a size or count is outside the documented contract  */
    DG_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required          */
    DG_ERR_HIP = 5,         /* the HIP runtime reported an error when launching    */
    DG_ERR_ARG = 6          /* another argument (a launch override) is invalid     */
} dg_status;

/* A hipStream_t, kept opaque so that this header needs no HIP include. */
typedef void* dg_stream;

/* Static text for a status code. */
const char* dg_status_string(dg_status status);

/* Text of the last DG_ERR_HIP seen by the calling thread ("" if none). */
const char* dg_last_hip_error(void);

/* ------------------------------------------------------------------------
 * Streaming-read ceiling probe
 *
 * Reads every byte of `buf` exactly once, 16 bytes per lane per load.  Each
 * workgroup b stores the wrapping (mod 2^32) sum of the little-endian 32-bit
 * words it read into d_partials[b] (a plain store, overwriting); the wrapping
 * sum of all G partials is the sum of every word of the buffer.  The sums are
 * what keep the loads alive.  No atomics are used: one same-address atomic per
 * workgroup would serialise and be measured instead of HBM.  This is the
 * denominator measurement of the batch1-cdna README ("01-ceiling": a read of a
 * buffer far larger than the last-level cache with 4 x 32-bit vector loads,
 * normal or non-temporal).
 *
 *   buf          device, 16-byte aligned, `bytes` long.
 *   bytes        multiple of 16 (0 is allowed: nothing is launched or written).
 *   d_partials   device uint32[G], 4-byte aligned, where G = grid_blocks, or
 *                DG_READ_DEFAULT_GRID when grid_blocks is 0; every entry is
 *                written (workgroups with no bytes to read store 0).
 *   grid_blocks  workgroups to launch; 0 = DG_READ_DEFAULT_GRID.
 *   block_threads threads per workgroup, a multiple of 64 in [64, 1024];
 *                0 = library default (512).
 *   flags        DG_READ_NONTEMPORAL: non-temporal loads (else ordinary);
 *                DG_READ_GRID_STRIDE: the page's order, consecutive lanes of
 *                the whole grid on consecutive vectors (else each wave reads
 *                8 KiB of consecutive bytes per step);
 *                DG_READ_DEEP: 16 loads in flight per lane instead of 8
 *                (16 KiB per wave step); DG_READ_SHORT: 4 (4 KiB);
 *                DG_READ_SHORTER: 2 (2 KiB) -- at most one of the three, and
 *                only in the wave-contiguous order.  A grid of
 *                bytes / (waves per workgroup * chunk) workgroups gives each
 *                wave one chunk, the shape of a one-shot GEMV launch;
 *                DG_READ_CAP(n), n in 1..15: at most n workgroups resident
 *                per CU (the launch reserves 1/n of a CU's 160 KiB of LDS
 *                that the kernel never touches), which bounds the streams
 *                in flight;
 *                DG_READ_HALF: only the even waves of each workgroup read,
 *                the odd ones hold their slots (the occupancy of a GEMV that
 *                gives each row to two waves of which one covers it);
 *                wave-contiguous order, a multiple of 128 threads per
 *                workgroup.
 * Errors: DG_ERR_NULL (buf or d_partials NULL with bytes > 0),
 * DG_ERR_MISALIGNED (buf not 16-byte aligned, d_partials not 4-byte aligned),
 * DG_ERR_SHAPE (bytes % 16 != 0), DG_ERR_ARG (grid/block/flags out of range).
 * ------------------------------------------------------------------------ */
enum { DG_READ_NONTEMPORAL = 1, DG_READ_GRID_STRIDE = 2, DG_READ_DEEP = 4, DG_READ_SHORT = 8,
       DG_READ_SHORTER = 16, DG_READ_HALF = 32, DG_READ_CAP_SHIFT = 8, DG_READ_DEFAULT_GRID = 1024 };
#define DG_READ_CAP(n) ((int)(n) << DG_READ_CAP_SHIFT)

dg_status dg_stream_read(const void* buf, size_t bytes, uint32_t* d_partials,
                         int grid_blocks, int block_threads, int flags,
                         dg_stream stream);

/* ------------------------------------------------------------------------
 * Dense GEMV, batch 1, fp32 accumulation
 *
 *   y[n] = sum_{k<K} W[n*ldw + k] * x[k],   0 <= n < N
 *
 * batch1-cdna README, "FP16 GEMV" section: one output element per row as the
 * dot product of x with one row of W, products accumulated in fp32 and
 * reduced across the lanes of a wavefront.  The summation order inside a row
 * is fixed by the kernel, so results are bit-reproducible run to run.
 *
 *   W    device, row-major [N][ldw] of 16-bit values, 16-byte aligned.
 *   x    device, [K] 16-bit values, 16-byte aligned.
 *   N    rows (>= 0; 0 launches nothing).  N < 2^31.
 *   K    columns used, multiple of 8, 0 <= K < 2^31 (K = 0 writes zeros).
 *   ldw  row stride in elements, ldw >= K, ldw % 8 == 0.
 * Errors: DG_ERR_NULL, DG_ERR_MISALIGNED (W or x not 16-byte aligned, y not
 * aligned to its element), DG_ERR_SHAPE (K % 8, ldw < K, ldw % 8, negative or
 * too large sizes), DG_ERR_HIP.
 * ------------------------------------------------------------------------ */

/* binary16 operands; y is [N] binary16, rounded to nearest-even from the
 * fp32 sum. */
dg_status dg_gemv_f16(const void* W, const void* x, void* y,
                      int64_t N, int64_t K, int64_t ldw, dg_stream stream);

/* bfloat16 operands; y is [N] float32 (the fp32 sum itself). */
dg_status dg_gemv_bf16(const void* W, const void* x, float* y,
                       int64_t N, int64_t K, int64_t ldw, dg_stream stream);

/* ------------------------------------------------------------------------
 * Q4_0 weights x Q8_1 activations, M = 1..24 activation columns
 *
 *   Y[m][n] = sum_b d4(n,b) * d8(m,b) * sum_{j<32} (q4(n,b,j) - 8) * q8(m,b,j)
 *
 * The quantised-weight decode GEMV of "The kernel that waited for itself"
 * (Q4_0/Q8_1 harness; the small-batch kernel for 1..24 columns) and of the
 * 4-bit M = 1 GEMV of the bitsandbytes issue on 70B 4-bit decode.  The inner
 * 32-term sum is exact in int32; the scaling and the sum over blocks are
 * fp32.  The fp16 block sum s of Q8_1 is not used.  (With exactly 17 columns
 * the 17th column's block sum is formed as four exact int32 partial sums of
 * 8 terms, each scaled in fp32, so its rounding differs from the other
 * columns' by a few fp32 ulps.)
 *
 *   Wq  device, N rows of K/32 Q4_0 blocks, 18 bytes each (binary16 d, then 16
 *       code bytes: byte i = weight i in the low nibble, weight i+16 in the
 *       high nibble), rows packed back to back; 16-byte aligned.
 *   Xq  device, M columns of K/32 Q8_1 blocks, 36 bytes each (binary16 d,
 *       binary16 s, 32 int8 codes), column m starting at block m*K/32;
 *       16-byte aligned (the kernels copy it in 16-byte pieces).
 *   Y   device float32 [M][N] (column m of the result at Y + m*N).
 *   N   rows, 0 <= N < 2^31.  K: multiple of 256, 0 <= K <= 2^26.
 *   M   columns, 0 <= M <= 24 (0 launches nothing).
 * Errors: DG_ERR_NULL, DG_ERR_MISALIGNED, DG_ERR_SHAPE, DG_ERR_HIP.
 * ------------------------------------------------------------------------ */
dg_status dg_gemv_q4_0(const void* Wq, const void* Xq, float* Y,
                       int64_t N, int64_t K, int M, dg_stream stream);

/* ------------------------------------------------------------------------
 * Q4_0 weights x fp32 activations: the Q8_1 quantisation and the GEMV in one
 * call
 *
 *   Xq = Q8_1(x) exactly as dg_quantize_q8_1 stores it, then
 *   Y  = exactly dg_gemv_q4_0(Wq, Xq, Y, N, K, M)
 *
 * The activation conversion before every quantised GEMV is the unfused step
 * the "Capability Gain" paper's LLM-decode notes price at 27.9 us per call,
 * more than the matrix product at a fifth of its cells.  Here it is the
 * quantiser's launch (one lane per activation, about 1.8 us for a column of
 * 8192), then the GEMV's.  A one-launch form for one column (M = 1, K <=
 * 16384), in which every workgroup of the row-streaming GEMV quantises the
 * column into its LDS copy while its first weight rows are in flight, is
 * selected by dg_gemv_q4_0_f32_ex with variant DG_VARIANT_Q4_LDSROW; on
 * MI355X it is slower than the two launches (each of hundreds of workgroups
 * repeats the whole conversion), so it is not the default.  With several
 * columns, whose matrix-core kernels re-stage the columns for every 16-row
 * tile, a conversion inside the GEMV would be repeated for every tile.
 *
 *   Wq, Y, N, K, M  as for dg_gemv_q4_0.
 *   x   device float32 [M][K], rows packed; 16-byte aligned.
 *   Xq  device, M columns of K/32 Q8_1 blocks (36 bytes each), 16-byte
 *       aligned: receives the quantised columns, byte for byte those of
 *       dg_quantize_q8_1 (so later calls on the same activations, such as
 *       the gate and up projections, can use dg_gemv_q4_0 on them).
 *       Required, except by the one-launch form (there NULL stores nothing).
 * Errors: DG_ERR_NULL, DG_ERR_MISALIGNED, DG_ERR_SHAPE, DG_ERR_HIP.
 * ------------------------------------------------------------------------ */
dg_status dg_gemv_q4_0_f32(const void* Wq, const float* x, float* Y, void* Xq,
                           int64_t N, int64_t K, int M, dg_stream stream);

/* ------------------------------------------------------------------------
 * Q4_0 weights in 16-row tiles: the rearrangement, and the small-batch GEMV
 * over it, M = 1..24 activation columns
 *
 *   Y = the sums of dg_gemv_q4_0 (the same exact int32 block sums and exact
 *       binary16 scale products), added in the order of this kernel
 *
 * The small-batch page ("The kernel that waited for itself", what remains
 * open) ends at a floor set by the weight format, and the bitsandbytes issue
 * on 4-bit decode (its analysis of the naive kernel) asks for a layout in
 * which consecutive lanes read consecutive 128-bit chunks before unpacking.
 * This is that layout for Q4_0: the information of the row-major blocks byte
 * for byte, rearranged once (when the weights are loaded) so that each
 * 16-byte load of a lane is directly the matrix-core operand of four blocks
 * of one row.  Scales are copied unchanged; each 4-bit code q is stored as q
 * XOR 8 (the two's-complement nibble of q - 8).  For tile t (rows
 * 16t..16t+15) and group s of 8 blocks, 2304 bytes at (t * K/256 + s) * 2304:
 *   bytes    0..1023  16 bytes per lane l = 16g + n: dword j = code bytes
 *                     4g..4g+3 of row 16t+n, block 8s+j (nibbles XOR 8);
 *   bytes 1024..2047  the same for blocks 8s+4..8s+7;
 *   bytes 2048..2303  16 bytes per row n: the binary16 scales of blocks
 *                     8s..8s+7, block 8s+i in half i%2 of dword i/2.
 * Rows past N (the last tile's padding) hold code nibbles 0 and scale 0.
 *
 * dg_q4_0_tiles_bytes: bytes of the tiled copy, ceil(N/16) * K/256 * 2304
 *   (0 for an invalid shape).
 * dg_repack_q4_0_tiles: Wq (row-major Q4_0 as for dg_gemv_q4_0, 2-byte
 *   aligned) -> Wt (device, dg_q4_0_tiles_bytes(N, K) bytes, 16-byte
 *   aligned); K % 256 == 0, K <= 2^26, 0 <= N < 2^31.  Wq is unchanged.
 * dg_gemv_q4_0_tiles: as dg_gemv_q4_0 with Wt in place of Wq.  Every
 *   workgroup copies its activation columns over its range of K into LDS
 *   once.  The columns may be split over several workgroups of one row group
 *   (column slices: each computes its own columns, nothing is exchanged);
 *   when K is split over several workgroups of one row group and slice (rows
 *   too long for the columns to fit a workgroup's LDS), their partial sums
 *   meet in the caller's workspace:
 *   ws        device, ws_bytes >= dg_gemv_q4_0_tiles_workspace_bytes(N, K,
 *             M) (0: ws may be NULL), 16-byte aligned.  Its first 64 KiB
 *             hold ticket counters (one per row group and column slice, at
 *             the same place for every shape), which must be zero before the
 *             first call: fill
 *             the workspace with zeros once after allocating it.  Every call
 *             leaves them zero again, so one workspace serves calls of any
 *             shapes in turn; calls that may overlap in time need workspaces
 *             of their own.
 *   Partial sums are added in a fixed order (K parts within a workgroup,
 *   then the workgroups' ranges in order of K): the result does not depend
 *   on which workgroup finishes last.  K = 0 gives Y = 0.
 * Errors: DG_ERR_NULL, DG_ERR_MISALIGNED, DG_ERR_SHAPE, DG_ERR_WORKSPACE,
 * DG_ERR_HIP.
 * ------------------------------------------------------------------------ */
size_t dg_q4_0_tiles_bytes(int64_t N, int64_t K);
dg_status dg_repack_q4_0_tiles(const void* Wq, void* Wt, int64_t N, int64_t K, dg_stream stream);
size_t dg_gemv_q4_0_tiles_workspace_bytes(int64_t N, int64_t K, int M);
dg_status dg_gemv_q4_0_tiles(const void* Wt, const void* Xq, float* Y, int64_t N, int64_t K, int M,
                             void* ws, size_t ws_bytes, dg_stream stream);

/* ------------------------------------------------------------------------
 * Q8_0 weights x Q8_1 activations, M = 1..24 activation columns
 *
 *   Y[m][n] = sum_b dw(n,b) * d8(m,b) * sum_{j<32} qw(n,b,j) * q8(m,b,j)
 *
 * The 8-bit weight format that "The kernel that waited for itself" runs next
 * to Q4_0 through the same Q8_1-activation path (its four-model comparison).
 * Exact int32 inner sums, fp32 scaling and sum over blocks (the 17th column
 * of a 17-column call as for Q4_0: four exact partial sums, each scaled).
 *
 *   Wq  device, N rows of K/32 Q8_0 blocks, 34 bytes each (binary16 d, then
 *       32 int8 codes), rows packed back to back; 16-byte aligned.
 *   Xq, Y, N, K, M  as for dg_gemv_q4_0 (Xq 16-byte aligned, K % 256 == 0,
 *       K <= 2^26, M <= 24).
 * Errors: DG_ERR_NULL, DG_ERR_MISALIGNED, DG_ERR_SHAPE, DG_ERR_HIP.
 * ------------------------------------------------------------------------ */
dg_status dg_gemv_q8_0(const void* Wq, const void* Xq, float* Y,
                       int64_t N, int64_t K, int M, dg_stream stream);

/* ------------------------------------------------------------------------
 * Q8_0 weights in 16-row tiles: the rearrangement, and the small-batch GEMV
 * over it, M = 1..24 activation columns
 *
 *   Y = the sums of dg_gemv_q8_0 (exact int32 block sums, exact binary16
 *       scale products), added in the order of this kernel
 *
 * The tiled layout of dg_repack_q4_0_tiles for the 8-bit format ("The kernel
 * that waited for itself" runs Q8_0 through the same small-batch path; the
 * bitsandbytes issue's 128-bit-chunk layout).  Scales and codes are copied
 * unchanged.  For tile t (rows 16t..16t+15) and group s of 8 blocks, 4352
 * bytes at (t * K/256 + s) * 4352:
 *   bytes 1024h..1024h+1023 (h = 0..3)  16 bytes per lane l = 16g + n:
 *                     code dwords g and 4 + g of row 16t+n, block 8s+2h,
 *                     then the same of block 8s+2h+1;
 *   bytes 4096..4351  16 bytes per row n: the binary16 scales of blocks
 *                     8s..8s+7, block 8s+i in half i%2 of dword i/2.
 * Rows past N hold codes 0 and scale 0.  Scales must be finite.
 *
 * dg_q8_0_tiles_bytes: ceil(N/16) * K/256 * 4352 (0 for an invalid shape).
 * dg_repack_q8_0_tiles: Wq (row-major Q8_0 as for dg_gemv_q8_0, 2-byte
 *   aligned) -> Wt (device, dg_q8_0_tiles_bytes(N, K) bytes, 16-byte
 *   aligned); K % 256 == 0, K <= 2^26, 0 <= N < 2^31.
 * dg_gemv_q8_0_tiles, dg_gemv_q8_0_tiles_workspace_bytes (and
 *   dg_gemv_q8_0_tiles_ex, with the launch overrides below): as the Q4_0
 *   tiled calls, with the same workspace rules.
 * Errors: DG_ERR_NULL, DG_ERR_MISALIGNED, DG_ERR_SHAPE, DG_ERR_WORKSPACE,
 * DG_ERR_ARG (an override not built or not fitting), DG_ERR_HIP.
 * ------------------------------------------------------------------------ */
size_t dg_q8_0_tiles_bytes(int64_t N, int64_t K);
dg_status dg_repack_q8_0_tiles(const void* Wq, void* Wt, int64_t N, int64_t K, dg_stream stream);
size_t dg_gemv_q8_0_tiles_workspace_bytes(int64_t N, int64_t K, int M);
dg_status dg_gemv_q8_0_tiles(const void* Wt, const void* Xq, float* Y, int64_t N, int64_t K, int M,
                             void* ws, size_t ws_bytes, dg_stream stream);

/* ------------------------------------------------------------------------
 * NF4 weights (4-bit codes into a 16-entry float table, per-block absmax)
 * x bfloat16 activations, one column
 *
 *   y[n] = sum_k table[q(n,k)] * absmax[n][k/B] * x[k]
 *
 * The lookup-table 4-bit M = 1 GEMV of the bitsandbytes issue on 70B 4-bit
 * decode (benchmark table: 28672 x 8192 NF4 weights against a bfloat16
 * activation; its optimisation phases: a float table quant_map, a per-block
 * absmax, float arithmetic).  The page fixes no byte layout; this library
 * reads it as follows:
 *
 *   codes   device, N rows of K/2 bytes, rows back to back; byte j of a row
 *           holds weight 2j in its HIGH nibble and weight 2j+1 in its LOW
 *           nibble; 16-byte aligned.
 *   absmax  device float32 [N][K/B] (absmax[n][b] scales weights bB..bB+B-1
 *           of row n); 16-byte aligned.
 *   table   device float32 [16], any finite values; 16-byte aligned.  The
 *           default kernel multiplies by the values themselves; variants
 *           DG_VARIANT_NF4_UNITS and DG_VARIANT_NF4_MFMA hold each value
 *           (scaled by a power of two) as a binary16 high part plus a
 *           binary16 remainder, about 22 significant bits (within about
 *           2^-23 of it, relative).
 *   x       device bfloat16 [K]; 16-byte aligned.
 *   y       device float32 [N]; 4-byte aligned.
 *   N       rows, 0 <= N < 2^31.
 *   K       multiple of 256 and of 4*B, 0 <= K <= 32768 (a workgroup has
 *           one wave per 2048 weights of a row).
 *   B       block size: 32, 64, 128 or 256.
 * Products and sums are fp32 (bfloat16 activations widened exactly); the
 * sum order is fixed by K, not by the launch.  K = 0 gives y = 0.
 * Errors: DG_ERR_NULL, DG_ERR_MISALIGNED, DG_ERR_SHAPE, DG_ERR_HIP.
 * ------------------------------------------------------------------------ */
dg_status dg_gemv_nf4(const void* codes, const float* absmax, const float* table, const void* x, float* y,
                      int64_t N, int64_t K, int B, dg_stream stream);

/* NF4 quantiser (the step that produces the operands of dg_gemv_nf4), per
 * block of B weights of a row: absmax = the largest |w| (binary32); r = w /
 * absmax correctly rounded in binary32 (r = 0 when absmax is 0); the code is
 * the number of j in 0..14 with r > (table[j] + table[j+1]) * 0.5f, each
 * midpoint in binary32 -- the nearest table level, a tie going to the lower
 * one.  table must be increasing.
 *   w       device float32 [N][K]; 16-byte aligned.
 *   codes   device, N*K/2 bytes, layout as for dg_gemv_nf4; 2-byte aligned.
 *   absmax  device float32 [N][K/B]; 4-byte aligned.
 *   table   device float32 [16]; 4-byte aligned.
 *   K multiple of B, B in {32, 64, 128, 256}.
 * Errors: DG_ERR_NULL, DG_ERR_MISALIGNED, DG_ERR_SHAPE, DG_ERR_HIP. */
dg_status dg_quantize_nf4(const float* w, void* codes, float* absmax, const float* table,
                          int64_t N, int64_t K, int B, dg_stream stream);

/* ------------------------------------------------------------------------
 * Quantisers (the step before dg_gemv_q4_0 / dg_gemv_q8_0)
 *
 * Q8_1, per 32-activation block: a = max|x|; d = a/127 (fp32); q = x/d
 * rounded half away from zero, clamped to [-127, 127] (d = 0 gives q = 0);
 * stored d = binary16(d), stored s = binary16(d * sum q).
 * Q4_0, per 32-weight block: m = the first element of largest |x|, sign
 * kept; d = m/-8 (fp32); q = min(15, floor(x/d + 8.5)) (d = 0 gives q = 8);
 * stored d = binary16(d).
 * Q8_0, per 32-weight block: a = max|x|; d = a/127 (fp32); q = x/d rounded
 * half away from zero, clamped to [-127, 127] (d = 0 gives q = 0); stored
 * d = binary16(d).
 * The per-call conversion cost of activations is the subject of the
 * "Capability Gain" paper's note on unfused conversion; the formats are those
 * of the Q4_0/Q8_1 harness in "The kernel that waited for itself".
 *
 *   x / w   device float32 [M][K] / [N][K], 16-byte aligned, rows packed.
 *   Xq / Wq device output, layouts as for dg_gemv_q4_0 / dg_gemv_q8_0; Xq
 *           4-byte aligned, Wq 2-byte aligned.
 *   K       multiple of 32.
 * Errors: DG_ERR_NULL, DG_ERR_MISALIGNED, DG_ERR_SHAPE, DG_ERR_HIP.
 * ------------------------------------------------------------------------ */
dg_status dg_quantize_q8_1(const float* x, void* Xq, int64_t M, int64_t K,
                           dg_stream stream);
dg_status dg_quantize_q4_0(const float* w, void* Wq, int64_t N, int64_t K,
                           dg_stream stream);
dg_status dg_quantize_q8_0(const float* w, void* Wq, int64_t N, int64_t K,
                           dg_stream stream);

/* ------------------------------------------------------------------------
 * argmax over rows (greedy sampling), lowest index on ties
 *
 *   idx[r] = min{ c < C : x[r*ld + c] = max_{c'<C} x[r*ld + c'] }
 *
 * IEEE comparisons (-0 equals +0); a NaN counts as larger than every number
 * and the first NaN of a row wins.  Split reduction: each row is cut into
 * chunks reduced by separate workgroups, then merged (IREE discussion
 * "ArgCompare Benchmark Results", "VD_Split" in "Implementations Compared";
 * the result does not depend on the chunking).  Any C is handled (no
 * power-of-two padding).
 *
 *   x        device float32 [R][ld], 4-byte aligned.
 *   idx      device int64 [R], 8-byte aligned.
 *   R        rows, 0 <= R < 2^31 (0 launches nothing).
 *   C        1 <= C < 2^31 - 1.   ld >= C.
 *   ws       device workspace of at least dg_argmax_workspace_bytes(R, C)
 *            bytes, 8-byte aligned; contents on entry do not matter; the
 *            call owns it until the stream passes the call.  NULL is allowed
 *            when the required size is 0.
 * Errors: DG_ERR_NULL, DG_ERR_MISALIGNED, DG_ERR_SHAPE, DG_ERR_WORKSPACE,
 * DG_ERR_HIP.
 * ------------------------------------------------------------------------ */
size_t dg_argmax_workspace_bytes(int64_t R, int64_t C);
dg_status dg_argmax_rows(const float* x, int64_t* idx, int64_t R, int64_t C,
                         int64_t ld, void* ws, size_t ws_bytes, dg_stream stream);

/* ------------------------------------------------------------------------
 * argmax over rows without a caller workspace, allocating nothing
 *
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Results are bit-identical to dg_argmax_rows (same kernels, same
 * chunking).  The chunk keys live in a fixed array of DG_ARGMAX_SCRATCH_BYTES
 * in device memory that the library holds on each GPU it runs on until the
 * process ends; the call itself allocates nothing.  Every call on a GPU
 * shares that GPU's array, so calls that overlap on one GPU (two streams, two
 * threads) race: serialise them.  The keys need no clearing (every key read
 * is written first by the same call).
 *
 *   x, idx, R, C, ld  as for dg_argmax_rows.
 * Errors: as dg_argmax_rows; DG_ERR_WORKSPACE when
 * dg_argmax_workspace_bytes(R, C) > DG_ARGMAX_SCRATCH_BYTES (checked before
 * any launch); DG_ERR_HIP when the array's device address cannot be found on
 * the current device.
 * ------------------------------------------------------------------------ */
#define DG_ARGMAX_SCRATCH_BYTES (1u << 20)
dg_status dg_argmax_rows_noalloc(const float* x, int64_t* idx, int64_t R, int64_t C, int64_t ld,
                                 dg_stream stream);

/* ------------------------------------------------------------------------
 * The greedy decode tail fused: bfloat16 lm-head GEMV and argmax of its logits
 *
 *   y[n] = sum_k W[n*ldw + k] * x[k]  (fp32, exactly as dg_gemv_bf16)
 *   idx[0] = min{ n : y[n] = max_n' y[n'] }   (exactly as dg_argmax_rows on y)
 *
 * The last two steps of a greedy decode step: the logits of the vocabulary
 * and the token they select ("The kernel that waited for itself" checks its
 * small-batch kernel by the tokens it produces; the IREE discussion's census
 * has the argmax over a 128K vocabulary).  It runs the GEMV, then the split
 * argmax of the logits: on MI355X that is faster than argmax epilogues inside
 * the GEMV, which were built and measured (a capped grid-stride GEMV, or one
 * device-scope atomic max per workgroup, each cost more than the 0.5 MB
 * argmax pass they save).
 *
 *   W, x, N, K, ldw  as for dg_gemv_bf16; N >= 1.
 *   y        device float32 [N] for the logits, or NULL to skip storing them.
 *   idx      device int64 [1], 8-byte aligned.
 *   ws       device workspace of dg_gemv_bf16_argmax_workspace_bytes(N, K)
 *            bytes (the logits when y is NULL, and the argmax's partials),
 *            16-byte aligned; contents on entry do not matter; the call owns
 *            it until the stream passes the call.
 * Errors: DG_ERR_NULL, DG_ERR_MISALIGNED, DG_ERR_SHAPE, DG_ERR_WORKSPACE,
 * DG_ERR_HIP.
 * ------------------------------------------------------------------------ */
size_t dg_gemv_bf16_argmax_workspace_bytes(int64_t N, int64_t K);
dg_status dg_gemv_bf16_argmax(const void* W, const void* x, float* y, int64_t* idx, int64_t N, int64_t K,
                              int64_t ldw, void* ws, size_t ws_bytes, dg_stream stream);

/* ------------------------------------------------------------------------
 * ArgCompare over rows: argmax or argmin of float32, binary16 or bfloat16
 *
 *   idx[r] = min{ c < C : x[r*ld + c] = max (or min) over c' < C of x[r*ld + c'] }
 *
 * The census of the IREE discussion "ArgCompare Benchmark Results and
 * Performance Analysis" lists argmax and argmin over the last axis of f16,
 * bf16 and f32 tensors with an int64 result; this is that operation.  The
 * 16-bit inputs are widened exactly; comparisons are IEEE (-0 equals +0); a
 * NaN counts as the extreme for both operations (it propagates) and the
 * first NaN of a row wins.  Same split reduction as dg_argmax_rows.
 *
 *   x        device, R rows of ld elements of `dtype`, aligned to the
 *            element size.
 *   dtype    DG_DTYPE_F32, DG_DTYPE_F16 or DG_DTYPE_BF16.
 *   op       DG_ARG_MAX or DG_ARG_MIN.
 *   idx, R, C, ld, ws, ws_bytes  as for dg_argmax_rows (the workspace size
 *            is dg_argmax_workspace_bytes(R, C) for every dtype).
 * Errors: DG_ERR_NULL, DG_ERR_MISALIGNED, DG_ERR_SHAPE, DG_ERR_WORKSPACE,
 * DG_ERR_ARG (unknown dtype or op), DG_ERR_HIP.
 * ------------------------------------------------------------------------ */
enum { DG_DTYPE_F32 = 0, DG_DTYPE_F16 = 1, DG_DTYPE_BF16 = 2 };
enum { DG_ARG_MAX = 0, DG_ARG_MIN = 1 };

dg_status dg_argcompare_rows(const void* x, int dtype, int op, int64_t* idx, int64_t R, int64_t C,
                             int64_t ld, void* ws, size_t ws_bytes, dg_stream stream);

/* ------------------------------------------------------------------------
 * Launch overrides (measurement and A/B runs)
 *
 * The *_ex variants take a launch configuration instead of the library's
 * choice; a zero field means "library default".  `variant` selects a kernel
 * variant by the ids below; 0 = default.  Invalid combinations return
 * DG_ERR_ARG.  Results are identical to the plain calls except where a
 * variant's summation order differs (documented per variant).
 * ------------------------------------------------------------------------ */
typedef struct {
    int variant;   /* kernel variant id, 0 = default                       */
    int grid;      /* workgroups, 0 = default                              */
    int block;     /* threads per workgroup (multiple of 64), 0 = default  */
    int unroll;    /* loads in flight per lane per step, 0 = default;
                      dense DG_VARIANT_DENSE_WIDE: U + 100*(S-1) also splits
                      each row's K over S in {1,2,4} waves of a workgroup;
                      Q4_0 DG_VARIANT_Q4_LDS: rows per wave (1, 2, 4);
                      *_LDSROW / *_UNITS: row (unit) buffers per wave
                      (2..4);
                      *_MFMA: RT*10000 + KS*100 + DEPTH*10 + CB/8 (row
                      tiles and K parts per workgroup, pipeline depth,
                      blocks per chunk);
                      *_MFMA_RES: RT*10000 + KS*100 + P*10 (row tiles and
                      K parts per workgroup, 8-block chunks in flight per
                      wave);
                      NF4: code-pair table copies (8, 16, 32) + 100 * partial
                      sums per lane (1, 2) + 1000 * rows in flight (4, 8)    */
} dg_launch;

enum {
    /* dense GEMV */
    DG_VARIANT_DENSE_WIDE = 1,      /* 16 B per lane, x reloaded per row (default for large K) */
    DG_VARIANT_DENSE_XREG = 2,      /* 16 B per lane, x held in registers across rows (K <= 64*8*unroll) */
    DG_VARIANT_DENSE_NARROW1 = 3,   /* 4 B per lane, one accumulator (ablation baseline)       */
    DG_VARIANT_DENSE_NARROW4 = 4,   /* 4 B per lane, four accumulators (ablation)              */
    /* Q4_0 */
    DG_VARIANT_Q4_REGS = 11,        /* activations in registers, one row per wave (M = 1)       */
    DG_VARIANT_Q4_LDS = 12,         /* activations staged in LDS, several rows per wave          */
    DG_VARIANT_Q4_LDSROW = 13,      /* M = 1: weight rows copied to LDS with coalesced loads     */
    DG_VARIANT_Q4_MFMA = 14,        /* int8 matrix cores, 16 rows x 16 columns per instruction   */
    DG_VARIANT_Q4_UNITS = 15,       /* rows copied to LDS in units of 64 block pairs, every
                                       column from one read (M * ceil(K/4096) <= 8, K <= 16384) */
    DG_VARIANT_Q4_MFMA_RES = 16,    /* int8 matrix cores with every activation column resident in
                                       LDS for the whole K; weights through registers (the
                                       columns must fit one workgroup's LDS)                   */
    /* Q8_0 */
    DG_VARIANT_Q8_LDSROW = 21,      /* M = 1: weight rows copied to LDS (K <= 16384)             */
    DG_VARIANT_Q8_MFMA = 22,        /* int8 matrix cores                                          */
    DG_VARIANT_Q8_UNITS = 23,       /* as DG_VARIANT_Q4_UNITS, Q8_0 weights; also 9..12 columns
                                       when K <= 4096                                          */
    DG_VARIANT_Q8_MFMA_RES = 24,    /* as DG_VARIANT_Q4_MFMA_RES, Q8_0 weights                     */
    /* NF4 */
    DG_VARIANT_NF4_UNITS = 31,      /* code bytes looked up in a byte-pair table in LDS; one
                                       wave per 2048 weights of a row (block = 64*ceil(K/2048)) */
    DG_VARIANT_NF4_MFMA = 32,       /* the looked-up pairs as operands of f16 matrix-core
                                       products, 16 rows x 32 weights per instruction; K = 2048,
                                       4096 or 8192, K/128 <= B <= K/16; no block or unroll
                                       override                                                */
    DG_VARIANT_NF4_ROWS = 33        /* the default: code bytes looked up in a table of binary32
                                       value pairs (32 conflict-free copies in LDS), fp32 FMA,
                                       lane sums reduced four rows at a time; block = G row groups
                                       x 64*ceil(K/2048) (<= 1024; 0: at least eight waves),
                                       unroll = rows in flight (4, 8; 0: 8 for K of 4097..8192,
                                       else 4) + 100 * partial sums per lane (1, 2, 4; 4 only
                                       with 4 rows in flight)                                   */
};

dg_status dg_gemv_f16_ex(const void* W, const void* x, void* y, int64_t N, int64_t K,
                         int64_t ldw, const dg_launch* cfg, dg_stream stream);
dg_status dg_gemv_bf16_ex(const void* W, const void* x, float* y, int64_t N, int64_t K,
                          int64_t ldw, const dg_launch* cfg, dg_stream stream);
dg_status dg_gemv_q4_0_ex(const void* Wq, const void* Xq, float* Y, int64_t N, int64_t K,
                          int M, const dg_launch* cfg, dg_stream stream);
dg_status dg_gemv_q8_0_ex(const void* Wq, const void* Xq, float* Y, int64_t N, int64_t K,
                          int M, const dg_launch* cfg, dg_stream stream);
dg_status dg_gemv_nf4_ex(const void* codes, const float* absmax, const float* table, const void* x, float* y,
                         int64_t N, int64_t K, int B, const dg_launch* cfg, dg_stream stream);
/* dg_gemv_q4_0_tiles with a launch override: variant, grid and block 0;
 * unroll = CS*100000000 + KP*1000000 + RT*10000 + KW*100 + D selects CS
 * column slices (ceil(M/CS) columns each, none empty; CS 0 means 1) and KP
 * ranges of K per row group, RT row tiles and KW parts of the range per
 * workgroup (RT*KW waves) and D groups of 8 blocks in flight per wave
 * (built: (RT, KW, D) in (1,4,2), (1,4,4), (1,8,2), (1,8,4), (1,16,2),
 * (2,4,2), (2,4,4), (2,2,4), (2,8,2), (4,1,4), (4,2,2), (4,2,4), (4,4,2),
 * (4,4,4); CS 1..8; KP 1..16; D + 10 issues the first D groups' weight
 * loads before waiting for the column copies, an earlier order kept for
 * measurements).  The workspace this configuration needs is
 * checked against ws_bytes (DG_ERR_WORKSPACE); a configuration not built,
 * with an empty slice, or whose columns do not fit a workgroup's LDS gives
 * DG_ERR_ARG. */
dg_status dg_gemv_q4_0_tiles_ex(const void* Wt, const void* Xq, float* Y, int64_t N, int64_t K, int M,
                                void* ws, size_t ws_bytes, const dg_launch* cfg, dg_stream stream);
/* dg_gemv_q8_0_tiles with a launch override, as dg_gemv_q4_0_tiles_ex. */
dg_status dg_gemv_q8_0_tiles_ex(const void* Wt, const void* Xq, float* Y, int64_t N, int64_t K, int M,
                                void* ws, size_t ws_bytes, const dg_launch* cfg, dg_stream stream);

/* dg_gemv_q4_0_f32 with a launch override: variant DG_VARIANT_Q4_LDSROW
 * selects the one-launch form (M = 1, K <= 16384), with its grid, block and
 * unroll (row buffers per wave, 2..4); 0 fields are defaults.  The default
 * (two-launch) form takes no other override. */
dg_status dg_gemv_q4_0_f32_ex(const void* Wq, const float* x, float* Y, void* Xq, int64_t N, int64_t K, int M,
                              const dg_launch* cfg, dg_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* DECODEGEMV_H */
