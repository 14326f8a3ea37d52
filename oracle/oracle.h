/*
 * oracle.h -- plain, slow, single-threaded CPU reference for the decode GEMV path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  The product
 * (libdecodegemv and its Python binding) never links, imports or calls it,
 * and this code shares nothing with the GPU path: every routine below is
 * written from the definition of the result, in fp64 where floating point
 * is involved.
 *
 * Sources (the pages each routine follows):
 *  - bitsandbytes issue "70B 4-bit LLM decode bottlenecked by HIP kernel
 *    (kgemm_4bit_inference_naive) efficiency", benchmark table and the
 *    optimisation phases of its first comment: an M = 1 GEMV over 4-bit
 *    weights that index a 16-entry float table, scaled per block by an
 *    absmax, with bfloat16 activations and float arithmetic.
 *  - batch1-cdna README ("Microbenchmarks for the batch-size-1 LLM decode
 *    regime on AMD CDNA3"), FP16 GEMV section: y = W x, one output per row,
 *    fp16 operands, checked against a CPU reference that accumulates in double.
 *  - "The kernel that waited for itself", section "What correctness was
 *    measured against": the reference computes on the quantised values
 *    (Q4_0 weights x Q8_1 activations), not on the original floats.
 *  - IREE discussion "ArgCompare Benchmark Results and Performance Analysis",
 *    census table "ArgMax/ArgMin Operations Analysis in real-world AI models":
 *    argmax over the last axis, int64 result.
 *  - batch1-cdna README, streaming-read section: each byte of a buffer read
 *    exactly once; the checksum here is the wrapping uint32 sum of its words.
 *
 * All pointers are host pointers owned by the caller.  No routine allocates
 * except where noted, none keeps state, none prints.
 */
#ifndef DG_ORACLE_H
#define DG_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- IEEE-754 16-bit formats, decoded exactly from their bit fields ---- */

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits; subnormals,
 * infinities and NaNs included.  Every binary16 value is exact in double. */
double orc_half_to_double(uint16_t h);

/* bfloat16: the upper 16 bits of a binary32 (1 sign, 8 exponent with bias
 * 127, 7 fraction bits).  Exact in double. */
double orc_bf16_to_double(uint16_t b);

/* binary32 -> binary16, round to nearest, ties to even; overflow goes to
 * infinity, NaN stays NaN (quiet).  Used by the quantisers to store scales. */
uint16_t orc_float_to_half_rne(float f);

/* ---- dense GEMV (batch 1) ---- */

/* y[n] = sum_{k<K} W[n*ldw + k] * x[k] for n < N, summed in increasing k in
 * double over the stored 16-bit values.  W and x hold binary16 bits. */
void orc_gemv_f16(const uint16_t* W, const uint16_t* x, double* y,
                  int64_t N, int64_t K, int64_t ldw);

/* Same with bfloat16 operands. */
void orc_gemv_bf16(const uint16_t* W, const uint16_t* x, double* y,
                   int64_t N, int64_t K, int64_t ldw);

/* ---- Q4_0 x Q8_1 ---- */

/* Byte layouts (GGUF):
 *   Q4_0 block, 18 bytes: binary16 scale d, then 16 code bytes; byte i holds
 *     weight i in its low nibble and weight i+16 in its high nibble; the
 *     weight's value is (q - 8) * d.
 *   Q8_1 block, 36 bytes: binary16 scale d, binary16 s, then 32 int8 codes;
 *     the activation's value is q * d; s is a stored block sum (d * sum q),
 *     which the reference does not use.
 * W holds N rows of K/32 Q4_0 blocks; X holds M columns of K/32 Q8_1 blocks,
 * column m starting at block m*K/32; Y is [M][N]:
 *   Y[m][n] = sum_b d4(n,b) * d8(m,b) * sum_{j<32} (q4(n,b,j) - 8) * q8(m,b,j)
 * with the inner sum in exact integers and the rest in double.
 * K must be a multiple of 32. */
void orc_gemv_q4_0_q8_1(const uint8_t* Wq, const uint8_t* Xq, double* Y,
                        int64_t N, int64_t K, int64_t M);

/* Decodes one Q4_0 block into 32 doubles ((q - 8) * d); one Q8_1 block into
 * 32 doubles (q * d).  Used by the brute-force cross-checks. */
void orc_dequant_q4_0_block(const uint8_t* blk, double out[32]);
void orc_dequant_q8_1_block(const uint8_t* blk, double out[32]);

/* Quantisers that produce the test operands.
 * Q4_0, per 32-weight block: m = the element of largest magnitude (first one
 *   on ties), sign kept; d = m / -8 in binary32; code q = min(15, floor(x/d +
 *   8.5)) with x/d and the add in binary32; a block of zeros gets d = 0 and
 *   all codes 8; the stored scale is binary16(d).
 * Q8_1, per 32-activation block: a = max |x|; d = a / 127 in binary32; code
 *   q = x/d rounded half away from zero, clamped to [-127, 127]; a block of
 *   zeros gets d = 0 and codes 0; stored d = binary16(d), stored
 *   s = binary16(d * sum q) with the product in binary32.
 * w is [N][K] (Q4_0) and x is [M][K] (Q8_1); K a multiple of 32. */
void orc_quantize_q4_0(const float* w, uint8_t* Wq, int64_t N, int64_t K);
void orc_quantize_q8_1(const float* x, uint8_t* Xq, int64_t M, int64_t K);

/* ---- Q8_0 x Q8_1 ---- */

/* Q8_0 block, 34 bytes (GGUF): binary16 scale d, then 32 int8 codes; the
 * weight's value is q * d.  W holds N rows of K/32 Q8_0 blocks; X and Y as
 * for Q4_0 above:
 *   Y[m][n] = sum_b dw(n,b) * d8(m,b) * sum_{j<32} qw(n,b,j) * q8(m,b,j)
 * with the inner sum in exact integers and the rest in double ("The kernel
 * that waited for itself" runs its Q8_0 model files through the same
 * Q8_1-activation path as Q4_0).  K must be a multiple of 32. */
void orc_gemv_q8_0_q8_1(const uint8_t* Wq, const uint8_t* Xq, double* Y,
                        int64_t N, int64_t K, int64_t M);

/* Decodes one Q8_0 block into 32 doubles (q * d). */
void orc_dequant_q8_0_block(const uint8_t* blk, double out[32]);

/* Q8_0 quantiser for test operands, per 32-weight block: a = max |x|;
 * d = a / 127 in binary32; code q = x/d rounded half away from zero, clamped
 * to [-127, 127]; a block of zeros gets d = 0 and codes 0; stored
 * d = binary16(d).  w is [N][K]. */
void orc_quantize_q8_0(const float* w, uint8_t* Wq, int64_t N, int64_t K);

/* ---- NF4: 4-bit table codes with a per-block absmax, bfloat16 activations ----
 *
 * Layout (readings; the page names the table, the block-wise absmax and the
 * bfloat16 activations but not the byte layout):
 *   codes   N rows of K/2 bytes; byte j of a row holds weight 2j in its HIGH
 *           nibble and weight 2j+1 in its LOW nibble;
 *   absmax  float32 [N][K/B]: absmax[n][b] scales weights bB .. bB+B-1 of row n;
 *   table   16 float32 values (the code table);
 *   x       K bfloat16 bits.
 *   y[n] = sum_{k<K} table[q(n,k)] * absmax[n][k/B] * x[k]
 * summed in increasing k in double.  K must be a multiple of B. */
void orc_gemv_nf4(const uint8_t* codes, const float* absmax, const float* table,
                  const uint16_t* x, double* y, int64_t N, int64_t K, int64_t B);

/* The quantiser that produces the test operands, per block of B weights of a
 * row: absmax = the largest |w| (binary32); r = w / absmax in binary32 (r = 0
 * when absmax is 0); the code is the number of j in 0..14 with
 * r > (table[j] + table[j+1]) * 0.5f, each midpoint in binary32: the nearest
 * table level, a tie going to the lower one.  table must be increasing. */
void orc_quantize_nf4(const float* w, uint8_t* codes, float* absmax, const float* table,
                      int64_t N, int64_t K, int64_t B);

/* ---- argmax over rows ---- */

/* idx[r] = the lowest c < C with x[r*ld + c] equal to the row maximum.
 * Values compare as IEEE numbers (so -0 equals +0); a NaN counts as larger
 * than every number and the first NaN of a row wins.  C >= 1. */
void orc_argmax_rows(const float* x, int64_t* idx, int64_t R, int64_t C, int64_t ld);

/* ArgCompare over rows of float32, binary16 or bfloat16 values (IREE
 * discussion "ArgCompare Benchmark Results and Performance Analysis": argmax
 * and argmin over the last axis, inputs in f32/f16/bf16, int64 out).
 * dtype: 0 = float32, 1 = binary16, 2 = bfloat16; op: 0 = max, 1 = min.
 * idx[r] = the lowest c < C whose value equals the row's maximum (op 0) or
 * minimum (op 1); values are decoded exactly and compared as IEEE numbers
 * (-0 equals +0); a NaN counts as the extreme for both ops (it propagates)
 * and the first NaN of a row wins.  x points to R rows of ld elements. */
void orc_argcompare_rows(const void* x, int dtype, int op, int64_t* idx, int64_t R, int64_t C, int64_t ld);

/* ---- row-partitioned multi-threaded driver (oracle_par.c) ----
 *
 * Each routine runs the single-threaded routine above of the same name on up
 * to nthreads disjoint, contiguous ranges of output rows (columns, for the
 * Q8_1 quantiser), one POSIX thread per range, and joins them.  No arithmetic
 * is added or reordered: the outputs are bit-identical to one single-threaded
 * call.  Returns 0, or -1 if a scratch buffer could not be allocated. */
int orc_par_gemv_f16(const uint16_t* W, const uint16_t* x, double* y, int64_t N, int64_t K, int64_t ldw,
                     int nthreads);
int orc_par_gemv_bf16(const uint16_t* W, const uint16_t* x, double* y, int64_t N, int64_t K, int64_t ldw,
                      int nthreads);
int orc_par_gemv_q4_0_q8_1(const uint8_t* Wq, const uint8_t* Xq, double* Y, int64_t N, int64_t K, int64_t M,
                           int nthreads);
int orc_par_gemv_q8_0_q8_1(const uint8_t* Wq, const uint8_t* Xq, double* Y, int64_t N, int64_t K, int64_t M,
                           int nthreads);
int orc_par_gemv_nf4(const uint8_t* codes, const float* absmax, const float* table, const uint16_t* x,
                     double* y, int64_t N, int64_t K, int64_t B, int nthreads);
int orc_par_argmax_rows(const float* x, int64_t* idx, int64_t R, int64_t C, int64_t ld, int nthreads);
int orc_par_argcompare_rows(const void* x, int dtype, int op, int64_t* idx, int64_t R, int64_t C, int64_t ld,
                            int nthreads);
int orc_par_quantize_q4_0(const float* w, uint8_t* Wq, int64_t N, int64_t K, int nthreads);
int orc_par_quantize_q8_0(const float* w, uint8_t* Wq, int64_t N, int64_t K, int nthreads);
int orc_par_quantize_q8_1(const float* x, uint8_t* Xq, int64_t M, int64_t K, int nthreads);
int orc_par_quantize_nf4(const float* w, uint8_t* codes, float* absmax, const float* table, int64_t N, int64_t K,
                         int64_t B, int nthreads);

/* ---- streaming-read checksum ---- */

/* Wrapping (mod 2^32) sum of n 32-bit words. */
uint32_t orc_checksum_u32(const uint32_t* w, size_t n);

#ifdef __cplusplus
}
#endif

#endif /* DG_ORACLE_H */
