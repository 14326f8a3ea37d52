/*
 * oracle.c -- plain CPU reference for the decode GEMV path.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product.  It shares no code with
 * the GPU library.  Each routine states the definition it writes out; see
 * oracle.h for the sources.
 *
 * Parity pins (the tests that tie this file to something other than itself)
 * live in tests/test_oracle_pins.py.
 */
#include "oracle.h"

#include <math.h>
#include <string.h>

/* ---------------------------------------------------------------------- */
/* IEEE-754 16-bit formats                                                 */
/* ---------------------------------------------------------------------- */

double orc_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1F;
    int frac = h & 0x3FF;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);               /* subnormal: frac * 2^-24 */
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/2^10) 2^(e-15) */
    }
    return sign ? -v : v;
}

double orc_bf16_to_double(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int expo = (b >> 7) & 0xFF;
    int frac = b & 0x7F;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -133);              /* subnormal: frac * 2^-126 * 2^-7 */
    } else if (expo == 255) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(128 + frac), expo - 134); /* (1 + frac/2^7) 2^(e-127) */
    }
    return sign ? -v : v;
}

/* Round a non-negative double to an integer, ties to even. */
static double round_half_even(double n)
{
    double fl = floor(n);
    double diff = n - fl;
    if (diff > 0.5) return fl + 1.0;
    if (diff < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

uint16_t orc_float_to_half_rne(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    if (isnan(f)) return (uint16_t)(sign | 0x7E00);
    double v = fabs((double)f);
    if (isinf(f)) return (uint16_t)(sign | 0x7C00);
    if (v == 0.0) return sign;
    int ex;
    frexp(v, &ex);              /* v = fr * 2^ex, fr in [0.5, 1) */
    int e = ex - 1;             /* v in [2^e, 2^(e+1)) */
    int E = e < -14 ? -14 : e;  /* binary16 exponent range starts at -14 */
    /* A binary16 with exponent E has quantum 2^(E-10). */
    double r = round_half_even(ldexp(v, 10 - E));
    /* Normal: r in [2^10, 2^11]; exponent field E+15, fraction r - 2^10.
     * Subnormal (E = -14, r < 2^10): exponent field 0, fraction r.
     * Both are ((E + 14) << 10) + r; r = 2^11 carries into the exponent. */
    double bits = ldexp((double)(E + 14), 10) + r;
    if (bits >= (double)0x7C00) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | (uint16_t)bits);
}

/* ---------------------------------------------------------------------- */
/* Dense GEMV                                                             */
/* ---------------------------------------------------------------------- */

void orc_gemv_f16(const uint16_t* W, const uint16_t* x, double* y,
                  int64_t N, int64_t K, int64_t ldw)
{
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += orc_half_to_double(W[n * ldw + k]) * orc_half_to_double(x[k]);
        y[n] = acc;
    }
}

void orc_gemv_bf16(const uint16_t* W, const uint16_t* x, double* y,
                   int64_t N, int64_t K, int64_t ldw)
{
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += orc_bf16_to_double(W[n * ldw + k]) * orc_bf16_to_double(x[k]);
        y[n] = acc;
    }
}

/* ---------------------------------------------------------------------- */
/* Q4_0 x Q8_1                                                            */
/* ---------------------------------------------------------------------- */

static uint16_t load_u16le(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

static void store_u16le(uint8_t* p, uint16_t v)
{
    p[0] = (uint8_t)(v & 0xFF);
    p[1] = (uint8_t)(v >> 8);
}

void orc_dequant_q4_0_block(const uint8_t* blk, double out[32])
{
    double d = orc_half_to_double(load_u16le(blk));
    for (int i = 0; i < 16; ++i) {
        int lo = blk[2 + i] & 0x0F;
        int hi = blk[2 + i] >> 4;
        out[i] = (double)(lo - 8) * d;
        out[i + 16] = (double)(hi - 8) * d;
    }
}

void orc_dequant_q8_1_block(const uint8_t* blk, double out[32])
{
    double d = orc_half_to_double(load_u16le(blk));
    for (int j = 0; j < 32; ++j) out[j] = (double)(int8_t)blk[4 + j] * d;
}

void orc_gemv_q4_0_q8_1(const uint8_t* Wq, const uint8_t* Xq, double* Y,
                        int64_t N, int64_t K, int64_t M)
{
    const int64_t nb = K / 32;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                const uint8_t* wb = Wq + (n * nb + b) * 18;
                const uint8_t* xb = Xq + (m * nb + b) * 36;
                const int8_t* q8 = (const int8_t*)(xb + 4);
                int32_t isum = 0;
                for (int i = 0; i < 16; ++i) {
                    int lo = wb[2 + i] & 0x0F;   /* weight i      */
                    int hi = wb[2 + i] >> 4;     /* weight i + 16 */
                    isum += (lo - 8) * q8[i] + (hi - 8) * q8[i + 16];
                }
                double d4 = orc_half_to_double(load_u16le(wb));
                double d8 = orc_half_to_double(load_u16le(xb));
                acc += d4 * d8 * (double)isum;
            }
            Y[m * N + n] = acc;
        }
    }
}

void orc_quantize_q4_0(const float* w, uint8_t* Wq, int64_t N, int64_t K)
{
    const int64_t nb = K / 32;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < nb; ++b) {
            const float* x = w + n * K + b * 32;
            float amax = 0.0f, m = 0.0f;
            for (int j = 0; j < 32; ++j) {
                float a = fabsf(x[j]);
                if (a > amax) { amax = a; m = x[j]; }
            }
            float d = m / -8.0f;
            uint8_t q[32];
            for (int j = 0; j < 32; ++j) {
                if (d == 0.0f) { q[j] = 8; continue; }
                float v = x[j] / d + 8.5f;   /* in [0.5, 16.5] */
                int c = (int)floorf(v);
                q[j] = (uint8_t)(c > 15 ? 15 : c);
            }
            uint8_t* blk = Wq + (n * nb + b) * 18;
            store_u16le(blk, orc_float_to_half_rne(d));
            for (int i = 0; i < 16; ++i) blk[2 + i] = (uint8_t)(q[i] | (q[i + 16] << 4));
        }
    }
}

void orc_quantize_q8_1(const float* xs, uint8_t* Xq, int64_t M, int64_t K)
{
    const int64_t nb = K / 32;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t b = 0; b < nb; ++b) {
            const float* x = xs + m * K + b * 32;
            float amax = 0.0f;
            for (int j = 0; j < 32; ++j) {
                float a = fabsf(x[j]);
                if (a > amax) amax = a;
            }
            float d = amax / 127.0f;
            int8_t q[32];
            int32_t sum = 0;
            for (int j = 0; j < 32; ++j) {
                int c = 0;
                if (d != 0.0f) {
                    float r = roundf(x[j] / d);   /* halves away from zero */
                    c = (int)r;
                    if (c > 127) c = 127;
                    if (c < -127) c = -127;
                }
                q[j] = (int8_t)c;
                sum += c;
            }
            uint8_t* blk = Xq + (m * nb + b) * 36;
            store_u16le(blk, orc_float_to_half_rne(d));
            store_u16le(blk + 2, orc_float_to_half_rne(d * (float)sum));
            memcpy(blk + 4, q, 32);
        }
    }
}

/* ---------------------------------------------------------------------- */
/* Q8_0 x Q8_1                                                            */
/* ---------------------------------------------------------------------- */

void orc_dequant_q8_0_block(const uint8_t* blk, double out[32])
{
    const double d = orc_half_to_double(load_u16le(blk));
    const int8_t* q = (const int8_t*)(blk + 2);
    for (int j = 0; j < 32; ++j) out[j] = (double)q[j] * d;
}

void orc_gemv_q8_0_q8_1(const uint8_t* Wq, const uint8_t* Xq, double* Y,
                        int64_t N, int64_t K, int64_t M)
{
    const int64_t nb = K / 32;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                const uint8_t* wb = Wq + (n * nb + b) * 34;
                const uint8_t* xb = Xq + (m * nb + b) * 36;
                const int8_t* qw = (const int8_t*)(wb + 2);
                const int8_t* q8 = (const int8_t*)(xb + 4);
                int32_t isum = 0;
                for (int j = 0; j < 32; ++j) isum += (int32_t)qw[j] * q8[j];
                const double dw = orc_half_to_double(load_u16le(wb));
                const double d8 = orc_half_to_double(load_u16le(xb));
                acc += dw * d8 * (double)isum;
            }
            Y[m * N + n] = acc;
        }
    }
}

void orc_quantize_q8_0(const float* w, uint8_t* Wq, int64_t N, int64_t K)
{
    const int64_t nb = K / 32;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < nb; ++b) {
            const float* x = w + n * K + b * 32;
            float amax = 0.0f;
            for (int j = 0; j < 32; ++j) {
                float a = fabsf(x[j]);
                if (a > amax) amax = a;
            }
            const float d = amax / 127.0f;
            uint8_t* blk = Wq + (n * nb + b) * 34;
            store_u16le(blk, orc_float_to_half_rne(d));
            for (int j = 0; j < 32; ++j) {
                int c = 0;
                if (d != 0.0f) {
                    c = (int)roundf(x[j] / d);   /* halves away from zero */
                    if (c > 127) c = 127;
                    if (c < -127) c = -127;
                }
                blk[2 + j] = (uint8_t)(int8_t)c;
            }
        }
    }
}

/* ---------------------------------------------------------------------- */
/* NF4                                                                    */
/* ---------------------------------------------------------------------- */

/* The 4-bit code of weight k of a row: byte k/2, the high nibble for even k. */
static int nf4_code(const uint8_t* row, int64_t k)
{
    const uint8_t byte = row[k / 2];
    return (k % 2 == 0) ? (byte >> 4) : (byte & 0x0F);
}

void orc_gemv_nf4(const uint8_t* codes, const float* absmax, const float* table,
                  const uint16_t* x, double* y, int64_t N, int64_t K, int64_t B)
{
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t* row = codes + n * (K / 2);
        const float* a = absmax + n * (K / B);
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double w = (double)table[nf4_code(row, k)] * (double)a[k / B];
            acc += w * orc_bf16_to_double(x[k]);
        }
        y[n] = acc;
    }
}

void orc_quantize_nf4(const float* w, uint8_t* codes, float* absmax, const float* table,
                      int64_t N, int64_t K, int64_t B)
{
    for (int64_t n = 0; n < N; ++n) {
        uint8_t* row = codes + n * (K / 2);
        for (int64_t j = 0; j < K / 2; ++j) row[j] = 0;
        for (int64_t b = 0; b < K / B; ++b) {
            const float* x = w + n * K + b * B;
            float amax = 0.0f;
            for (int64_t i = 0; i < B; ++i) {
                float m = fabsf(x[i]);
                if (m > amax) amax = m;
            }
            absmax[n * (K / B) + b] = amax;
            for (int64_t i = 0; i < B; ++i) {
                const float r = amax != 0.0f ? x[i] / amax : 0.0f;
                int c = 0;
                for (int j = 0; j < 15; ++j) {
                    const float mid = (table[j] + table[j + 1]) * 0.5f;
                    if (r > mid) ++c;
                }
                const int64_t k = b * B + i;
                if (k % 2 == 0) row[k / 2] |= (uint8_t)(c << 4);
                else row[k / 2] |= (uint8_t)c;
            }
        }
    }
}

/* ---------------------------------------------------------------------- */
/* argmax                                                                 */
/* ---------------------------------------------------------------------- */

void orc_argmax_rows(const float* x, int64_t* idx, int64_t R, int64_t C, int64_t ld)
{
    for (int64_t r = 0; r < R; ++r) {
        const float* row = x + r * ld;
        int64_t best = 0;
        float bv = row[0];
        for (int64_t c = 1; c < C; ++c) {
            if (isnan(bv)) break;                 /* the first NaN wins */
            float v = row[c];
            if (isnan(v) || v > bv) { bv = v; best = c; }   /* only a strictly greater value replaces */
        }
        idx[r] = best;
    }
}

static double argcompare_value(const void* x, int dtype, int64_t i)
{
    if (dtype == 1) return orc_half_to_double(((const uint16_t*)x)[i]);
    if (dtype == 2) return orc_bf16_to_double(((const uint16_t*)x)[i]);
    return (double)((const float*)x)[i];
}

void orc_argcompare_rows(const void* x, int dtype, int op, int64_t* idx, int64_t R, int64_t C, int64_t ld)
{
    for (int64_t r = 0; r < R; ++r) {
        int64_t best = 0;
        double bv = argcompare_value(x, dtype, r * ld);
        for (int64_t c = 1; c < C; ++c) {
            if (isnan(bv)) break;                 /* the first NaN wins */
            double v = argcompare_value(x, dtype, r * ld + c);
            /* only a strictly more extreme value replaces */
            if (isnan(v) || (op == 0 ? v > bv : v < bv)) { bv = v; best = c; }
        }
        idx[r] = best;
    }
}

/* ---------------------------------------------------------------------- */
/* Streaming-read checksum                                                */
/* ---------------------------------------------------------------------- */

uint32_t orc_checksum_u32(const uint32_t* w, size_t n)
{
    uint32_t s = 0;
    for (size_t i = 0; i < n; ++i) s += w[i];
    return s;
}
