/*
 * oracle_par.c -- row-partitioned multi-threaded driver over the oracle.
 *
 * TEST INFRASTRUCTURE ONLY, like oracle.c: used by the tests (to compare every
 * row of the full-size decode shapes in seconds), the smoke check and the
 * benchmark's CPU-baseline leg (its all-core timing).  It holds no arithmetic
 * of the method.  Each thread calls the unchanged single-threaded routine of
 * oracle.c on a disjoint, contiguous range of output rows.  Every output row
 * of those routines depends only on its own weight row and on the shared
 * activations, and each row's sum runs in the same order whichever thread
 * computes it, so the results are bit-identical to one single-threaded call
 * (the CPU tests check this).
 *
 * Each routine returns 0, or -1 when a thread could not be started or a
 * scratch buffer could not be allocated (then the output is incomplete).
 * nthreads < 1 is taken as 1; a call never uses more threads than rows.
 */
#include "oracle.h"

#include <pthread.h>
#include <stdlib.h>
#include <string.h>

enum job_kind {
    JOB_GEMV_F16, JOB_GEMV_BF16, JOB_GEMV_Q4_0, JOB_GEMV_Q8_0, JOB_GEMV_NF4,
    JOB_ARGMAX, JOB_ARGCOMPARE, JOB_QUANT_Q4_0, JOB_QUANT_Q8_0, JOB_QUANT_Q8_1, JOB_QUANT_NF4
};

struct job {
    enum job_kind kind;
    int64_t r0, r1;           /* this thread's rows [r0, r1) */
    /* operands, as the serial routine takes them (full arrays) */
    const void* a;            /* W / Wq / codes / x / w          */
    const void* b;            /* x / Xq / absmax                 */
    const void* c;            /* table                           */
    const void* d;            /* x of NF4                        */
    void* out;                /* y / Y / idx / Wq / Xq / codes   */
    void* out2;               /* absmax of the NF4 quantiser     */
    int64_t N, K, M, ld, B;
    int dtype, op;
    int status;
};

/* Rows [r0, r1) of a quantised GEMV with M columns: the serial routine writes
 * a [M][rows] block, which is scattered into Y[M][N]. */
static int quant_gemv_rows(struct job* j, int64_t block_bytes)
{
    const int64_t rows = j->r1 - j->r0;
    const uint8_t* Wq = (const uint8_t*)j->a + j->r0 * (j->K / 32) * block_bytes;
    double* Y = (double*)j->out;
    if (j->M == 1) {
        if (block_bytes == 18) orc_gemv_q4_0_q8_1(Wq, (const uint8_t*)j->b, Y + j->r0, rows, j->K, 1);
        else orc_gemv_q8_0_q8_1(Wq, (const uint8_t*)j->b, Y + j->r0, rows, j->K, 1);
        return 0;
    }
    double* tmp = (double*)malloc((size_t)(j->M * rows) * sizeof(double));
    if (!tmp) return -1;
    if (block_bytes == 18) orc_gemv_q4_0_q8_1(Wq, (const uint8_t*)j->b, tmp, rows, j->K, j->M);
    else orc_gemv_q8_0_q8_1(Wq, (const uint8_t*)j->b, tmp, rows, j->K, j->M);
    for (int64_t m = 0; m < j->M; ++m)
        memcpy(Y + m * j->N + j->r0, tmp + m * rows, (size_t)rows * sizeof(double));
    free(tmp);
    return 0;
}

static void* run_job(void* arg)
{
    struct job* j = (struct job*)arg;
    const int64_t r0 = j->r0, rows = j->r1 - j->r0;
    j->status = 0;
    switch (j->kind) {
    case JOB_GEMV_F16:
        orc_gemv_f16((const uint16_t*)j->a + r0 * j->ld, (const uint16_t*)j->b, (double*)j->out + r0,
                     rows, j->K, j->ld);
        break;
    case JOB_GEMV_BF16:
        orc_gemv_bf16((const uint16_t*)j->a + r0 * j->ld, (const uint16_t*)j->b, (double*)j->out + r0,
                      rows, j->K, j->ld);
        break;
    case JOB_GEMV_Q4_0:
        j->status = quant_gemv_rows(j, 18);
        break;
    case JOB_GEMV_Q8_0:
        j->status = quant_gemv_rows(j, 34);
        break;
    case JOB_GEMV_NF4:
        orc_gemv_nf4((const uint8_t*)j->a + r0 * (j->K / 2), (const float*)j->b + r0 * (j->K / j->B),
                     (const float*)j->c, (const uint16_t*)j->d, (double*)j->out + r0, rows, j->K, j->B);
        break;
    case JOB_ARGMAX:
        orc_argmax_rows((const float*)j->a + r0 * j->ld, (int64_t*)j->out + r0, rows, j->K, j->ld);
        break;
    case JOB_ARGCOMPARE: {
        const size_t esz = j->dtype == 0 ? 4 : 2;
        orc_argcompare_rows((const uint8_t*)j->a + (size_t)(r0 * j->ld) * esz, j->dtype, j->op,
                            (int64_t*)j->out + r0, rows, j->K, j->ld);
        break;
    }
    case JOB_QUANT_Q4_0:
        orc_quantize_q4_0((const float*)j->a + r0 * j->K, (uint8_t*)j->out + r0 * (j->K / 32) * 18, rows, j->K);
        break;
    case JOB_QUANT_Q8_0:
        orc_quantize_q8_0((const float*)j->a + r0 * j->K, (uint8_t*)j->out + r0 * (j->K / 32) * 34, rows, j->K);
        break;
    case JOB_QUANT_Q8_1:
        orc_quantize_q8_1((const float*)j->a + r0 * j->K, (uint8_t*)j->out + r0 * (j->K / 32) * 36, rows, j->K);
        break;
    case JOB_QUANT_NF4:
        orc_quantize_nf4((const float*)j->a + r0 * j->K, (uint8_t*)j->out + r0 * (j->K / 2),
                         (float*)j->out2 + r0 * (j->K / j->B), (const float*)j->c, rows, j->K, j->B);
        break;
    }
    return NULL;
}

/* Splits rows [0, R) into up to nthreads contiguous ranges, runs one thread
 * per range (the calling thread takes the first) and joins them. */
static int run_rows(struct job proto, int64_t R, int nthreads)
{
    if (R <= 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if ((int64_t)nthreads > R) nthreads = (int)R;
    struct job* jobs = (struct job*)calloc((size_t)nthreads, sizeof(struct job));
    pthread_t* tids = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    int* started = (int*)calloc((size_t)nthreads, sizeof(int));
    if (!jobs || !tids || !started) {
        free(jobs); free(tids); free(started);
        return -1;
    }
    const int64_t per = R / nthreads, extra = R % nthreads;
    int64_t r = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = proto;
        jobs[t].r0 = r;
        r += per + (t < extra ? 1 : 0);
        jobs[t].r1 = r;
    }
    int status = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, run_job, &jobs[t]) == 0) started[t] = 1;
        else run_job(&jobs[t]);     /* no thread: run the range here */
    }
    run_job(&jobs[0]);
    for (int t = 1; t < nthreads; ++t)
        if (started[t]) pthread_join(tids[t], NULL);
    for (int t = 0; t < nthreads; ++t)
        if (jobs[t].status) status = -1;
    free(jobs); free(tids); free(started);
    return status;
}

static struct job blank(enum job_kind k)
{
    struct job j;
    memset(&j, 0, sizeof j);
    j.kind = k;
    return j;
}

int orc_par_gemv_f16(const uint16_t* W, const uint16_t* x, double* y, int64_t N, int64_t K, int64_t ldw,
                     int nthreads)
{
    struct job j = blank(JOB_GEMV_F16);
    j.a = W; j.b = x; j.out = y; j.N = N; j.K = K; j.ld = ldw;
    return run_rows(j, N, nthreads);
}

int orc_par_gemv_bf16(const uint16_t* W, const uint16_t* x, double* y, int64_t N, int64_t K, int64_t ldw,
                      int nthreads)
{
    struct job j = blank(JOB_GEMV_BF16);
    j.a = W; j.b = x; j.out = y; j.N = N; j.K = K; j.ld = ldw;
    return run_rows(j, N, nthreads);
}

int orc_par_gemv_q4_0_q8_1(const uint8_t* Wq, const uint8_t* Xq, double* Y, int64_t N, int64_t K, int64_t M,
                           int nthreads)
{
    struct job j = blank(JOB_GEMV_Q4_0);
    j.a = Wq; j.b = Xq; j.out = Y; j.N = N; j.K = K; j.M = M;
    return M > 0 ? run_rows(j, N, nthreads) : 0;
}

int orc_par_gemv_q8_0_q8_1(const uint8_t* Wq, const uint8_t* Xq, double* Y, int64_t N, int64_t K, int64_t M,
                           int nthreads)
{
    struct job j = blank(JOB_GEMV_Q8_0);
    j.a = Wq; j.b = Xq; j.out = Y; j.N = N; j.K = K; j.M = M;
    return M > 0 ? run_rows(j, N, nthreads) : 0;
}

int orc_par_gemv_nf4(const uint8_t* codes, const float* absmax, const float* table, const uint16_t* x,
                     double* y, int64_t N, int64_t K, int64_t B, int nthreads)
{
    struct job j = blank(JOB_GEMV_NF4);
    j.a = codes; j.b = absmax; j.c = table; j.d = x; j.out = y; j.N = N; j.K = K; j.B = B;
    return run_rows(j, N, nthreads);
}

int orc_par_argmax_rows(const float* x, int64_t* idx, int64_t R, int64_t C, int64_t ld, int nthreads)
{
    struct job j = blank(JOB_ARGMAX);
    j.a = x; j.out = idx; j.K = C; j.ld = ld;
    return run_rows(j, R, nthreads);
}

int orc_par_argcompare_rows(const void* x, int dtype, int op, int64_t* idx, int64_t R, int64_t C, int64_t ld,
                            int nthreads)
{
    struct job j = blank(JOB_ARGCOMPARE);
    j.a = x; j.dtype = dtype; j.op = op; j.out = idx; j.K = C; j.ld = ld;
    return run_rows(j, R, nthreads);
}

int orc_par_quantize_q4_0(const float* w, uint8_t* Wq, int64_t N, int64_t K, int nthreads)
{
    struct job j = blank(JOB_QUANT_Q4_0);
    j.a = w; j.out = Wq; j.K = K;
    return run_rows(j, N, nthreads);
}

int orc_par_quantize_q8_0(const float* w, uint8_t* Wq, int64_t N, int64_t K, int nthreads)
{
    struct job j = blank(JOB_QUANT_Q8_0);
    j.a = w; j.out = Wq; j.K = K;
    return run_rows(j, N, nthreads);
}

int orc_par_quantize_q8_1(const float* x, uint8_t* Xq, int64_t M, int64_t K, int nthreads)
{
    struct job j = blank(JOB_QUANT_Q8_1);
    j.a = x; j.out = Xq; j.K = K;
    return run_rows(j, M, nthreads);
}

int orc_par_quantize_nf4(const float* w, uint8_t* codes, float* absmax, const float* table, int64_t N, int64_t K,
                         int64_t B, int nthreads)
{
    struct job j = blank(JOB_QUANT_NF4);
    j.a = w; j.out = codes; j.out2 = absmax; j.c = table; j.K = K; j.B = B;
    return run_rows(j, N, nthreads);
}
