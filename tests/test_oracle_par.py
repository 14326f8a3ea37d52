"""The oracle's row-partitioned multi-threaded driver (CPU only).

It only runs the single-threaded routines on disjoint row ranges, so every
output must be bit-identical to one single-threaded call: odd row counts that
do not divide by the thread count, more threads than rows, several columns
(scattered back into [M][N]), padded leading dimensions.
"""
import numpy as np
import pytest

import synth

THREADS = [2, 3, 7, 16]


def _same(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape and a.dtype == b.dtype
    assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("threads", THREADS)
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("N,K,ldw", [(1, 8, 8), (5, 64, 72), (131, 520, 528)])
def test_par_dense_gemv_bit_identical(orc, threads, fmt, N, K, ldw):
    gen = synth.normal_f16_bits if fmt == "f16" else synth.normal_bf16_bits
    W = gen((700, 0, 0, 0), (N, ldw), 0.02)
    x = gen((700, 1, 0, 0), (K,), 1.0)
    fn = orc.gemv_f16 if fmt == "f16" else orc.gemv_bf16
    _same(fn(W, x, N=N, K=K, ldw=ldw, threads=threads), fn(W, x, N=N, K=K, ldw=ldw))


@pytest.mark.parametrize("threads", THREADS + [0])
@pytest.mark.parametrize("N,K,M", [(1, 256, 1), (37, 512, 1), (101, 768, 3), (50, 256, 24), (3, 1024, 5)])
def test_par_quantised_gemv_bit_identical(orc, threads, N, K, M):
    w = synth.normal_f32((701, 0, 0, 0), (N, K))
    x = synth.normal_f32((701, 1, 0, 0), (M, K))
    Xq = orc.quantize_q8_1(x)
    for quant, gemv in ((orc.quantize_q4_0, orc.gemv_q4_0_q8_1), (orc.quantize_q8_0, orc.gemv_q8_0_q8_1)):
        Wq = quant(w)
        _same(quant(w, threads=threads), Wq)
        _same(gemv(Wq, Xq, N, K, M, threads=threads), gemv(Wq, Xq, N, K, M))
    _same(orc.quantize_q8_1(x, threads=threads), Xq)


@pytest.mark.parametrize("threads", THREADS)
@pytest.mark.parametrize("N,K,B", [(1, 256, 64), (29, 512, 32), (70, 1024, 256)])
def test_par_nf4_bit_identical(orc, threads, N, K, B):
    table = synth.nf4_table()
    w = synth.normal_f32((702, 0, 0, 0), (N, K))
    codes, absmax = orc.quantize_nf4(w, table, B)
    c2, a2 = orc.quantize_nf4(w, table, B, threads=threads)
    _same(c2, codes)
    _same(a2, absmax)
    x = synth.normal_bf16_bits((702, 1, 0, 0), (K,))
    _same(orc.gemv_nf4(codes, absmax, table, x, N, K, B, threads=threads),
          orc.gemv_nf4(codes, absmax, table, x, N, K, B))


@pytest.mark.parametrize("threads", THREADS)
def test_par_argmax_bit_identical(orc, threads):
    x, _ = synth.argmax_logits(703, 67, 1000)
    _same(orc.argmax_rows(x, threads=threads), orc.argmax_rows(x))
    _same(orc.argmax_rows(x, C=900, ld=1000, threads=threads), orc.argmax_rows(x, C=900, ld=1000))
    h = synth.to_f16_bits(x)
    for op in ("max", "min"):
        _same(orc.argcompare_rows(h, "f16", op, threads=threads), orc.argcompare_rows(h, "f16", op))
        _same(orc.argcompare_rows(x, "f32", op, C=999, ld=1000, threads=threads),
              orc.argcompare_rows(x, "f32", op, C=999, ld=1000))


def test_par_thread_count_is_bounded(orc):
    n = orc.all_threads()
    assert 1 <= n <= orc.MAX_THREADS
