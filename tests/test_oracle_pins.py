"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test ties an oracle routine to the pages' definitions, to exact
mathematics (rational arithmetic, closed forms, brute force on tiny inputs) or
to an independent library routine (numpy's binary16 casts, numpy.argmax), so
that a plausible mistake -- a dropped term, a wrong sign, a swapped nibble, a
transposed operand, a misused leading dimension -- fails at least one of them.
CPU only.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hex(s):
    return np.frombuffer(bytes.fromhex(s.replace(" ", "")), dtype=np.uint8)


# ---------------------------------------------------------------------------
# binary16 / bfloat16 decoding and rounding (IEEE-754 definition vs numpy)
# ---------------------------------------------------------------------------

def test_half_decode_matches_numpy_for_every_pattern(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero is kept
    assert math.copysign(1.0, orc.half_to_double(0x8000)) == -1.0


def test_bf16_decode_matches_float32_upper_half_for_every_pattern(orc):
    bits = np.arange(65536, dtype=np.uint32)
    ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = np.array([orc.bf16_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_float_to_half_rne_matches_numpy(orc):
    g = np.random.default_rng(1)
    # random bit patterns over every exponent, plus exact midpoints between halves
    rnd = g.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    h = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    mids = ((h[:-1] + h[1:]) / 2).astype(np.float32)          # exact in float32 (12 bits)
    near = np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf))
    edge = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e30, 5.96e-8, 2.98e-8,
                     2.9802322e-08, 2.9802326e-08, 6.1e-5, np.inf, -np.inf], dtype=np.float32)
    vals = np.concatenate([rnd, mids, -mids, near[0], near[1], edge]).astype(np.float32)
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([orc.float_to_half_rne(float(v)) for v in vals], dtype=np.uint16)
    isn = np.isnan(vals)
    assert np.array_equal(got[~isn], ref[~isn])
    assert np.all((got[isn] & 0x7C00) == 0x7C00) and np.all((got[isn] & 0x3FF) != 0)


# ---------------------------------------------------------------------------
# dense GEMV: exact rational sums, closed forms, layout
# ---------------------------------------------------------------------------

def _exact_gemv(Wf, xf):
    """Exact rational y = W x from float64 values (binary16/bfloat16 are exact there)."""
    out = []
    for row in Wf:
        out.append(sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(row, xf)), Fraction(0)))
    return out


def _check_fp64_sum(y, Wf, xf):
    """|y - exact| <= gamma_K * sum |w x|, the error bound of a recursive fp64 sum."""
    K = Wf.shape[1]
    u = 2.0 ** -53
    gamma = K * u / (1 - K * u)
    exact = _exact_gemv(Wf, xf)
    for n in range(Wf.shape[0]):
        bound = gamma * float(np.sum(np.abs(Wf[n] * xf)))
        assert abs(Fraction(float(y[n])) - exact[n]) <= Fraction(bound) + Fraction(0), (n, y[n], float(exact[n]))


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_dense_gemv_against_exact_rationals_non_square(orc, fmt):
    g = np.random.default_rng(7)
    N, K = 5, 24                         # N != K catches a transposed operand
    Wf32 = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    xf32 = g.standard_normal(K).astype(np.float32)
    # adversarial row: large cancelling terms plus small ones
    Wf32[2, :4] = [1000.0, -1000.0, 0.001, 3.0]
    if fmt == "f16":
        Wb, xb = Wf32.astype(np.float16).view(np.uint16), xf32.astype(np.float16).view(np.uint16)
        Wf, xf = Wb.view(np.float16).astype(np.float64), xb.view(np.float16).astype(np.float64)
        y = orc.gemv_f16(Wb, xb)
    else:
        import synth
        Wb, xb = synth.to_bf16_bits(Wf32), synth.to_bf16_bits(xf32)
        Wf = (Wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        y = orc.gemv_bf16(Wb, xb)
    assert y.shape == (N,)
    _check_fp64_sum(y, Wf, xf)
    # a dropped term anywhere shows up: every product is far above the fp64 error
    prods = np.abs(Wf * xf)
    assert np.all(np.abs(y - Wf @ xf) < 1e-3 * prods[prods > 0].min())


def test_gemv_f16_small_integers_are_exact(orc):
    # all-ones W with small-integer x: y = sum x exactly
    K = 40
    x = np.arange(-20, 20, dtype=np.float16)
    W = np.ones((3, K), dtype=np.float16)
    W[1] *= -1
    W[2, ::2] = 0
    y = orc.gemv_f16(W.view(np.uint16), x.view(np.uint16))
    assert y.tolist() == [float(x.astype(np.float64).sum()), -float(x.astype(np.float64).sum()),
                          float(x.astype(np.float64)[1::2].sum())]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_one_hot_x_selects_a_column_and_ldw_padding_is_ignored(orc, fmt):
    import synth
    g = np.random.default_rng(3)
    N, K, ldw = 6, 16, 24
    Wf32 = g.standard_normal((N, ldw)).astype(np.float32)
    Wb = Wf32.astype(np.float16).view(np.uint16) if fmt == "f16" else synth.to_bf16_bits(Wf32)
    Wb = Wb.copy()
    Wb[:, K:] = 0x7E00 if fmt == "f16" else 0x7FC0      # NaN in the padding
    dec = (lambda b: b.view(np.float16).astype(np.float64)) if fmt == "f16" else \
          (lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    fn = orc.gemv_f16 if fmt == "f16" else orc.gemv_bf16
    one = np.uint16(0x3C00 if fmt == "f16" else 0x3F80)
    for k in (0, 5, K - 1):
        x = np.zeros(K, dtype=np.uint16)
        x[k] = one
        y = fn(Wb, x, N=N, K=K, ldw=ldw)
        assert np.array_equal(y, dec(Wb[:, k]))


def test_dense_gemv_agrees_with_numpy_fp64_matmul(orc):
    import synth
    W = synth.normal_f16_bits((0, 0, 0, 0), (64, 512), 0.02)
    x = synth.normal_f16_bits((0, 1, 0, 0), (512,), 1.0)
    y = orc.gemv_f16(W, x)
    ref = W.view(np.float16).astype(np.float64) @ x.view(np.float16).astype(np.float64)
    assert np.max(np.abs(y - ref)) <= 1e-13 * np.max(np.abs(ref))


def test_subnormal_halves_are_kept(orc):
    # a row made only of binary16 subnormals (|w| < 2^-14) times x = 1
    W = np.arange(1, 1025, dtype=np.uint32).astype(np.uint16).reshape(1, -1)      # every positive subnormal
    x = np.full(1024, 0x3C00, dtype=np.uint16)
    y = orc.gemv_f16(W, x)
    assert y[0] == sum(range(1, 1025)) * 2.0 ** -24


# ---------------------------------------------------------------------------
# Q4_0 x Q8_1
# ---------------------------------------------------------------------------

def _golden():
    with open(os.path.join(GOLDEN, "q4_0_q8_1_worked.json")) as f:
        return json.load(f)


def test_q4_0_worked_blocks(orc):
    for ex in _golden()["dot_examples"]:
        W, X = _hex(ex["q4_0_block_hex"]), _hex(ex["q8_1_block_hex"])
        assert W.size == 18 and X.size == 36
        y = orc.gemv_q4_0_q8_1(W, X, N=1, K=32, M=1)
        assert y[0, 0] == ex["y"], ex["name"]


def _py_decode_q4_0(blk):
    d = Fraction(float(np.frombuffer(bytes(blk[:2]), dtype=np.float16)[0]))
    vals = [None] * 32
    for i in range(16):
        vals[i] = (int(blk[2 + i]) & 15) - 8
        vals[i + 16] = (int(blk[2 + i]) >> 4) - 8
    return [d * v for v in vals]


def _py_decode_q8_1(blk):
    d = Fraction(float(np.frombuffer(bytes(blk[:2]), dtype=np.float16)[0]))
    return [d * int(v) for v in np.frombuffer(bytes(blk[4:36]), dtype=np.int8)]


def _random_blocks(g, nblk, kind):
    size = 18 if kind == "q4" else 36
    b = g.integers(0, 256, size=(nblk, size), dtype=np.uint8)
    scales = (g.standard_normal(nblk) * 0.3).astype(np.float16).view(np.uint16)
    b[:, 0] = scales & 0xFF
    b[:, 1] = scales >> 8
    return b


def test_q4_0_against_brute_force_dequantise_then_dot(orc):
    """Dequantise every weight and activation to an exact rational and sum all
    products: a different route to the same definition, in exact arithmetic."""
    g = np.random.default_rng(11)
    N, K, M = 3, 96, 2
    nb = K // 32
    W = _random_blocks(g, N * nb, "q4")
    X = _random_blocks(g, M * nb, "q8")
    Y = orc.gemv_q4_0_q8_1(W, X, N=N, K=K, M=M)
    for m in range(M):
        xv = sum((_py_decode_q8_1(X[m * nb + b]) for b in range(nb)), [])
        for n in range(N):
            wv = sum((_py_decode_q4_0(W[n * nb + b]) for b in range(nb)), [])
            exact = sum((a * c for a, c in zip(wv, xv)), Fraction(0))
            # the oracle's only rounding is the fp64 sum over nb exactly-scaled blocks
            assert abs(Fraction(float(Y[m, n])) - exact) <= abs(exact) * Fraction(nb, 2 ** 52) + Fraction(1, 2 ** 1000)


def test_q4_0_oracle_dequant_helpers_match_python_decoding(orc):
    g = np.random.default_rng(5)
    for blk in _random_blocks(g, 8, "q4"):
        assert [Fraction(v) for v in orc.dequant_q4_0_block(blk)] == _py_decode_q4_0(blk)
    for blk in _random_blocks(g, 8, "q8"):
        assert [Fraction(v) for v in orc.dequant_q8_1_block(blk)] == _py_decode_q8_1(blk)


def test_q4_0_invariants(orc):
    g = np.random.default_rng(13)
    N, K = 4, 128
    nb = K // 32
    W = _random_blocks(g, N * nb, "q4")
    X1 = _random_blocks(g, nb, "q8")
    # identical activation columns give identical output columns
    X = np.concatenate([X1, X1, X1])
    Y = orc.gemv_q4_0_q8_1(W, X, N=N, K=K, M=3)
    assert np.array_equal(Y[0], Y[1]) and np.array_equal(Y[0], Y[2])
    # doubling every weight scale (exact in binary16 here) doubles y exactly
    d = W[:, :2].copy().view(np.uint16).reshape(-1).view(np.float16)
    if np.all(np.abs(d.astype(np.float32)) < 1000):
        W2 = W.copy()
        W2[:, :2] = (d.astype(np.float32) * 2).astype(np.float16).view(np.uint8).reshape(-1, 2)
        Y2 = orc.gemv_q4_0_q8_1(W2, X1, N=N, K=K, M=1)
        assert np.array_equal(Y2[0], 2 * Y[0])
    # the -8 offset: codes all 8 give y = 0 whatever the activations
    W8 = W.copy()
    W8[:, 2:] = 0x88
    assert np.all(orc.gemv_q4_0_q8_1(W8, X1, N=N, K=K, M=1) == 0)


def test_q4_0_quantiser_worked_blocks(orc):
    for ex in _golden()["q4_0_quantiser_examples"]:
        j = np.arange(32)
        tie = np.zeros(32)
        tie[:2] = [-2, 2]
        x = {"(j-16)/4 for j in 0..31": (j - 16) / 4, "(16-j)/4 for j in 0..31": (16 - j) / 4,
             "0 for j in 0..31": np.zeros(32), "[-2, 2, 0 x 30]": tie}[ex["x"]].astype(np.float32)
        got = orc.quantize_q4_0(x.reshape(1, 32))
        assert bytes(got.reshape(-1)) == bytes(_hex(ex["block_hex"])), ex["name"]


def test_q8_1_quantiser_worked_blocks(orc):
    for ex in _golden()["q8_1_quantiser_examples"]:
        x = np.array(ex["x"], dtype=np.float32).reshape(1, 32)
        got = orc.quantize_q8_1(x)
        assert bytes(got.reshape(-1)) == bytes(_hex(ex["block_hex"])), ex["name"]


def test_quantiser_properties_on_random_blocks(orc):
    g = np.random.default_rng(17)
    w = g.standard_normal((64, 256)).astype(np.float32)
    Wq = orc.quantize_q4_0(w).reshape(-1, 18)
    blocks = w.reshape(-1, 32)
    for blk, x in zip(Wq, blocks):
        m = x[np.argmax(np.abs(x))]
        d32 = np.float32(m) / np.float32(-8.0)
        assert np.frombuffer(bytes(blk[:2]), np.float16)[0] == np.float16(d32)
        codes = np.concatenate([blk[2:] & 15, blk[2:] >> 4]).astype(np.int64)
        assert codes[np.argmax(np.abs(x))] == 0                 # the extreme value maps to q = 0
        err = np.abs(x.astype(np.float64) - (codes - 8) * float(d32))
        clamped = codes == 15
        assert np.all(err[~clamped] <= abs(float(d32)) * (0.5 + 1e-5))
        assert np.all(err[clamped] <= abs(float(d32)) * (1.0 + 1e-5))
    a = g.standard_normal((8, 256)).astype(np.float32)
    Xq = orc.quantize_q8_1(a).reshape(-1, 36)
    for blk, x in zip(Xq, a.reshape(-1, 32)):
        d32 = np.float32(np.max(np.abs(x))) / np.float32(127.0)
        q = np.frombuffer(bytes(blk[4:]), np.int8).astype(np.int64)
        assert np.frombuffer(bytes(blk[:2]), np.float16)[0] == np.float16(d32)
        assert abs(q[np.argmax(np.abs(x))]) == 127
        assert np.all(np.abs(x - q * float(d32)) <= float(d32) * (0.5 + 1e-5))
        s = np.frombuffer(bytes(blk[2:4]), np.float16)[0]
        assert s == np.float16(d32 * np.float32(q.sum()))


# ---------------------------------------------------------------------------
# Q8_0 x Q8_1
# ---------------------------------------------------------------------------

def _golden_q8_0():
    with open(os.path.join(GOLDEN, "q8_0_q8_1_worked.json")) as f:
        return json.load(f)


def _py_decode_q8_0(blk):
    d = Fraction(float(np.frombuffer(bytes(blk[:2]), dtype=np.float16)[0]))
    return [d * int(v) for v in np.frombuffer(bytes(blk[2:34]), dtype=np.int8)]


def _random_q8_0_blocks(g, nblk):
    b = g.integers(0, 256, size=(nblk, 34), dtype=np.uint8)
    b[:, 2:][b[:, 2:] == 0x80] = 0x81          # codes stay in [-127, 127]
    scales = (g.standard_normal(nblk) * 0.3).astype(np.float16).view(np.uint16)
    b[:, 0] = scales & 0xFF
    b[:, 1] = scales >> 8
    return b


def test_q8_0_worked_blocks(orc):
    for ex in _golden_q8_0()["dot_examples"]:
        W, X = _hex(ex["q8_0_block_hex"]), _hex(ex["q8_1_block_hex"])
        assert W.size == 34 and X.size == 36
        y = orc.gemv_q8_0_q8_1(W, X, N=1, K=32, M=1)
        assert y[0, 0] == ex["y"], ex["name"]


def test_q8_0_against_brute_force_dequantise_then_dot(orc):
    g = np.random.default_rng(31)
    N, K, M = 3, 128, 2
    nb = K // 32
    W = _random_q8_0_blocks(g, N * nb)
    X = _random_blocks(g, M * nb, "q8")
    Y = orc.gemv_q8_0_q8_1(W, X, N=N, K=K, M=M)
    for m in range(M):
        xv = sum((_py_decode_q8_1(X[m * nb + b]) for b in range(nb)), [])
        for n in range(N):
            wv = sum((_py_decode_q8_0(W[n * nb + b]) for b in range(nb)), [])
            exact = sum((a * c for a, c in zip(wv, xv)), Fraction(0))
            assert abs(Fraction(float(Y[m, n])) - exact) <= abs(exact) * Fraction(nb, 2 ** 52) + Fraction(1, 2 ** 1000)
    for blk in W[:6]:
        assert [Fraction(v) for v in orc.dequant_q8_0_block(blk)] == _py_decode_q8_0(blk)


def test_q8_0_invariants(orc):
    g = np.random.default_rng(37)
    N, K = 4, 128
    nb = K // 32
    W = _random_q8_0_blocks(g, N * nb)
    X1 = _random_blocks(g, nb, "q8")
    X = np.concatenate([X1, X1])
    Y = orc.gemv_q8_0_q8_1(W, X, N=N, K=K, M=2)
    assert np.array_equal(Y[0], Y[1])
    # negating every weight code (exact for codes in [-127, 127]) negates y exactly
    Wn = W.copy()
    Wn[:, 2:] = (-(W[:, 2:].view(np.int8).astype(np.int16))).astype(np.int8).view(np.uint8)
    assert np.array_equal(orc.gemv_q8_0_q8_1(Wn, X1, N=N, K=K, M=1)[0], -Y[0])


def test_q8_0_quantiser_worked_blocks_and_properties(orc):
    for ex in _golden_q8_0()["q8_0_quantiser_examples"]:
        got = orc.quantize_q8_0(np.array(ex["x"], dtype=np.float32).reshape(1, 32))
        assert bytes(got.reshape(-1)) == bytes(_hex(ex["block_hex"])), ex["name"]
    g = np.random.default_rng(41)
    w = g.standard_normal((16, 256)).astype(np.float32)
    for blk, x in zip(orc.quantize_q8_0(w).reshape(-1, 34), w.reshape(-1, 32)):
        d32 = np.float32(np.max(np.abs(x))) / np.float32(127.0)
        q = np.frombuffer(bytes(blk[2:]), np.int8).astype(np.int64)
        assert np.frombuffer(bytes(blk[:2]), np.float16)[0] == np.float16(d32)
        assert abs(q[np.argmax(np.abs(x))]) == 127
        assert np.all(np.abs(x - q * float(d32)) <= float(d32) * (0.5 + 1e-5))


# ---------------------------------------------------------------------------
# argmax
# ---------------------------------------------------------------------------

def _parse(v):
    return {"-0": -0.0, "+0": 0.0, "nan": math.nan, "inf": math.inf, "-inf": -math.inf}.get(v, v) \
        if isinstance(v, str) else float(v)


def test_argmax_hand_rows(orc):
    with open(os.path.join(GOLDEN, "argmax_rows.json")) as f:
        rows = json.load(f)["rows"]
    for r in rows:
        x = np.array([_parse(v) for v in r["x"]], dtype=np.float32)
        assert orc.argmax_rows(x)[0] == r["idx"], r


def test_argmax_brute_force_against_numpy_with_heavy_ties(orc):
    g = np.random.default_rng(19)
    R, C, ld = 200, 77, 80
    x = g.integers(0, 3, size=(R, ld)).astype(np.float32)
    x[:, C:] = 1e30                                   # padding beyond C must be ignored
    x[5, 10] = np.nan
    x[6, [3, 40]] = np.nan
    x[7, :] = -0.0
    x[7, 9] = 0.0
    idx = orc.argmax_rows(x, C=C, ld=ld)
    ref = np.argmax(x[:, :C], axis=1)                 # numpy: first max, first NaN
    assert np.array_equal(idx, ref)


def test_argmax_is_invariant_under_any_chunking(orc):
    g = np.random.default_rng(23)
    x = g.integers(0, 4, size=(1, 1000)).astype(np.float32)
    whole = orc.argmax_rows(x)[0]
    for chunk in (1, 7, 64, 333):
        best = None
        for c0 in range(0, 1000, chunk):
            i = c0 + int(orc.argmax_rows(x[:, c0:c0 + chunk].copy())[0])
            if best is None or x[0, i] > x[0, best]:
                best = i
        assert best == whole


def _golden_argcompare():
    with open(os.path.join(GOLDEN, "argcompare_rows.json")) as f:
        return json.load(f)


def test_argcompare_hand_rows(orc):
    g = _golden_argcompare()
    for r in g["f32_min_rows"]:
        x = np.array([_parse(v) for v in r["x"]], dtype=np.float32)
        assert orc.argcompare_rows(x, "f32", "min")[0] == r["idx"], r
    for r in g["bits_rows"]:
        bits = np.array([int(b, 16) for b in r["bits"]], dtype=np.uint16)
        assert orc.argcompare_rows(bits, r["dtype"], r["op"])[0] == r["idx"], r
    # argmax on float32 is the argmax routine's own definition
    with open(os.path.join(GOLDEN, "argmax_rows.json")) as f:
        for r in json.load(f)["rows"]:
            x = np.array([_parse(v) for v in r["x"]], dtype=np.float32)
            assert orc.argcompare_rows(x, "f32", "max")[0] == r["idx"], r


def test_argcompare_against_numpy_every_dtype_with_heavy_ties(orc):
    g = np.random.default_rng(43)
    R, C, ld = 120, 61, 64
    for op in ("max", "min"):
        npfn = np.argmax if op == "max" else np.argmin
        v = (g.integers(0, 3, size=(R, ld)) - 1).astype(np.float32)
        v[:, C:] = np.nan                                 # padding beyond C must be ignored
        v[3, 20] = np.nan
        v[4, [2, 30]] = np.nan
        v[5, :] = -0.0
        v[5, 11] = 0.0
        h = v.astype(np.float16)
        b = (v.view(np.uint32) >> 16).astype(np.uint16)   # exact: these values fit in bfloat16
        ref = npfn(v[:, :C], axis=1)                      # numpy: first extreme, first NaN
        assert np.array_equal(orc.argcompare_rows(v, "f32", op, C=C, ld=ld), ref)
        assert np.array_equal(orc.argcompare_rows(h.view(np.uint16), "f16", op, C=C, ld=ld),
                              npfn(h[:, :C], axis=1))
        assert np.array_equal(orc.argcompare_rows(b, "bf16", op, C=C, ld=ld), ref)


def test_argmin_is_argmax_of_the_negation(orc):
    """-x reverses every comparison and keeps NaN a NaN and +-0 equal, so the
    first minimum of x is the first maximum of -x, bit patterns included."""
    g = np.random.default_rng(47)
    x = g.integers(-3, 4, size=(50, 200)).astype(np.float32) * np.float32(0.5)
    x[1, 7] = np.nan
    x[2, :] = 0.0
    x[2, 5] = -0.0
    assert np.array_equal(orc.argcompare_rows(x, "f32", "min"), orc.argmax_rows(-x))
    h = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(orc.argcompare_rows(h, "f16", "min"), orc.argcompare_rows(h ^ np.uint16(0x8000), "f16", "max"))


# ---------------------------------------------------------------------------
# streaming-read checksum
# ---------------------------------------------------------------------------

def test_checksum_closed_forms(orc):
    assert orc.checksum_u32(np.zeros(1000, np.uint32)) == 0
    n = 1 << 20
    assert orc.checksum_u32(np.arange(n, dtype=np.uint32)) == (n * (n - 1) // 2) % 2**32
    assert orc.checksum_u32(np.full(3, 0xFFFFFFFF, np.uint32)) == (3 * 0xFFFFFFFF) % 2**32
    g = np.random.default_rng(29)
    w = g.integers(0, 2**32, size=12345, dtype=np.uint64).astype(np.uint32)
    assert orc.checksum_u32(w) == int(sum(int(v) for v in w)) % 2**32


# ---------------------------------------------------------------------------
# NF4: 4-bit table codes, per-block absmax, bfloat16 activations
# ---------------------------------------------------------------------------

def _golden_nf4():
    with open(os.path.join(GOLDEN, "nf4_worked.json")) as f:
        return json.load(f)


def _bf16(v):
    """bfloat16 bits of values that bfloat16 holds exactly."""
    a = np.asarray(v, dtype=np.float32)
    bits = a.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)
    return (bits >> 16).astype(np.uint16)


def test_nf4_worked_example(orc):
    g = _golden_nf4()
    codes = np.stack([_hex(h) for h in g["codes_hex"]])
    y = orc.gemv_nf4(codes, np.array(g["absmax"], np.float32), np.array(g["table"], np.float32),
                     _bf16(g["x"]), g["N"], g["K"], g["B"])
    assert list(y) == g["y"]


def test_nf4_closed_forms(orc):
    """Constant codes and absmax: y = table[c] * a * sum(x); one nibble of each
    byte selected by the activations; one block selected by the activations."""
    t = np.array([(j - 7) / 4 for j in range(16)], np.float32)
    K, B = 256, 64
    g = np.random.default_rng(5)
    x = np.round(g.standard_normal(K) * 8) / 8                      # exact in bfloat16
    xb = _bf16(x)
    for c in (0, 3, 7, 15):
        codes = np.full((1, K // 2), c * 17, np.uint8)
        y = orc.gemv_nf4(codes, np.full((1, K // B), 0.5, np.float32), t, xb, 1, K, B)
        assert y[0] == float(t[c]) * 0.5 * math.fsum(x)
    hi, lo = 13, 2
    codes = np.full((1, K // 2), hi * 16 + lo, np.uint8)
    even = np.zeros(K)
    even[0::2] = 1.0
    y = orc.gemv_nf4(codes, np.ones((1, K // B), np.float32), t, _bf16(even), 1, K, B)
    assert y[0] == float(t[hi]) * (K // 2)                          # even weights: the high nibble
    y = orc.gemv_nf4(codes, np.ones((1, K // B), np.float32), t, _bf16(1.0 - even), 1, K, B)
    assert y[0] == float(t[lo]) * (K // 2)
    absmax = np.array([[1.0, 2.0, 4.0, 8.0]], np.float32)
    codes = np.full((1, K // 2), 15 * 17, np.uint8)
    for b in range(K // B):
        sel = np.zeros(K)
        sel[b * B:(b + 1) * B] = 1.0
        y = orc.gemv_nf4(codes, absmax, t, _bf16(sel), 1, K, B)
        assert y[0] == float(t[15]) * float(absmax[0, b]) * B


def test_nf4_against_brute_force_in_rationals(orc):
    """Tiny random operands evaluated exactly (fractions) from the definition;
    the double sum may differ only by its own rounding."""
    g = np.random.default_rng(41)
    t = np.sort(g.standard_normal(16)).astype(np.float32)
    N, K, B = 3, 64, 32
    codes = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    absmax = np.abs(g.standard_normal((N, K // B))).astype(np.float32)
    x = g.standard_normal(K).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    xv = [Fraction(float((np.uint32(v) << 16).view(np.float32))) for v in xb]
    y = orc.gemv_nf4(codes, absmax, t, xb, N, K, B)
    for n in range(N):
        exact = Fraction(0)
        for j in range(K // 2):
            for k, q in ((2 * j, int(codes[n, j]) >> 4), (2 * j + 1, int(codes[n, j]) & 15)):
                exact += Fraction(float(t[q])) * Fraction(float(absmax[n, k // B])) * xv[k]
        assert abs(Fraction(y[n]) - exact) <= Fraction(2.0 ** -40) * sum(
            abs(Fraction(float(t[q]))) for q in range(16)) * max(abs(v) for v in xv) * 64


def test_nf4_quantiser_round_trip_nearest_level_and_ties(orc):
    import synth
    t = synth.nf4_table()
    g = np.random.default_rng(43)
    N, K, B = 4, 256, 64
    q = g.integers(0, 16, size=(N, K))
    q[:, ::B] = 15                                                  # every block holds the level 1.0
    a = np.float32(2.0) ** g.integers(-3, 4, size=(N, K // B)).astype(np.float32)
    w = t[q] * np.repeat(a, B, axis=1)
    codes, absmax = orc.quantize_nf4(w.astype(np.float32), t, B)
    assert np.array_equal(absmax, a)
    got = np.stack([codes >> 4, codes & 15], axis=2).reshape(N, K)
    assert np.array_equal(got, q)
    # random weights: the nearest level of r = w / absmax (binary32), ties to the lower
    w = g.standard_normal((N, K)).astype(np.float32)
    codes, absmax = orc.quantize_nf4(w, t, B)
    assert np.array_equal(absmax, np.abs(w).reshape(N, K // B, B).max(axis=2))
    got = np.stack([codes >> 4, codes & 15], axis=2).reshape(N, K)
    r = (w.reshape(N, K // B, B) / absmax[:, :, None]).reshape(N, K).astype(np.float64)
    dist = np.abs(r[:, :, None] - t.astype(np.float64)[None, None, :])
    best = dist.min(axis=2)
    assert np.all(dist[np.arange(N)[:, None], np.arange(K)[None, :], got] == best)
    # exact ties: r on a midpoint of a dyadic table goes to the lower level
    td = np.array([(j - 7) / 8 for j in range(16)], np.float32)
    wt = np.array([[1.0, 0.0625, -0.0625, 0.1875, 0.0, -1.0, 0.5, 0.4375]], np.float32)
    codes, absmax = orc.quantize_nf4(wt, td, 8)
    got = np.stack([codes >> 4, codes & 15], axis=2).reshape(-1)
    assert list(got) == [15, 7, 6, 8, 7, 0, 11, 10]
    assert absmax[0, 0] == 1.0
    # a block of zeros: absmax 0, every code the level of 0
    codes, absmax = orc.quantize_nf4(np.zeros((1, 64), np.float32), t, 64)
    assert absmax[0, 0] == 0 and np.all(codes == 7 * 17)


def test_nf4_workload_table(orc):
    """The NF4 workload's table: increasing, exact 0 and +-1 at the ends, and
    its levels are standard-normal quantiles (scipy's, an independent routine)."""
    import synth
    from scipy.stats import norm
    t = synth.nf4_table()
    assert t.dtype == np.float32 and t.size == 16 and np.all(np.diff(t) > 0)
    assert t[0] == -1.0 and t[7] == 0.0 and t[15] == 1.0
    p_hi = 1.0 - (1.0 / 32.0 + 1.0 / 30.0) / 2.0
    top = norm.ppf(p_hi)
    pos = norm.ppf(np.linspace(p_hi, 0.5, 9)[:-1]) / top
    neg = -norm.ppf(np.linspace(p_hi, 0.5, 8)[:-1]) / top
    ref = np.sort(np.concatenate([pos, [0.0], neg])).astype(np.float32)
    assert np.allclose(t, ref, rtol=0, atol=2e-7)
