"""Mutation check of the oracle pins (CPU only).

Each mutant is a copy of oracle/oracle.c with one plausible mistake planted in
it (a dropped term, a wrong sign or offset, swapped nibbles, a transposed
operand, a misused leading dimension, a wrong tie rule, a wrong rounding).
The mutant is compiled into a temporary library and every pin in
test_oracle_pins.py is run against it, in a child process: at least one pin
must fail.  A mistake in an index can also make a pin read outside its
arrays; when the child dies of a signal, that pin has caught the mutant too
(and the test process survives it).  The planted mistakes exist only in the
temporary copies, never in oracle.c.
"""
import inspect
import os
import subprocess
import sys

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = [
    ("nibble order swapped", "int lo = wb[2 + i] & 0x0F;   /* weight i      */\n                    int hi = wb[2 + i] >> 4;",
     "int lo = wb[2 + i] >> 4;   /* weight i      */\n                    int hi = wb[2 + i] & 0x0F;"),
    ("offset -8 dropped", "isum += (lo - 8) * q8[i] + (hi - 8) * q8[i + 16];", "isum += lo * q8[i] + hi * q8[i + 16];"),
    ("offset sign flipped on high nibble", "(hi - 8) * q8[i + 16]", "(hi + 8) * q8[i + 16]"),
    ("high nibble paired with wrong activation", "(hi - 8) * q8[i + 16]", "(hi - 8) * q8[i]"),
    ("activation scale taken from column 0", "const uint8_t* xb = Xq + (m * nb + b) * 36;", "const uint8_t* xb = Xq + b * 36;"),
    ("weight scale ignored", "acc += d4 * d8 * (double)isum;", "acc += d8 * (double)isum;"),
    ("last dense term dropped", "for (int64_t k = 0; k < K; ++k)\n            acc += orc_half_to_double",
     "for (int64_t k = 0; k + 1 < K; ++k)\n            acc += orc_half_to_double"),
    ("dense W transposed", "acc += orc_half_to_double(W[n * ldw + k])", "acc += orc_half_to_double(W[k * ldw + n])"),
    ("leading dimension ignored", "acc += orc_bf16_to_double(W[n * ldw + k])", "acc += orc_bf16_to_double(W[n * K + k])"),
    ("half subnormal exponent off by one", "v = ldexp((double)frac, -24);", "v = ldexp((double)frac, -25);"),
    ("half normal bias off by one", "v = ldexp((double)(1024 + frac), expo - 25);", "v = ldexp((double)(1024 + frac), expo - 24);"),
    ("bf16 bias off by one", "v = ldexp((double)(128 + frac), expo - 134);", "v = ldexp((double)(128 + frac), expo - 133);"),
    ("half rounding ties away", "return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl + 1.0;"),
    ("q4_0 scale sign dropped", "float d = m / -8.0f;", "float d = m / 8.0f;"),
    ("q4_0 rounding offset", "float v = x[j] / d + 8.5f;", "float v = x[j] / d + 8.0f;"),
    ("q4_0 magnitude ties take the last", "if (a > amax) { amax = a; m = x[j]; }", "if (a >= amax) { amax = a; m = x[j]; }"),
    ("q8_1 rounds half to even", "float r = roundf(x[j] / d);", "float r = rintf(x[j] / d);"),
    ("q8_1 block sum unscaled", "orc_float_to_half_rne(d * (float)sum)", "orc_float_to_half_rne((float)sum)"),
    ("argmax last index wins ties", "if (isnan(v) || v > bv)", "if (isnan(v) || v >= bv)"),
    ("argmax ignores NaN", "if (isnan(v) || v > bv)", "if (v > bv)"),
    ("argmax ignores ld", "const float* row = x + r * ld;", "const float* row = x + r * C;"),
    ("q8_0 codes read unsigned", "const int8_t* qw = (const int8_t*)(wb + 2);",
     "const uint8_t* qw = (const uint8_t*)(wb + 2);"),
    ("q8_0 weight scale ignored", "acc += dw * d8 * (double)isum;", "acc += d8 * (double)isum;"),
    ("q8_0 block stride 32 bytes", "const uint8_t* wb = Wq + (n * nb + b) * 34;",
     "const uint8_t* wb = Wq + (n * nb + b) * 32;"),
    ("q8_0 activation scale taken from column 0",
     "const uint8_t* wb = Wq + (n * nb + b) * 34;\n                const uint8_t* xb = Xq + (m * nb + b) * 36;",
     "const uint8_t* wb = Wq + (n * nb + b) * 34;\n                const uint8_t* xb = Xq + b * 36;"),
    ("q8_0 quantiser rounds half to even", "c = (int)roundf(x[j] / d);   /* halves away from zero */",
     "c = (int)rintf(x[j] / d);"),
    ("argcompare min compares like max", "(op == 0 ? v > bv : v < bv)", "(op == 0 ? v > bv : v > bv)"),
    ("argcompare min keeps the last tie", "(op == 0 ? v > bv : v < bv)", "(op == 0 ? v > bv : v <= bv)"),
    ("argcompare bfloat16 decoded as binary16", "if (dtype == 2) return orc_bf16_to_double(((const uint16_t*)x)[i]);",
     "if (dtype == 2) return orc_half_to_double(((const uint16_t*)x)[i]);"),
    ("argcompare ignores ld", "double v = argcompare_value(x, dtype, r * ld + c);",
     "double v = argcompare_value(x, dtype, r * C + c);"),
    ("nf4 nibble order swapped", "return (k % 2 == 0) ? (byte >> 4) : (byte & 0x0F);",
     "return (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);"),
    ("nf4 absmax of the first block only", "(double)a[k / B];", "(double)a[0];"),
    ("nf4 absmax ignored", "const double w = (double)table[nf4_code(row, k)] * (double)a[k / B];",
     "const double w = (double)table[nf4_code(row, k)];"),
    ("nf4 absmax rows strided by B", "const float* a = absmax + n * (K / B);", "const float* a = absmax + n * B;"),
    ("nf4 quantiser ties go up", "if (r > mid) ++c;", "if (r >= mid) ++c;"),
    ("nf4 quantiser signed maximum", "float m = fabsf(x[i]);", "float m = x[i];"),
    ("nf4 quantiser packs the low nibble first", "if (k % 2 == 0) row[k / 2] |= (uint8_t)(c << 4);\n                else row[k / 2] |= (uint8_t)c;",
     "if (k % 2 == 1) row[k / 2] |= (uint8_t)(c << 4);\n                else row[k / 2] |= (uint8_t)c;"),
    ("checksum xor instead of add", "for (size_t i = 0; i < n; ++i) s += w[i];", "for (size_t i = 0; i < n; ++i) s ^= w[i];"),
]


def _pin_calls():
    calls = []
    for name, fn in sorted(vars(pins).items()):
        if not name.startswith("test_") or not callable(fn):
            continue
        params = inspect.signature(fn).parameters
        if "fmt" in params:
            calls += [(f"{name}[{f}]", fn, {"fmt": f}) for f in ("f16", "bf16")]
        else:
            calls.append((name, fn, {}))
    return calls


def test_mutant_list_applies_to_the_current_source():
    src = open(SRC).read()
    for name, old, _ in MUTANTS:
        assert src.count(old) >= 1, name


def run_pins(lib):
    """Every pin against the library at `lib`; returns the names of the pins
    that failed (the child process's side)."""
    failed = []
    with oracle.use_library(lib):
        for pin_name, fn, kw in _pin_calls():
            try:
                fn(oracle, **kw)
            except (AssertionError, ValueError, IndexError, OverflowError):
                failed.append(pin_name)
    return failed


_CHILD = """
import sys
from tests import test_oracle_mutants as m
failed = m.run_pins(sys.argv[1])
print("caught by:", ", ".join(failed) if failed else "-")
sys.exit(0 if failed else 1)
"""


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_some_pin_catches_the_mutant(tmp_path, orc, name, old, new):
    src = open(SRC).read()
    assert old in src
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(src.replace(old, new, 1))
    lib = oracle.compile_c(str(mutant), str(tmp_path / "liboracle_mutant.so"))
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([root, os.environ.get("PYTHONPATH", "")]))
    r = subprocess.run([sys.executable, "-c", _CHILD, lib], cwd=root, env=env, capture_output=True, text=True,
                       timeout=600)
    if r.returncode < 0:
        return   # a pin ran into the planted mistake hard enough to kill the process
    assert r.returncode == 0, f"no pin caught the mutant '{name}'\n{r.stdout}\n{r.stderr[-2000:]}"
