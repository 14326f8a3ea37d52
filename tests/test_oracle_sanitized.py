"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

oracle.c and its row-partitioned driver are built again with gcc's address
and undefined-behaviour sanitizers (host code; nothing here touches a GPU),
and every pin of test_oracle_pins.py and every bit-identity case of
test_oracle_par.py runs against that build in a child process.  An access
outside an array, a use after free, a signed overflow, an invalid shift or a
misaligned load in any oracle routine ends the child with a sanitizer report,
and the test fails with it.  The child's pytest captures Python-level output
only (--capture=sys), so a report written to file descriptor 2 as the
process ends is not lost with pytest's own capture.  The pins must also all
pass on the sanitized build: the sanitizers change no arithmetic
(-ffp-contract=off is kept).
"""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed to build the sanitized oracle")
def test_pins_and_threaded_driver_under_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    src = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")
    lib = oracle.compile_c(src, str(tmp_path / "liboracle_san.so"), SAN_FLAGS)
    env = dict(os.environ,
               PYTHONPATH=os.pathsep.join([ROOT, os.environ.get("PYTHONPATH", "")]),
               LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               **{oracle.LIB_ENV: lib})
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "--capture=sys",
                        "tests/test_oracle_pins.py", "tests/test_oracle_par.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    report = r.stdout[-3000:] + r.stderr[-6000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report
    assert r.returncode == 0, report
    assert " passed" in r.stdout, report


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed to build the sanitized oracle")
def test_sanitized_build_reports_a_planted_out_of_bounds_read(tmp_path):
    """The harness above can see a fault: a copy of oracle.c whose binary16
    GEMV reads one activation past the end (k <= K) is reported by
    AddressSanitizer when the dense pins run against it.  The mistake exists
    only in the temporary copy."""
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    src_path = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")
    src = open(src_path).read()
    old = "for (int64_t k = 0; k < K; ++k)\n            acc += orc_half_to_double(W[n * ldw + k])"
    assert src.count(old) == 1
    planted = tmp_path / "oracle_oob.c"
    planted.write_text(src.replace(old, old.replace("k < K", "k <= K")))
    lib = oracle.compile_c(str(planted), str(tmp_path / "liboracle_oob.so"), SAN_FLAGS)
    env = dict(os.environ,
               PYTHONPATH=os.pathsep.join([ROOT, os.environ.get("PYTHONPATH", "")]),
               LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               **{oracle.LIB_ENV: lib})
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "--capture=sys",
                        "tests/test_oracle_pins.py", "-k", "dense or gemv"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr, r.stdout[-2000:] + r.stderr[-2000:]
