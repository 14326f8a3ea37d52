"""CPU oracle for the decode GEMV path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (``memory_bound_decode_gemv_amd``
and ``libdecodegemv.so``) never imports, links or calls it, and the two share no
code.  The arithmetic lives in ``oracle.c`` (plain single-threaded C, fp64);
``oracle_par.c`` only runs those routines on disjoint row ranges in POSIX
threads (bit-identical results; every ``threads=`` argument below selects it).
This module only builds the two with gcc and marshals numpy arrays through
ctypes.

Parity pins that tie the oracle to the pages and to mathematics rather than to
itself are in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_PAR_SRC = os.path.join(_HERE, "oracle_par.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Host threads the row-partitioned driver uses when asked for "all": the
# CPUs this process may run on, at most 16 (the host share of one GPU on an
# MI355X node).
MAX_THREADS = 16


def all_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, MAX_THREADS))


def _nthreads(threads) -> int:
    """threads: 1 = the single-threaded routine; 0 or None = all_threads()."""
    if threads is None or threads == 0:
        return all_threads()
    return max(1, int(threads))


_lib = None


def compile_c(src: str, out: str, extra_flags=()) -> str:
    """gcc -O2, no fast-math, no FMA contraction, src linked with the
    row-partitioned driver (oracle_par.c, which calls src's routines).
    extra_flags go after the defaults (the sanitizer test builds a copy with
    AddressSanitizer and UndefinedBehaviorSanitizer this way)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [
        "gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
        "-fno-fast-math", "-Wall", "-Wextra", *extra_flags, "-I", _HERE, "-o", tmp, src, _PAR_SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (when missing, stale, or forced)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(
        os.path.getmtime(_SRC), os.path.getmtime(_PAR_SRC), os.path.getmtime(os.path.join(_HERE, "oracle.h"))
    ):
        compile_c(_SRC, _LIB)
    return _LIB


# Another build of oracle.c to load instead of liboracle.so (the sanitizer
# test runs the pins in a child process against such a build).
LIB_ENV = "DG_ORACLE_LIB"


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get(LIB_ENV)
    if not path:
        if not os.path.exists(_LIB):
            build()
        path = _LIB
    _lib = _bind(ctypes.CDLL(path))
    return _lib


def _bind(lib):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.orc_half_to_double.argtypes = [ctypes.c_uint16]
    lib.orc_half_to_double.restype = ctypes.c_double
    lib.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_to_double.restype = ctypes.c_double
    lib.orc_float_to_half_rne.argtypes = [ctypes.c_float]
    lib.orc_float_to_half_rne.restype = ctypes.c_uint16
    for name in ("orc_gemv_f16", "orc_gemv_bf16"):
        getattr(lib, name).argtypes = [P, P, P, I64, I64, I64]
        getattr(lib, name).restype = None
    lib.orc_gemv_q4_0_q8_1.argtypes = [P, P, P, I64, I64, I64]
    lib.orc_gemv_q4_0_q8_1.restype = None
    lib.orc_dequant_q4_0_block.argtypes = [P, P]
    lib.orc_dequant_q8_1_block.argtypes = [P, P]
    lib.orc_quantize_q4_0.argtypes = [P, P, I64, I64]
    lib.orc_quantize_q8_1.argtypes = [P, P, I64, I64]
    lib.orc_gemv_q8_0_q8_1.argtypes = [P, P, P, I64, I64, I64]
    lib.orc_dequant_q8_0_block.argtypes = [P, P]
    lib.orc_quantize_q8_0.argtypes = [P, P, I64, I64]
    lib.orc_gemv_nf4.argtypes = [P, P, P, P, P, I64, I64, I64]
    lib.orc_gemv_nf4.restype = None
    lib.orc_quantize_nf4.argtypes = [P, P, P, P, I64, I64, I64]
    lib.orc_quantize_nf4.restype = None
    lib.orc_argmax_rows.argtypes = [P, P, I64, I64, I64]
    lib.orc_argcompare_rows.argtypes = [P, ctypes.c_int, ctypes.c_int, P, I64, I64, I64]
    lib.orc_checksum_u32.argtypes = [P, ctypes.c_size_t]
    lib.orc_checksum_u32.restype = ctypes.c_uint32
    T = ctypes.c_int
    par = {
        "orc_par_gemv_f16": [P, P, P, I64, I64, I64, T],
        "orc_par_gemv_bf16": [P, P, P, I64, I64, I64, T],
        "orc_par_gemv_q4_0_q8_1": [P, P, P, I64, I64, I64, T],
        "orc_par_gemv_q8_0_q8_1": [P, P, P, I64, I64, I64, T],
        "orc_par_gemv_nf4": [P, P, P, P, P, I64, I64, I64, T],
        "orc_par_argmax_rows": [P, P, I64, I64, I64, T],
        "orc_par_argcompare_rows": [P, ctypes.c_int, ctypes.c_int, P, I64, I64, I64, T],
        "orc_par_quantize_q4_0": [P, P, I64, I64, T],
        "orc_par_quantize_q8_0": [P, P, I64, I64, T],
        "orc_par_quantize_q8_1": [P, P, I64, I64, T],
        "orc_par_quantize_nf4": [P, P, P, P, I64, I64, I64, T],
    }
    for name, args in par.items():
        getattr(lib, name).argtypes = args
        getattr(lib, name).restype = ctypes.c_int
    return lib


def _call(name, threads, *args):
    """The single-threaded routine `name`, or with threads != 1 the
    row-partitioned driver over it (ctypes releases the GIL during the call)."""
    lib = _load()
    n = _nthreads(threads)
    if n == 1:
        getattr(lib, name)(*args)
        return
    if getattr(lib, name.replace("orc_", "orc_par_", 1))(*args, n) != 0:
        raise MemoryError(f"{name}: the row-partitioned driver could not allocate its scratch")


class use_library:
    """Context manager: route this module's calls to another build of oracle.c
    (the mutation tests load deliberately broken copies this way)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self._saved = _lib
        _lib = _bind(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved
        return False


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


# ---- scalar format helpers -------------------------------------------------

def half_to_double(h: int) -> float:
    return _load().orc_half_to_double(int(h) & 0xFFFF)


def bf16_to_double(b: int) -> float:
    return _load().orc_bf16_to_double(int(b) & 0xFFFF)


def float_to_half_rne(f: float) -> int:
    return int(_load().orc_float_to_half_rne(float(np.float32(f))))


# ---- dense GEMV -------------------------------------------------------------

def gemv_f16(W_bits: np.ndarray, x_bits: np.ndarray, N: int | None = None,
             K: int | None = None, ldw: int | None = None, threads: int = 1) -> np.ndarray:
    """fp64 y = W x over binary16 bit patterns (uint16).  W is [N][ldw]."""
    return _gemv("orc_gemv_f16", W_bits, x_bits, N, K, ldw, threads)


def gemv_bf16(W_bits: np.ndarray, x_bits: np.ndarray, N: int | None = None,
              K: int | None = None, ldw: int | None = None, threads: int = 1) -> np.ndarray:
    """fp64 y = W x over bfloat16 bit patterns (uint16).  W is [N][ldw]."""
    return _gemv("orc_gemv_bf16", W_bits, x_bits, N, K, ldw, threads)


def _gemv(name, W_bits, x_bits, N, K, ldw, threads=1):
    W = _c(W_bits, np.uint16)
    x = _c(x_bits, np.uint16).reshape(-1)
    if W.ndim == 2:
        N = W.shape[0] if N is None else N
        ldw = W.shape[1] if ldw is None else ldw
    K = x.shape[0] if K is None else K
    if ldw is None:
        ldw = K
    assert N is not None and ldw >= K
    if N > 0:
        assert W.size >= (N - 1) * ldw + K
    y = np.zeros(N, dtype=np.float64)
    _call(name, threads, _ptr(W), _ptr(x), _ptr(y), N, K, ldw)
    return y


# ---- Q4_0 x Q8_1 -----------------------------------------------------------

def gemv_q4_0_q8_1(Wq: np.ndarray, Xq: np.ndarray, N: int, K: int, M: int, threads: int = 1) -> np.ndarray:
    """fp64 Y[M][N] from Q4_0 weight bytes and Q8_1 activation bytes."""
    assert K % 32 == 0
    W = _c(Wq, np.uint8).reshape(-1)
    X = _c(Xq, np.uint8).reshape(-1)
    assert W.size >= N * (K // 32) * 18 and X.size >= M * (K // 32) * 36
    Y = np.zeros((M, N), dtype=np.float64)
    _call("orc_gemv_q4_0_q8_1", threads, _ptr(W), _ptr(X), _ptr(Y), N, K, M)
    return Y


def dequant_q4_0_block(blk: bytes | np.ndarray) -> np.ndarray:
    b = _c(np.frombuffer(bytes(blk), dtype=np.uint8) if isinstance(blk, (bytes, bytearray)) else blk, np.uint8)
    assert b.size >= 18
    out = np.zeros(32, dtype=np.float64)
    _load().orc_dequant_q4_0_block(_ptr(b), _ptr(out))
    return out


def dequant_q8_1_block(blk: bytes | np.ndarray) -> np.ndarray:
    b = _c(np.frombuffer(bytes(blk), dtype=np.uint8) if isinstance(blk, (bytes, bytearray)) else blk, np.uint8)
    assert b.size >= 36
    out = np.zeros(32, dtype=np.float64)
    _load().orc_dequant_q8_1_block(_ptr(b), _ptr(out))
    return out


def quantize_q4_0(w: np.ndarray, threads: int = 1) -> np.ndarray:
    """w: float32 [N][K] -> Q4_0 bytes, shape [N, K//32*18]."""
    w = _c(w, np.float32)
    if w.ndim == 1:
        w = w.reshape(1, -1)
    N, K = w.shape
    assert K % 32 == 0
    out = np.zeros((N, K // 32 * 18), dtype=np.uint8)
    _call("orc_quantize_q4_0", threads, _ptr(w), _ptr(out), N, K)
    return out


def quantize_q8_1(x: np.ndarray, threads: int = 1) -> np.ndarray:
    """x: float32 [M][K] -> Q8_1 bytes, shape [M, K//32*36]."""
    x = _c(x, np.float32)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    M, K = x.shape
    assert K % 32 == 0
    out = np.zeros((M, K // 32 * 36), dtype=np.uint8)
    _call("orc_quantize_q8_1", threads, _ptr(x), _ptr(out), M, K)
    return out


# ---- Q8_0 x Q8_1 -----------------------------------------------------------

def gemv_q8_0_q8_1(Wq: np.ndarray, Xq: np.ndarray, N: int, K: int, M: int, threads: int = 1) -> np.ndarray:
    """fp64 Y[M][N] from Q8_0 weight bytes and Q8_1 activation bytes."""
    assert K % 32 == 0
    W = _c(Wq, np.uint8).reshape(-1)
    X = _c(Xq, np.uint8).reshape(-1)
    assert W.size >= N * (K // 32) * 34 and X.size >= M * (K // 32) * 36
    Y = np.zeros((M, N), dtype=np.float64)
    _call("orc_gemv_q8_0_q8_1", threads, _ptr(W), _ptr(X), _ptr(Y), N, K, M)
    return Y


def dequant_q8_0_block(blk: bytes | np.ndarray) -> np.ndarray:
    b = _c(np.frombuffer(bytes(blk), dtype=np.uint8) if isinstance(blk, (bytes, bytearray)) else blk, np.uint8)
    assert b.size >= 34
    out = np.zeros(32, dtype=np.float64)
    _load().orc_dequant_q8_0_block(_ptr(b), _ptr(out))
    return out


def quantize_q8_0(w: np.ndarray, threads: int = 1) -> np.ndarray:
    """w: float32 [N][K] -> Q8_0 bytes, shape [N, K//32*34]."""
    w = _c(w, np.float32)
    if w.ndim == 1:
        w = w.reshape(1, -1)
    N, K = w.shape
    assert K % 32 == 0
    out = np.zeros((N, K // 32 * 34), dtype=np.uint8)
    _call("orc_quantize_q8_0", threads, _ptr(w), _ptr(out), N, K)
    return out


# ---- NF4 ----------------------------------------------------------------------

def gemv_nf4(codes: np.ndarray, absmax: np.ndarray, table: np.ndarray, x_bits: np.ndarray,
             N: int, K: int, B: int, threads: int = 1) -> np.ndarray:
    """fp64 y[N] from NF4 codes (uint8 [N][K/2]), float32 absmax [N][K/B], a
    16-entry float32 table and bfloat16 activation bits x[K]."""
    assert K % B == 0 and K % 2 == 0
    c = _c(codes, np.uint8).reshape(-1)
    a = _c(absmax, np.float32).reshape(-1)
    t = _c(table, np.float32).reshape(-1)
    x = _c(x_bits, np.uint16).reshape(-1)
    assert c.size >= N * K // 2 and a.size >= N * (K // B) and t.size == 16 and x.size >= K
    y = np.zeros(N, dtype=np.float64)
    _call("orc_gemv_nf4", threads, _ptr(c), _ptr(a), _ptr(t), _ptr(x), _ptr(y), N, K, B)
    return y


def quantize_nf4(w: np.ndarray, table: np.ndarray, B: int, threads: int = 1):
    """w: float32 [N][K] -> (codes uint8 [N][K/2], absmax float32 [N][K/B])."""
    w = _c(w, np.float32)
    if w.ndim == 1:
        w = w.reshape(1, -1)
    N, K = w.shape
    assert K % B == 0 and K % 2 == 0
    t = _c(table, np.float32).reshape(-1)
    assert t.size == 16
    codes = np.zeros((N, K // 2), dtype=np.uint8)
    absmax = np.zeros((N, K // B), dtype=np.float32)
    _call("orc_quantize_nf4", threads, _ptr(w), _ptr(codes), _ptr(absmax), _ptr(t), N, K, B)
    return codes, absmax


# ---- argmax and checksum ---------------------------------------------------

def argmax_rows(x: np.ndarray, C: int | None = None, ld: int | None = None, threads: int = 1) -> np.ndarray:
    """int64 index of the first maximum of each row of float32 x ([R][ld])."""
    a = _c(x, np.float32)
    if a.ndim == 1:
        a = a.reshape(1, -1)
    R = a.shape[0]
    ld = a.shape[1] if ld is None else ld
    C = a.shape[1] if C is None else C
    assert C >= 1 and ld >= C
    idx = np.zeros(R, dtype=np.int64)
    _call("orc_argmax_rows", threads, _ptr(a), _ptr(idx), R, C, ld)
    return idx


ARG_DTYPES = {"f32": (0, np.float32), "f16": (1, np.uint16), "bf16": (2, np.uint16)}


def argcompare_rows(x: np.ndarray, dtype: str = "f32", op: str = "max", C: int | None = None,
                    ld: int | None = None, threads: int = 1) -> np.ndarray:
    """int64 index of the first maximum / minimum of each row.  x holds float32
    values ("f32") or binary16 / bfloat16 bit patterns (uint16)."""
    code, npt = ARG_DTYPES[dtype]
    a = _c(x, npt)
    if a.ndim == 1:
        a = a.reshape(1, -1)
    R = a.shape[0]
    ld = a.shape[1] if ld is None else ld
    C = a.shape[1] if C is None else C
    assert C >= 1 and ld >= C
    idx = np.zeros(R, dtype=np.int64)
    _call("orc_argcompare_rows", threads, _ptr(a), code, {"max": 0, "min": 1}[op], _ptr(idx), R, C, ld)
    return idx


def checksum_u32(words: np.ndarray) -> int:
    w = _c(words, np.uint32).reshape(-1)
    return int(_load().orc_checksum_u32(_ptr(w), w.size))
