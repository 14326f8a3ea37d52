"""Python binding of libdecodegemv (argument marshalling only).

Each function has the name of the C entry point it calls (declared in
include/decodegemv.h) and takes torch tensors that live in device memory.  It
checks dtypes and devices, passes raw pointers, sizes and the current HIP
stream to the C ABI, and raises DGError on a non-zero status.  Every step of
the computation runs in the library's HIP kernels; there is no fallback of any
kind: without the built library on a GPU machine, every call raises.

PyTorch is used only for device memory and streams.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdecodegemv.so")

DG_OK = 0
DG_ERR_NULL = 1
DG_ERR_MISALIGNED = 2
DG_ERR_SHAPE = 3
DG_ERR_WORKSPACE = 4
DG_ERR_HIP = 5
DG_ERR_ARG = 6

DG_READ_NONTEMPORAL = 1
DG_READ_GRID_STRIDE = 2
DG_READ_DEEP = 4
DG_READ_SHORT = 8
DG_READ_SHORTER = 16
DG_READ_HALF = 32
DG_READ_CAP_SHIFT = 8


def DG_READ_CAP(n: int) -> int:
    """flags bits: at most n (1..15) workgroups of dg_stream_read resident per CU."""
    return int(n) << DG_READ_CAP_SHIFT
DG_READ_DEFAULT_GRID = 1024

DG_DTYPE_F32 = 0
DG_DTYPE_F16 = 1
DG_DTYPE_BF16 = 2
DG_ARG_MAX = 0
DG_ARG_MIN = 1

DG_VARIANT_DENSE_WIDE = 1
DG_VARIANT_DENSE_XREG = 2
DG_VARIANT_DENSE_NARROW1 = 3
DG_VARIANT_DENSE_NARROW4 = 4
DG_VARIANT_Q4_REGS = 11
DG_VARIANT_Q4_LDS = 12
DG_VARIANT_Q4_LDSROW = 13
DG_VARIANT_Q4_MFMA = 14
DG_VARIANT_Q4_UNITS = 15
DG_VARIANT_Q4_MFMA_RES = 16
DG_VARIANT_Q8_LDSROW = 21
DG_VARIANT_Q8_MFMA = 22
DG_VARIANT_Q8_UNITS = 23
DG_VARIANT_Q8_MFMA_RES = 24
DG_VARIANT_NF4_UNITS = 31
DG_VARIANT_NF4_MFMA = 32
DG_VARIANT_NF4_ROWS = 33

# Every symbol include/decodegemv.h declares.
EXPORTED = (
    "dg_status_string", "dg_last_hip_error", "dg_stream_read",
    "dg_gemv_f16", "dg_gemv_bf16", "dg_gemv_q4_0",
    "dg_quantize_q8_1", "dg_quantize_q4_0",
    "dg_argmax_workspace_bytes", "dg_argmax_rows",
    "dg_gemv_f16_ex", "dg_gemv_bf16_ex", "dg_gemv_q4_0_ex",
    "dg_gemv_q8_0", "dg_gemv_q8_0_ex", "dg_quantize_q8_0",
    "dg_argcompare_rows", "dg_gemv_bf16_argmax_workspace_bytes", "dg_gemv_bf16_argmax",
    "dg_gemv_nf4", "dg_gemv_nf4_ex", "dg_quantize_nf4",
    "dg_argmax_rows_noalloc", "dg_gemv_q4_0_f32", "dg_gemv_q4_0_f32_ex",
    "dg_q4_0_tiles_bytes", "dg_repack_q4_0_tiles", "dg_gemv_q4_0_tiles_workspace_bytes",
    "dg_gemv_q4_0_tiles", "dg_gemv_q4_0_tiles_ex",
    "dg_q8_0_tiles_bytes", "dg_repack_q8_0_tiles", "dg_gemv_q8_0_tiles_workspace_bytes",
    "dg_gemv_q8_0_tiles", "dg_gemv_q8_0_tiles_ex",
)

# Size of the library's fixed per-device argmax key array (include/decodegemv.h).
DG_ARGMAX_SCRATCH_BYTES = 1 << 20


class DGError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib().dg_status_string(status).decode()
        if status == DG_ERR_HIP:
            msg += " (" + _lib().dg_last_hip_error().decode() + ")"
        super().__init__(f"{where}: {msg}")


class dg_launch(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int), ("grid", ctypes.c_int),
                ("block", ctypes.c_int), ("unroll", ctypes.c_int)]


_handle = None


def _hip_runtimes_mapped():
    """Paths of every HIP runtime (libamdhip64) mapped into this process."""
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


def _lib():
    global _handle
    if _handle is not None:
        return _handle
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    # torch ships its own HIP runtime (same soname, libamdhip64.so.7).  Importing
    # torch first makes libdecodegemv bind to that one runtime; loaded the other
    # way round, the process would hold two runtimes that share neither streams
    # nor graphs.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError(f"two HIP runtimes are mapped into this process: {sorted(runtimes)}")
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    st = ctypes.c_int
    lib.dg_status_string.argtypes = [st]
    lib.dg_status_string.restype = ctypes.c_char_p
    lib.dg_last_hip_error.argtypes = []
    lib.dg_last_hip_error.restype = ctypes.c_char_p
    lib.dg_stream_read.argtypes = [P, ctypes.c_size_t, P, I32, I32, I32, P]
    lib.dg_stream_read.restype = st
    for n in ("dg_gemv_f16", "dg_gemv_bf16"):
        getattr(lib, n).argtypes = [P, P, P, I64, I64, I64, P]
        getattr(lib, n).restype = st
        getattr(lib, n + "_ex").argtypes = [P, P, P, I64, I64, I64, ctypes.POINTER(dg_launch), P]
        getattr(lib, n + "_ex").restype = st
    for n in ("dg_gemv_q4_0", "dg_gemv_q8_0"):
        getattr(lib, n).argtypes = [P, P, P, I64, I64, I32, P]
        getattr(lib, n).restype = st
        getattr(lib, n + "_ex").argtypes = [P, P, P, I64, I64, I32, ctypes.POINTER(dg_launch), P]
        getattr(lib, n + "_ex").restype = st
    lib.dg_quantize_q8_1.argtypes = [P, P, I64, I64, P]
    lib.dg_quantize_q8_1.restype = st
    for n in ("dg_quantize_q4_0", "dg_quantize_q8_0"):
        getattr(lib, n).argtypes = [P, P, I64, I64, P]
        getattr(lib, n).restype = st
    lib.dg_argmax_workspace_bytes.argtypes = [I64, I64]
    lib.dg_argmax_workspace_bytes.restype = ctypes.c_size_t
    lib.dg_argmax_rows.argtypes = [P, P, I64, I64, I64, P, ctypes.c_size_t, P]
    lib.dg_argmax_rows.restype = st
    lib.dg_argmax_rows_noalloc.argtypes = [P, P, I64, I64, I64, P]
    lib.dg_argmax_rows_noalloc.restype = st
    lib.dg_gemv_q4_0_f32.argtypes = [P, P, P, P, I64, I64, I32, P]
    lib.dg_gemv_q4_0_f32.restype = st
    lib.dg_gemv_q4_0_f32_ex.argtypes = [P, P, P, P, I64, I64, I32, P, P]
    lib.dg_gemv_q4_0_f32_ex.restype = st
    lib.dg_argcompare_rows.argtypes = [P, I32, I32, P, I64, I64, I64, P, ctypes.c_size_t, P]
    lib.dg_argcompare_rows.restype = st
    lib.dg_gemv_bf16_argmax_workspace_bytes.argtypes = [I64, I64]
    lib.dg_gemv_bf16_argmax_workspace_bytes.restype = ctypes.c_size_t
    lib.dg_gemv_bf16_argmax.argtypes = [P, P, P, P, I64, I64, I64, P, ctypes.c_size_t, P]
    lib.dg_gemv_bf16_argmax.restype = st
    lib.dg_gemv_nf4.argtypes = [P, P, P, P, P, I64, I64, I32, P]
    lib.dg_gemv_nf4.restype = st
    lib.dg_gemv_nf4_ex.argtypes = [P, P, P, P, P, I64, I64, I32, ctypes.POINTER(dg_launch), P]
    lib.dg_gemv_nf4_ex.restype = st
    lib.dg_quantize_nf4.argtypes = [P, P, P, P, I64, I64, I32, P]
    lib.dg_quantize_nf4.restype = st
    for f in ("q4_0", "q8_0"):
        getattr(lib, f"dg_{f}_tiles_bytes").argtypes = [I64, I64]
        getattr(lib, f"dg_{f}_tiles_bytes").restype = ctypes.c_size_t
        getattr(lib, f"dg_repack_{f}_tiles").argtypes = [P, P, I64, I64, P]
        getattr(lib, f"dg_repack_{f}_tiles").restype = st
        getattr(lib, f"dg_gemv_{f}_tiles_workspace_bytes").argtypes = [I64, I64, I32]
        getattr(lib, f"dg_gemv_{f}_tiles_workspace_bytes").restype = ctypes.c_size_t
        getattr(lib, f"dg_gemv_{f}_tiles").argtypes = [P, P, P, I64, I64, I32, P, ctypes.c_size_t, P]
        getattr(lib, f"dg_gemv_{f}_tiles").restype = st
        getattr(lib, f"dg_gemv_{f}_tiles_ex").argtypes = [P, P, P, I64, I64, I32, P, ctypes.c_size_t,
                                                          ctypes.POINTER(dg_launch), P]
        getattr(lib, f"dg_gemv_{f}_tiles_ex").restype = st
    _handle = lib
    return lib


def raw():
    """The ctypes handle of libdecodegemv.so (for tests that call the C ABI directly)."""
    return _lib()


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, dtypes, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _fits(t, nbytes, name):
    """Raises unless tensor t spans at least nbytes (the extent the call reads or writes)."""
    have = t.numel() * t.element_size()
    if nbytes > have:
        raise ValueError(f"{name} holds {have} bytes but the call touches {nbytes}")


def _check(status, where):
    if status != DG_OK:
        raise DGError(status, where)


def _cfg(variant=0, grid=0, block=0, unroll=0):
    return dg_launch(variant, grid, block, unroll)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def dg_stream_read(buf, partials, nbytes=None, grid_blocks=0, block_threads=0,
                   flags=DG_READ_NONTEMPORAL, stream=None):
    """Reads every byte of buf once; workgroup b stores the wrapping uint32 sum
    of the words it read into partials[b] (int32 [G], G = grid_blocks or
    DG_READ_DEFAULT_GRID).  The buffer's word sum is the wrapping sum of the
    G partials."""
    torch = _torch()
    _need(partials, (torch.int32,), "partials")
    if not buf.is_cuda:
        raise ValueError("buf must be a device tensor")
    nbytes = buf.numel() * buf.element_size() if nbytes is None else int(nbytes)
    _fits(buf, nbytes, "buf")
    grid = int(grid_blocks) if grid_blocks else DG_READ_DEFAULT_GRID
    if grid > 0 and nbytes > 0:
        _fits(partials, grid * 4, "partials")
    _check(_lib().dg_stream_read(_ptr(buf), nbytes, _ptr(partials), int(grid_blocks),
                                 int(block_threads), int(flags), _stream(stream)),
           "dg_stream_read")


def _dense(name, W, x, y, N, K, ldw, launch, stream, wdtype, ydtype):
    _need(W, (wdtype,), "W")
    _need(x, (wdtype,), "x")
    _need(y, (ydtype,), "y")
    if N is None:
        N = W.shape[0]
    if K is None:
        K = x.numel()
    if ldw is None:
        ldw = W.shape[1] if W.dim() == 2 else K
    N, K, ldw = int(N), int(K), int(ldw)
    if N > 0 and K > 0 and 0 <= K <= ldw:
        _fits(W, ((N - 1) * ldw + K) * 2, "W")
        _fits(x, K * 2, "x")
    _fits(y, max(N, 0) * y.element_size(), "y")
    lib = _lib()
    if launch is None:
        st = getattr(lib, name)(_ptr(W), _ptr(x), _ptr(y), N, K, ldw, _stream(stream))
    else:
        st = getattr(lib, name + "_ex")(_ptr(W), _ptr(x), _ptr(y), N, K, ldw,
                                        ctypes.byref(_cfg(**launch)), _stream(stream))
    _check(st, name)
    return y


def dg_gemv_f16(W, x, y, N=None, K=None, ldw=None, launch=None, stream=None):
    """y[N] (float16) = W[N][ldw] (float16) . x[K] (float16), fp32 accumulation."""
    torch = _torch()
    return _dense("dg_gemv_f16", W, x, y, N, K, ldw, launch, stream, torch.float16, torch.float16)


def dg_gemv_bf16(W, x, y, N=None, K=None, ldw=None, launch=None, stream=None):
    """y[N] (float32) = W[N][ldw] (bfloat16) . x[K] (bfloat16), fp32 accumulation."""
    torch = _torch()
    return _dense("dg_gemv_bf16", W, x, y, N, K, ldw, launch, stream, torch.bfloat16, torch.float32)


def _gemv_quant(name, block_bytes, Wq, Xq, Y, N, K, M, launch, stream):
    torch = _torch()
    _need(Wq, (torch.uint8,), "Wq")
    _need(Xq, (torch.uint8,), "Xq")
    _need(Y, (torch.float32,), "Y")
    N, K, M = int(N), int(K), int(M)
    if N > 0 and K > 0 and M > 0:
        _fits(Wq, N * (K // 32) * block_bytes, "Wq")
        _fits(Xq, M * (K // 32) * 36, "Xq")
    if N > 0 and M > 0:
        _fits(Y, M * N * 4, "Y")
    lib = _lib()
    if launch is None:
        st = getattr(lib, name)(_ptr(Wq), _ptr(Xq), _ptr(Y), N, K, M, _stream(stream))
    else:
        st = getattr(lib, name + "_ex")(_ptr(Wq), _ptr(Xq), _ptr(Y), N, K, M, ctypes.byref(_cfg(**launch)),
                                        _stream(stream))
    _check(st, name)
    return Y


def dg_gemv_q4_0(Wq, Xq, Y, N, K, M, launch=None, stream=None):
    """Y[M][N] (float32) from Q4_0 weight bytes and Q8_1 activation bytes (uint8 tensors)."""
    return _gemv_quant("dg_gemv_q4_0", 18, Wq, Xq, Y, N, K, M, launch, stream)


def dg_gemv_q4_0_f32(Wq, x, Y, N, K, M, Xq=None, launch=None, stream=None):
    """Y[M][N] (float32) from Q4_0 weight bytes and float32 activations x[M][K]:
    the Q8_1 quantisation and the GEMV in one call (two launches; the
    one-launch form for M = 1 is launch=dict(variant=DG_VARIANT_Q4_LDSROW)).
    Xq (uint8, M*K/32*36 bytes) receives the quantised columns; required
    except by the one-launch form."""
    torch = _torch()
    _need(Wq, (torch.uint8,), "Wq")
    _need(x, (torch.float32,), "x")
    _need(Y, (torch.float32,), "Y")
    N, K, M = int(N), int(K), int(M)
    if Xq is not None:
        _need(Xq, (torch.uint8,), "Xq")
    if N > 0 and K > 0 and M > 0:
        _fits(Wq, N * (K // 32) * 18, "Wq")
        _fits(x, M * K * 4, "x")
        if Xq is not None:
            _fits(Xq, M * (K // 32) * 36, "Xq")
    if N > 0 and M > 0:
        _fits(Y, M * N * 4, "Y")
    xq = _ptr(Xq) if Xq is not None else None
    if launch is None:
        st = _lib().dg_gemv_q4_0_f32(_ptr(Wq), _ptr(x), _ptr(Y), xq, N, K, M, _stream(stream))
    else:
        st = _lib().dg_gemv_q4_0_f32_ex(_ptr(Wq), _ptr(x), _ptr(Y), xq, N, K, M, ctypes.byref(_cfg(**launch)),
                                        _stream(stream))
    _check(st, "dg_gemv_q4_0_f32")
    return Y


def _tiles_fmt(fmt):
    if fmt not in ("q4_0", "q8_0"):
        raise ValueError(f"tiled format must be q4_0 or q8_0, not {fmt!r}")
    return fmt, (18 if fmt == "q4_0" else 34)


def dg_q4_0_tiles_bytes(N, K):
    """Bytes of the 16-row-tile copy of an N x K Q4_0 matrix (0 for an invalid shape)."""
    return int(_lib().dg_q4_0_tiles_bytes(int(N), int(K)))


def dg_q8_0_tiles_bytes(N, K):
    """Bytes of the 16-row-tile copy of an N x K Q8_0 matrix (0 for an invalid shape)."""
    return int(_lib().dg_q8_0_tiles_bytes(int(N), int(K)))


def _repack_tiles(fmt, Wq, Wt, N, K, stream):
    torch = _torch()
    fmt, block_bytes = _tiles_fmt(fmt)
    _need(Wq, (torch.uint8,), "Wq")
    _need(Wt, (torch.uint8,), "Wt")
    N, K = int(N), int(K)
    if N > 0 and K > 0:
        _fits(Wq, N * (K // 32) * block_bytes, "Wq")
        _fits(Wt, int(getattr(_lib(), f"dg_{fmt}_tiles_bytes")(N, K)), "Wt")
    name = f"dg_repack_{fmt}_tiles"
    _check(getattr(_lib(), name)(_ptr(Wq), _ptr(Wt), N, K, _stream(stream)), name)
    return Wt


def dg_repack_q4_0_tiles(Wq, Wt, N, K, stream=None):
    """Wt (uint8, dg_q4_0_tiles_bytes(N, K)) = the row-major Q4_0 bytes Wq rearranged into 16-row tiles."""
    return _repack_tiles("q4_0", Wq, Wt, N, K, stream)


def dg_repack_q8_0_tiles(Wq, Wt, N, K, stream=None):
    """Wt (uint8, dg_q8_0_tiles_bytes(N, K)) = the row-major Q8_0 bytes Wq rearranged into 16-row tiles."""
    return _repack_tiles("q8_0", Wq, Wt, N, K, stream)


def dg_gemv_q4_0_tiles_workspace_bytes(N, K, M):
    return int(_lib().dg_gemv_q4_0_tiles_workspace_bytes(int(N), int(K), int(M)))


def dg_gemv_q8_0_tiles_workspace_bytes(N, K, M):
    return int(_lib().dg_gemv_q8_0_tiles_workspace_bytes(int(N), int(K), int(M)))


def _gemv_tiles(fmt, Wt, Xq, Y, N, K, M, ws, launch, stream):
    torch = _torch()
    fmt, _ = _tiles_fmt(fmt)
    _need(Wt, (torch.uint8,), "Wt")
    _need(Xq, (torch.uint8,), "Xq")
    _need(Y, (torch.float32,), "Y")
    N, K, M = int(N), int(K), int(M)
    lib = _lib()
    if N > 0 and K > 0 and M > 0:
        _fits(Wt, int(getattr(lib, f"dg_{fmt}_tiles_bytes")(N, K)), "Wt")
        _fits(Xq, M * (K // 32) * 36, "Xq")
    if N > 0 and M > 0:
        _fits(Y, M * N * 4, "Y")
    if ws is not None:
        _need(ws, (torch.uint8,), "ws")
    wsp, wsb = (_ptr(ws), ws.numel()) if ws is not None else (None, 0)
    name = f"dg_gemv_{fmt}_tiles"
    if launch is None:
        st = getattr(lib, name)(_ptr(Wt), _ptr(Xq), _ptr(Y), N, K, M, wsp, wsb, _stream(stream))
    else:
        st = getattr(lib, name + "_ex")(_ptr(Wt), _ptr(Xq), _ptr(Y), N, K, M, wsp, wsb,
                                        ctypes.byref(_cfg(**launch)), _stream(stream))
    _check(st, name)
    return Y


def dg_gemv_q4_0_tiles(Wt, Xq, Y, N, K, M, ws=None, launch=None, stream=None):
    """Y[M][N] (float32) from the tiled Q4_0 copy Wt and Q8_1 activation bytes.
    ws: a uint8 device tensor, zero-filled once when allocated (its ticket
    counters must start at zero; every call leaves them zero), of at least
    dg_gemv_q4_0_tiles_workspace_bytes(N, K, M) bytes for the default launch;
    None is allowed when that is 0."""
    return _gemv_tiles("q4_0", Wt, Xq, Y, N, K, M, ws, launch, stream)


def dg_gemv_q8_0_tiles(Wt, Xq, Y, N, K, M, ws=None, launch=None, stream=None):
    """Y[M][N] (float32) from the tiled Q8_0 copy Wt and Q8_1 activation bytes
    (workspace as for dg_gemv_q4_0_tiles)."""
    return _gemv_tiles("q8_0", Wt, Xq, Y, N, K, M, ws, launch, stream)


def dg_gemv_q8_0(Wq, Xq, Y, N, K, M, launch=None, stream=None):
    """Y[M][N] (float32) from Q8_0 weight bytes and Q8_1 activation bytes (uint8 tensors)."""
    return _gemv_quant("dg_gemv_q8_0", 34, Wq, Xq, Y, N, K, M, launch, stream)


def dg_gemv_nf4(codes, absmax, table, x, y, N=None, K=None, B=64, launch=None, stream=None):
    """y[N] (float32) from NF4 codes (uint8 [N*K/2]), float32 absmax [N*K/B],
    a float32 table [16] and bfloat16 activations x [K]."""
    torch = _torch()
    _need(codes, (torch.uint8,), "codes")
    _need(absmax, (torch.float32,), "absmax")
    _need(table, (torch.float32,), "table")
    _need(x, (torch.bfloat16,), "x")
    _need(y, (torch.float32,), "y")
    K = x.numel() if K is None else int(K)
    N = y.numel() if N is None else int(N)
    B = int(B)
    if N > 0 and K > 0 and B > 0:
        _fits(codes, N * K // 2, "codes")
        _fits(absmax, N * (K // B) * 4, "absmax")
        _fits(table, 64, "table")
        _fits(x, K * 2, "x")
    if N > 0:
        _fits(y, N * 4, "y")
    lib = _lib()
    args = (_ptr(codes), _ptr(absmax), _ptr(table), _ptr(x), _ptr(y), N, K, B)
    if launch is None:
        st = lib.dg_gemv_nf4(*args, _stream(stream))
    else:
        st = lib.dg_gemv_nf4_ex(*args, ctypes.byref(_cfg(**launch)), _stream(stream))
    _check(st, "dg_gemv_nf4")
    return y


def dg_quantize_nf4(w, codes, absmax, table, N, K, B=64, stream=None):
    """float32 [N][K] -> NF4 codes (uint8 [N*K/2]) and float32 absmax [N*K/B]."""
    torch = _torch()
    _need(w, (torch.float32,), "w")
    _need(codes, (torch.uint8,), "codes")
    _need(absmax, (torch.float32,), "absmax")
    _need(table, (torch.float32,), "table")
    N, K, B = int(N), int(K), int(B)
    if N > 0 and K > 0 and B > 0:
        _fits(w, N * K * 4, "w")
        _fits(codes, N * K // 2, "codes")
        _fits(absmax, N * (K // B) * 4, "absmax")
        _fits(table, 64, "table")
    _check(_lib().dg_quantize_nf4(_ptr(w), _ptr(codes), _ptr(absmax), _ptr(table), N, K, B, _stream(stream)),
           "dg_quantize_nf4")
    return codes, absmax


def dg_quantize_q8_1(x, Xq, M, K, stream=None):
    """float32 [M][K] -> Q8_1 bytes (uint8 [M*K/32*36])."""
    torch = _torch()
    _need(x, (torch.float32,), "x")
    _need(Xq, (torch.uint8,), "Xq")
    if M > 0 and K > 0:
        _fits(x, int(M) * int(K) * 4, "x")
        _fits(Xq, int(M) * (int(K) // 32) * 36, "Xq")
    _check(_lib().dg_quantize_q8_1(_ptr(x), _ptr(Xq), int(M), int(K), _stream(stream)), "dg_quantize_q8_1")
    return Xq


def dg_quantize_q4_0(w, Wq, N, K, stream=None):
    """float32 [N][K] -> Q4_0 bytes (uint8 [N*K/32*18])."""
    torch = _torch()
    _need(w, (torch.float32,), "w")
    _need(Wq, (torch.uint8,), "Wq")
    if N > 0 and K > 0:
        _fits(w, int(N) * int(K) * 4, "w")
        _fits(Wq, int(N) * (int(K) // 32) * 18, "Wq")
    _check(_lib().dg_quantize_q4_0(_ptr(w), _ptr(Wq), int(N), int(K), _stream(stream)), "dg_quantize_q4_0")
    return Wq


def dg_quantize_q8_0(w, Wq, N, K, stream=None):
    """float32 [N][K] -> Q8_0 bytes (uint8 [N*K/32*34])."""
    torch = _torch()
    _need(w, (torch.float32,), "w")
    _need(Wq, (torch.uint8,), "Wq")
    if N > 0 and K > 0:
        _fits(w, int(N) * int(K) * 4, "w")
        _fits(Wq, int(N) * (int(K) // 32) * 34, "Wq")
    _check(_lib().dg_quantize_q8_0(_ptr(w), _ptr(Wq), int(N), int(K), _stream(stream)), "dg_quantize_q8_0")
    return Wq


def dg_argmax_workspace_bytes(R, C):
    return int(_lib().dg_argmax_workspace_bytes(int(R), int(C)))


def dg_argmax_rows(x, idx, R=None, C=None, ld=None, ws=None, stream=None):
    """idx[R] (int64) = lowest index of each row's maximum of x (float32 [R][ld])."""
    torch = _torch()
    _need(x, (torch.float32,), "x")
    _need(idx, (torch.int64,), "idx")
    if R is None:
        R = x.shape[0] if x.dim() == 2 else 1
    if C is None:
        C = x.shape[-1]
    if ld is None:
        ld = x.shape[-1]
    R, C, ld = int(R), int(C), int(ld)
    if R > 0 and C > 0 and ld >= C:
        _fits(x, ((R - 1) * ld + C) * 4, "x")
        _fits(idx, R * 8, "idx")
    need = dg_argmax_workspace_bytes(R, C)
    if ws is None:
        raise ValueError(f"dg_argmax_rows needs a device workspace of {need} bytes")
    _need(ws, (torch.uint8, torch.int64), "ws")
    ws_bytes = ws.numel() * ws.element_size()
    _check(_lib().dg_argmax_rows(_ptr(x), _ptr(idx), int(R), int(C), int(ld), _ptr(ws), ws_bytes,
                                 _stream(stream)), "dg_argmax_rows")
    return idx


def dg_argmax_rows_noalloc(x, idx, R=None, C=None, ld=None, stream=None):
    """As dg_argmax_rows, with the chunk keys in the library's fixed per-device
    array instead of a workspace: the call allocates nothing.  Calls that
    overlap on one GPU race (they share the array)."""
    torch = _torch()
    _need(x, (torch.float32,), "x")
    _need(idx, (torch.int64,), "idx")
    if R is None:
        R = x.shape[0] if x.dim() == 2 else 1
    if C is None:
        C = x.shape[-1]
    if ld is None:
        ld = x.shape[-1]
    R, C, ld = int(R), int(C), int(ld)
    if R > 0 and C > 0 and ld >= C:
        _fits(x, ((R - 1) * ld + C) * 4, "x")
        _fits(idx, R * 8, "idx")
    _check(_lib().dg_argmax_rows_noalloc(_ptr(x), _ptr(idx), R, C, ld, _stream(stream)), "dg_argmax_rows_noalloc")
    return idx


def dg_argcompare_rows(x, idx, op="max", R=None, C=None, ld=None, ws=None, stream=None):
    """idx[R] (int64) = lowest index of each row's maximum (op "max") or minimum
    (op "min") of x (float32, float16 or bfloat16 [R][ld]); a NaN wins for both.
    ws: a device workspace of dg_argmax_workspace_bytes(R, C) bytes."""
    torch = _torch()
    _need(x, (torch.float32, torch.float16, torch.bfloat16), "x")
    _need(idx, (torch.int64,), "idx")
    dtype = {torch.float32: DG_DTYPE_F32, torch.float16: DG_DTYPE_F16, torch.bfloat16: DG_DTYPE_BF16}[x.dtype]
    if R is None:
        R = x.shape[0] if x.dim() == 2 else 1
    if C is None:
        C = x.shape[-1]
    if ld is None:
        ld = x.shape[-1]
    R, C, ld = int(R), int(C), int(ld)
    if R > 0 and C > 0 and ld >= C:
        _fits(x, ((R - 1) * ld + C) * x.element_size(), "x")
        _fits(idx, R * 8, "idx")
    need = dg_argmax_workspace_bytes(R, C)
    if ws is None:
        raise ValueError(f"dg_argcompare_rows needs a device workspace of {need} bytes")
    _need(ws, (torch.uint8, torch.int64), "ws")
    ws_bytes = ws.numel() * ws.element_size()
    _check(_lib().dg_argcompare_rows(_ptr(x), dtype, {"max": DG_ARG_MAX, "min": DG_ARG_MIN}[op], _ptr(idx),
                                     R, C, ld, _ptr(ws), ws_bytes, _stream(stream)), "dg_argcompare_rows")
    return idx


def dg_gemv_bf16_argmax_workspace_bytes(N, K):
    return int(_lib().dg_gemv_bf16_argmax_workspace_bytes(int(N), int(K)))


def dg_gemv_bf16_argmax(W, x, idx, y=None, N=None, K=None, ldw=None, ws=None, stream=None):
    """The fused greedy tail: idx[0] (int64) = argmax over n of y[n] = W[n] . x
    (bfloat16 operands, fp32 logits stored in y unless y is None)."""
    torch = _torch()
    _need(W, (torch.bfloat16,), "W")
    _need(x, (torch.bfloat16,), "x")
    _need(idx, (torch.int64,), "idx")
    if y is not None:
        _need(y, (torch.float32,), "y")
    if N is None:
        N = W.shape[0]
    if K is None:
        K = x.numel()
    if ldw is None:
        ldw = W.shape[1] if W.dim() == 2 else K
    N, K, ldw = int(N), int(K), int(ldw)
    if N > 0 and K > 0 and 0 <= K <= ldw:
        _fits(W, ((N - 1) * ldw + K) * 2, "W")
        _fits(x, K * 2, "x")
    if y is not None:
        _fits(y, max(N, 0) * 4, "y")
    _fits(idx, 8, "idx")
    if ws is None:
        raise ValueError(f"dg_gemv_bf16_argmax needs a device workspace of "
                         f"{dg_gemv_bf16_argmax_workspace_bytes(N, K)} bytes")
    _need(ws, (torch.uint8, torch.int64), "ws")
    _check(_lib().dg_gemv_bf16_argmax(_ptr(W), _ptr(x), _ptr(y), _ptr(idx), N, K, ldw, _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)), "dg_gemv_bf16_argmax")
    return idx
