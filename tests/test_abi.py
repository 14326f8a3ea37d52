"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, and rejects invalid arguments before touching the HIP runtime
(no compute is launched here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "decodegemv.h")


@pytest.fixture(scope="module")
def lib():
    import memory_bound_decode_gemv_amd as m
    if not os.path.exists(m.LIB_PATH):
        from memory_bound_decode_gemv_amd import _build
        _build.build()
    return m.raw()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 13
    import memory_bound_decode_gemv_amd as m
    assert sorted(m.EXPORTED) == names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(7):
        assert lib.dg_status_string(s).startswith(b"DG_")


P = ctypes.c_void_p
A16 = P(0x1000)       # a 16-byte-aligned fake device address (never dereferenced)
A2 = P(0x1002)


@pytest.mark.parametrize("args,expect", [
    ((A16, A16, A16, 4, 12, 16), 3),      # K % 8
    ((A16, A16, A16, 4, 16, 8), 3),       # ldw < K
    ((A16, A16, A16, 4, 16, 20), 3),      # ldw % 8
    ((A16, A16, A16, -1, 16, 16), 3),     # N < 0
    ((A16, A16, A16, 1 << 31, 16, 16), 3),
    ((None, A16, A16, 4, 16, 16), 1),     # NULL W
    ((A16, A16, None, 4, 16, 16), 1),     # NULL y
    ((A2, A16, A16, 4, 16, 16), 2),       # W misaligned
    ((A16, A2, A16, 4, 16, 16), 2),       # x misaligned
    ((A16, A16, P(0x1001), 4, 16, 16), 2),  # y misaligned
    ((None, None, None, 0, 16, 16), 0),   # empty: nothing launched
])
def test_gemv_f16_rejects_before_launch(lib, args, expect):
    assert lib.dg_gemv_f16(*args, None) == expect
    if expect != 2 or args[2] != P(0x1001):
        assert lib.dg_gemv_bf16(*args, None) == expect


@pytest.mark.parametrize("args,expect", [
    ((A16, A16, A16, 4, 100, 1), 3),      # K % 256
    ((A16, A16, A16, 4, 256, 25), 3),     # M > 24
    ((A16, A16, A16, 4, (1 << 26) + 256, 1), 3),   # K > 2^26
    ((A16, A16, A16, 4, 256, -1), 3),
    ((None, A16, A16, 4, 256, 1), 1),
    ((A16, None, A16, 4, 256, 1), 1),
    ((A2, A16, A16, 4, 256, 1), 2),       # Wq must be 16-byte aligned
    ((A16, A16, A2, 4, 256, 1), 2),       # Y must be 4-byte aligned
    ((A16, P(0x1004), A16, 4, 256, 1), 2),  # Xq must be 16-byte aligned
    ((None, None, None, 4, 256, 0), 0),   # M = 0
    ((None, None, None, 0, 256, 3), 0),   # N = 0
])
def test_gemv_q4_0_rejects_before_launch(lib, args, expect):
    assert lib.dg_gemv_q4_0(*args, None) == expect
    assert lib.dg_gemv_q8_0(*args, None) == expect


def test_launch_overrides_rejected(lib):
    import memory_bound_decode_gemv_amd as m
    bad = [m.dg_launch(-1, 0, 0, 0), m.dg_launch(0, 0, 100, 0), m.dg_launch(0, 0, 2048, 0)]
    for cfg in bad:
        assert lib.dg_gemv_f16_ex(A16, A16, A16, 4, 16, 16, ctypes.byref(cfg), None) == 6
        assert lib.dg_gemv_q4_0_ex(A16, A16, A16, 4, 256, 1, ctypes.byref(cfg), None) == 6
        assert lib.dg_gemv_q8_0_ex(A16, A16, A16, 4, 256, 1, ctypes.byref(cfg), None) == 6


def test_units_kernel_rejects_too_many_columns(lib):
    """The units kernels hold M * ceil(K / 4096) <= 8 activation pairs per lane."""
    import memory_bound_decode_gemv_amd as m
    cfg = m.dg_launch(15, 0, 0, 0)
    assert lib.dg_gemv_q4_0_ex(A16, A16, A16, 4, 8192, 5, ctypes.byref(cfg), None) == 6
    assert lib.dg_gemv_q4_0_ex(A16, A16, A16, 4, 4096, 9, ctypes.byref(cfg), None) == 6
    cfg = m.dg_launch(23, 0, 0, 0)
    assert lib.dg_gemv_q8_0_ex(A16, A16, A16, 4, 16384, 3, ctypes.byref(cfg), None) == 6
    assert lib.dg_gemv_q8_0_ex(A16, A16, A16, 4, 20480, 1, ctypes.byref(cfg), None) == 6   # rows over 4 units


def test_stream_read_rejects_before_launch(lib):
    assert lib.dg_stream_read(A16, 24, A16, 0, 0, 1, None) == 3          # bytes % 16
    assert lib.dg_stream_read(A16, 32, A16, 0, 96, 1, None) == 6         # block not a multiple of 64
    assert lib.dg_stream_read(A16, 32, A16, 0, 0, 64, None) == 6         # unknown flag
    assert lib.dg_stream_read(A16, 32, A16, 0, 0, 4 | 8, None) == 6      # two chunk depths
    assert lib.dg_stream_read(A16, 32, A16, 0, 0, 8 | 16, None) == 6
    assert lib.dg_stream_read(A16, 32, A16, 0, 0, 2 | 16, None) == 6     # a depth with the grid-stride order
    assert lib.dg_stream_read(A16, 32, A16, 0, 64, 32, None) == 6        # half the waves of a 1-wave group
    assert lib.dg_stream_read(A16, 32, A16, 0, 192, 32, None) == 6       # ... of an odd wave count
    assert lib.dg_stream_read(A16, 32, A16, 0, 0, 2 | 32, None) == 6     # half with the grid-stride order
    assert lib.dg_stream_read(A16, 32, A16, 0, 0, 1 << 12, None) == 6    # past the cap field
    assert lib.dg_stream_read(None, 32, A16, 0, 0, 1, None) == 1
    assert lib.dg_stream_read(A2, 32, A16, 0, 0, 1, None) == 2
    assert lib.dg_stream_read(A16, 32, A2, 0, 0, 1, None) == 2          # partials not 4-byte aligned
    assert lib.dg_stream_read(A16, 32, None, 0, 0, 1, None) == 1
    assert lib.dg_stream_read(None, 0, None, 0, 0, 1, None) == 0         # empty


def test_argmax_rejects_before_launch(lib):
    need = lib.dg_argmax_workspace_bytes(64, 1000000)
    assert need == 64 * 62 * 8
    assert lib.dg_argmax_workspace_bytes(0, 10) == 0
    assert lib.dg_argmax_rows(A16, A16, 4, 0, 4, A16, 1 << 20, None) == 3    # C = 0
    assert lib.dg_argmax_rows(A16, A16, 4, 10, 9, A16, 1 << 20, None) == 3   # ld < C
    assert lib.dg_argmax_rows(A16, A16, 64, 1000000, 1000000, A16, need - 1, None) == 4
    assert lib.dg_argmax_rows(A16, A16, 64, 1000000, 1000000, None, need, None) == 4
    assert lib.dg_argmax_rows(None, A16, 4, 10, 10, A16, 1 << 20, None) == 1
    assert lib.dg_argmax_rows(A16, P(0x1004), 4, 10, 10, A16, 1 << 20, None) == 2
    assert lib.dg_argmax_rows(None, None, 0, 10, 10, None, 0, None) == 0


def test_argmax_noalloc_rejects_before_launch(lib):
    """The no-allocation argmax checks its arguments, and that the chunk keys fit
    the library's fixed array, before touching the HIP runtime."""
    import memory_bound_decode_gemv_amd as m
    f = lib.dg_argmax_rows_noalloc
    assert f(A16, A16, 4, 0, 4, None) == 3                     # C = 0
    assert f(A16, A16, 4, 10, 9, None) == 3                    # ld < C
    assert f(None, A16, 4, 10, 10, None) == 1
    assert f(A16, P(0x1004), 4, 10, 10, None) == 2
    assert f(None, None, 0, 10, 10, None) == 0                 # empty: nothing launched
    # the largest row count whose keys still fit, and one more row
    C = 1 << 20
    rmax = noalloc_max_rows(lib, C, m.DG_ARGMAX_SCRATCH_BYTES)
    assert rmax >= 64        # the [64, 1M] workload fits
    assert lib.dg_argmax_workspace_bytes(rmax + 1, C) > m.DG_ARGMAX_SCRATCH_BYTES
    assert f(A16, A16, rmax + 1, C, C, None) == 4


def noalloc_max_rows(lib, C, limit):
    """The largest R with dg_argmax_workspace_bytes(R, C) <= limit (the key
    count per row depends on R through the chunk choice, so search)."""
    lo, hi = 0, 1
    while lib.dg_argmax_workspace_bytes(hi, C) <= limit:
        lo, hi = hi, 2 * hi
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if lib.dg_argmax_workspace_bytes(mid, C) <= limit:
            lo = mid
        else:
            hi = mid
    return lo


def test_argcompare_rejects_before_launch(lib):
    need = lib.dg_argmax_workspace_bytes(4, 10)
    assert lib.dg_argcompare_rows(A16, 3, 0, A16, 4, 10, 10, A16, 1 << 20, None) == 6      # unknown dtype
    assert lib.dg_argcompare_rows(A16, 1, 2, A16, 4, 10, 10, A16, 1 << 20, None) == 6      # unknown op
    assert lib.dg_argcompare_rows(A16, 1, 1, A16, 4, 10, 9, A16, 1 << 20, None) == 3       # ld < C
    assert lib.dg_argcompare_rows(P(0x1001), 1, 1, A16, 4, 10, 10, A16, 1 << 20, None) == 2  # odd address
    assert lib.dg_argcompare_rows(P(0x1002), 0, 1, A16, 4, 10, 10, A16, 1 << 20, None) == 2  # f32 needs 4
    assert lib.dg_argcompare_rows(P(0x1002), 2, 1, A16, 4, 10, 10, None, 0, None) == (4 if need else 0)
    assert lib.dg_argcompare_rows(None, 2, 0, A16, 4, 10, 10, A16, 1 << 20, None) == 1
    assert lib.dg_argcompare_rows(None, 2, 0, None, 0, 10, 10, None, 0, None) == 0          # R = 0


def test_fused_tail_rejects_before_launch(lib):
    need = lib.dg_gemv_bf16_argmax_workspace_bytes(100, 64)
    assert need >= 400 + lib.dg_argmax_workspace_bytes(1, 100)
    assert lib.dg_gemv_bf16_argmax_workspace_bytes(0, 64) == 0
    assert lib.dg_gemv_bf16_argmax(A16, A16, A16, A16, 0, 64, 64, A16, need, None) == 3      # N = 0
    assert lib.dg_gemv_bf16_argmax(A16, A16, A16, A16, 100, 60, 64, A16, need, None) == 3    # K % 8
    assert lib.dg_gemv_bf16_argmax(A16, A16, A16, None, 100, 64, 64, A16, need, None) == 1   # no idx
    assert lib.dg_gemv_bf16_argmax(A16, A16, None, P(0x1004), 100, 64, 64, A16, need, None) == 2
    assert lib.dg_gemv_bf16_argmax(A16, A16, None, A16, 100, 64, 64, A16, need - 1, None) == 4
    assert lib.dg_gemv_bf16_argmax(A16, A16, None, A16, 100, 64, 64, None, need, None) == 4


def test_nf4_rejects_before_launch(lib):
    g = lib.dg_gemv_nf4
    assert g(A16, A16, A16, A16, A16, 4, 300, 64, None) == 3           # K % 256
    assert g(A16, A16, A16, A16, A16, 4, 33024, 64, None) == 3         # K > 32768
    assert g(A16, A16, A16, A16, A16, 4, 512, 48, None) == 3           # block size
    assert g(A16, A16, A16, A16, A16, 4, 768, 256, None) == 3          # K % (4 B)
    assert g(A16, A16, A16, A16, A16, -1, 512, 64, None) == 3
    assert g(None, A16, A16, A16, A16, 4, 512, 64, None) == 1
    assert g(A16, A16, None, A16, A16, 4, 512, 64, None) == 1
    assert g(A16, A16, A16, A16, None, 4, 512, 64, None) == 1
    assert g(A16, A16, P(0x1004), A16, A16, 4, 512, 64, None) == 2    # table 16-byte aligned
    assert g(A16, P(0x1008), A16, A16, A16, 4, 512, 64, None) == 2    # absmax 16-byte aligned
    assert g(A16, A16, A16, A2, A16, 4, 512, 64, None) == 2           # x
    assert g(A16, A16, A16, A16, P(0x1002), 4, 512, 64, None) == 2    # y
    assert g(None, None, None, None, None, 0, 512, 64, None) == 0     # N = 0
    import memory_bound_decode_gemv_amd as m
    for cfg in (m.dg_launch(5, 0, 0, 0), m.dg_launch(31, 0, 128, 0), m.dg_launch(31, 0, 0, 5),
                m.dg_launch(31, 0, 0, 122), m.dg_launch(31, 0, 0, 308), m.dg_launch(31, 0, 0, 6008)):
        assert lib.dg_gemv_nf4_ex(A16, A16, A16, A16, A16, 4, 512, 64, ctypes.byref(cfg), None) == 6
    q = lib.dg_quantize_nf4
    assert q(A16, A16, A16, A16, 2, 100, 64, None) == 3              # K % B
    assert q(A16, A16, A16, A16, 2, 128, 16, None) == 3              # block size
    assert q(A2, A16, A16, A16, 2, 128, 64, None) == 2               # w 16-byte aligned
    assert q(A16, A16, A16, None, 2, 128, 64, None) == 1
    assert q(None, None, None, None, 0, 128, 64, None) == 0


def test_quantisers_reject_before_launch(lib):
    assert lib.dg_quantize_q8_1(A16, A16, 2, 48, None) == 3
    assert lib.dg_quantize_q4_0(A16, A16, 2, 48, None) == 3
    assert lib.dg_quantize_q8_1(A2, A16, 2, 64, None) == 2
    assert lib.dg_quantize_q4_0(None, A16, 2, 64, None) == 1
    assert lib.dg_quantize_q8_1(None, None, 0, 64, None) == 0
    assert lib.dg_quantize_q8_0(A16, A16, 2, 48, None) == 3
    assert lib.dg_quantize_q8_0(A16, P(0x1001), 2, 64, None) == 2
    assert lib.dg_quantize_q8_0(None, A16, 2, 64, None) == 1


def test_binding_refuses_tensors_smaller_than_the_call_touches():
    """The binding checks that each tensor spans what the call would read or
    write, so a size argument larger than its tensor never reaches a kernel."""
    import torch
    import memory_bound_decode_gemv_amd as dg
    t = torch.zeros(10, dtype=torch.uint8)
    dg._fits(t, 10, "t")
    with pytest.raises(ValueError, match="holds 10 bytes"):
        dg._fits(t, 11, "t")
    f = torch.zeros((3, 4), dtype=torch.float32)
    dg._fits(f[1:], 32, "f")
    with pytest.raises(ValueError):
        dg._fits(f[1:], 33, "f")


def test_gemv_q4_0_f32_rejects_before_launch(lib):
    f = lib.dg_gemv_q4_0_f32
    assert f(A16, A16, A16, None, 4, 256, 1, None) == 1          # the two-launch form needs the Q8_1 buffer
    assert f(A16, A16, A16, None, 4, 256, 2, None) == 1
    assert f(A16, None, A16, None, 4, 256, 1, None) == 1          # no activations
    assert f(A16, A16, A16, P(0x1004), 4, 256, 1, None) == 2      # Q8_1 buffer not 16-byte aligned
    assert f(A16, P(0x1008), A16, A16, 4, 256, 1, None) == 2      # x not 16-byte aligned
    assert f(A16, A16, A16, A16, 4, 250, 1, None) == 3            # K % 256
    assert f(A16, A16, A16, A16, 4, 256, 25, None) == 3           # M > 24
    assert f(None, None, None, None, 0, 256, 1, None) == 0        # empty: nothing launched


def test_tiles_sizes(lib):
    lib.dg_q4_0_tiles_bytes.restype = ctypes.c_size_t
    lib.dg_q4_0_tiles_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64]
    assert lib.dg_q4_0_tiles_bytes(16, 256) == 2304
    assert lib.dg_q4_0_tiles_bytes(17, 512) == 2 * 2 * 2304
    assert lib.dg_q4_0_tiles_bytes(4096, 14336) == 256 * 56 * 2304
    assert lib.dg_q4_0_tiles_bytes(16, 100) == 0
    assert lib.dg_q4_0_tiles_bytes(-1, 256) == 0
    f = lib.dg_gemv_q4_0_tiles_workspace_bytes
    f.restype = ctypes.c_size_t
    f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
    assert f(4096, 28672, 24) > 0      # K split over workgroups
    assert f(4096, 14336, 16) == 0     # the columns in two slices instead
    assert f(4096, 4000, 16) == 0      # invalid shape
    assert f(4096, 14336, 25) == 0


@pytest.mark.parametrize("args,expect", [
    ((A16, A16, 4, 100), 3),              # K % 256
    ((A16, A16, -1, 256), 3),
    ((None, A16, 4, 256), 1),
    ((A16, None, 4, 256), 1),
    ((P(0x1001), A16, 4, 256), 2),        # Wq: 2-byte reads
    ((A16, A2, 4, 256), 2),               # Wt must be 16-byte aligned
    ((None, None, 0, 256), 0),            # N = 0
    ((None, None, 4, 0), 0),              # K = 0
])
def test_repack_q4_0_tiles_rejects_before_launch(lib, args, expect):
    assert lib.dg_repack_q4_0_tiles(*args, None) == expect


@pytest.mark.parametrize("args,expect", [
    ((A16, A16, A16, 4, 100, 1, None, 0), 3),                 # K % 256
    ((A16, A16, A16, 4, 256, 25, None, 0), 3),                # M > 24
    ((A16, A16, A16, 4, (1 << 26) + 256, 1, None, 0), 3),
    ((None, A16, A16, 4, 256, 1, None, 0), 1),
    ((A16, None, A16, 4, 256, 1, None, 0), 1),
    ((A16, A16, None, 4, 256, 1, None, 0), 1),
    ((A2, A16, A16, 4, 256, 1, None, 0), 2),                  # Wt 16-byte aligned
    ((A16, P(0x1004), A16, 4, 256, 1, None, 0), 2),           # Xq 16-byte aligned
    ((A16, A16, A2, 4, 256, 1, None, 0), 2),                  # Y 4-byte aligned
    ((A16, A16, A16, 4096, 28672, 24, A2, 1 << 24), 2),       # workspace 16-byte aligned
    ((A16, A16, A16, 4096, 28672, 24, None, 0), 4),           # K split: workspace needed
    ((A16, A16, A16, 4096, 28672, 24, A16, 64), 4),           # too small
    ((None, None, None, 4, 256, 0, None, 0), 0),              # M = 0
    ((None, None, None, 0, 256, 3, None, 0), 0),              # N = 0
])
def test_gemv_q4_0_tiles_rejects_before_launch(lib, args, expect):
    lib.dg_gemv_q4_0_tiles.argtypes = [P, P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, P, ctypes.c_size_t, P]
    assert lib.dg_gemv_q4_0_tiles(*args, None) == expect


def test_q8_0_tiles_sizes_and_rejections(lib):
    f = lib.dg_q8_0_tiles_bytes
    f.restype = ctypes.c_size_t
    f.argtypes = [ctypes.c_int64, ctypes.c_int64]
    assert f(16, 256) == 4352
    assert f(17, 512) == 2 * 2 * 4352
    assert f(16, 100) == 0
    assert lib.dg_repack_q8_0_tiles(A16, A16, 4, 100, None) == 3
    assert lib.dg_repack_q8_0_tiles(P(0x1001), A16, 4, 256, None) == 2
    assert lib.dg_repack_q8_0_tiles(None, A16, 4, 256, None) == 1
    g = lib.dg_gemv_q8_0_tiles
    g.argtypes = [P, P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, P, ctypes.c_size_t, P]
    assert g(A16, A16, A16, 4, 100, 1, None, 0, None) == 3
    assert g(A16, A16, A16, 4096, 14336, 24, None, 0, None) == 4   # Q8_0 splits K here, Q4_0 does not
    w = lib.dg_gemv_q8_0_tiles_workspace_bytes
    w.restype = ctypes.c_size_t
    w.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
    assert w(4096, 14336, 24) > 0
    w4 = lib.dg_gemv_q4_0_tiles_workspace_bytes
    w4.restype = ctypes.c_size_t
    w4.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
    assert w4(4096, 14336, 24) == 0
    assert g(A2, A16, A16, 4, 256, 1, None, 0, None) == 2
    assert g(None, None, None, 0, 256, 3, None, 0, None) == 0
