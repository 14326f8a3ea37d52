"""Parity of dg_gemv_nf4 and dg_quantize_nf4 with the oracle (GPU).

Operands are drawn by the seeded generators and quantised on the CPU by the
oracle's NF4 quantiser, with the workload's NormalFloat table; the GPU
quantiser is checked byte for byte against the oracle's separately.
"""
import functools

import numpy as np
import pytest

import synth
from tests._parity import assert_close

pytestmark = pytest.mark.gpu

# Floored relative error (the R5 form) against the fp64 oracle.  No page states
# a bound for NF4; it is a 4-bit weight GEMV like Q4_0, so it takes Q4_0's
# per-row bound.  Its fp32 products and sums (table values exact in the
# default kernel, held to 22 bits in the other two) leave an absolute error
# of a few 1e-5 on rows whose |y| is ~1e-3 of the rms: over all 28672 rows of
# the 70B shape the worst such row reaches about 3e-4.  One dropped weight
# moves y by ~0.1..1, far above 1e-3 of the rms.
TOL = 1e-3


@functools.lru_cache(maxsize=16)
def _operands(orc, cfg, N, K, B):
    w = synth.normal_f32((cfg, synth.KIND_W, 0, 0), (N, K))
    codes, absmax = orc.quantize_nf4(w, synth.nf4_table(), B, threads=0)
    xb = synth.normal_bf16_bits((cfg, synth.KIND_X, 0, 0), (K,), 1.0)
    return codes, absmax, xb


def _gpu(dg, dev, codes, absmax, table, xb, N, K, B, launch=None):
    import torch
    c = torch.from_numpy(np.ascontiguousarray(codes).reshape(-1)).to(dev)
    a = torch.from_numpy(np.ascontiguousarray(absmax, dtype=np.float32).reshape(-1)).to(dev)
    t = torch.from_numpy(np.ascontiguousarray(table, dtype=np.float32)).to(dev)
    x = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.full((max(N, 1),), float("nan"), dtype=torch.float32, device=dev)
    dg.dg_gemv_nf4(c, a, t, x, y, N=N, K=K, B=B, launch=launch)
    torch.cuda.synchronize()
    return y[:N].cpu().numpy().astype(np.float64)


SHAPES = [(1, 256, 64), (7, 2048, 32), (33, 4352, 64), (70, 8192, 64), (19, 14336, 128), (5, 16384, 256),
          (130, 1024, 256), (300, 2560, 64), (64, 6144, 32), (9, 28672, 64), (3, 32768, 128)]


@pytest.mark.parametrize("N,K,B", SHAPES)
def test_nf4_matches_oracle(dg, dev, orc, N, K, B):
    codes, absmax, xb = _operands(orc, 600 + K % 97, N, K, B)
    t = synth.nf4_table()
    got = _gpu(dg, dev, codes, absmax, t, xb, N, K, B)
    assert_close(got, orc.gemv_nf4(codes, absmax, t, xb, N, K, B), TOL, f"{N}x{K} B={B}")


LAUNCHES = [dict(variant=31), dict(variant=31, unroll=8), dict(variant=31, unroll=16), dict(variant=31, unroll=108),
            dict(variant=31, unroll=216), dict(variant=31, unroll=8216), dict(variant=31, unroll=4108),
            dict(variant=31, unroll=8008), dict(variant=31, grid=3),
            dict(variant=31, grid=2, unroll=16), dict(variant=31, grid=5, unroll=8208), dict(variant=31, grid=1),
            dict(variant=31, grid=4000), dict(variant=31, unroll=32), dict(variant=31, unroll=132),
            dict(variant=31, unroll=8032), dict(variant=31, unroll=4132, grid=3)]


@pytest.mark.parametrize("launch", LAUNCHES, ids=[str(v) for v in LAUNCHES])
@pytest.mark.parametrize("N,K,B", [(301, 8192, 64), (1000, 512, 32), (64, 4352, 64), (40, 6144, 128)])
def test_nf4_launch_variants(dg, dev, orc, launch, N, K, B):
    """Table copies, partial sums, and grids from one workgroup (every row in
    one workgroup: batches of 64 rows, then the rest) to more workgroups than
    rows."""
    codes, absmax, xb = _operands(orc, 620, N, K, B)
    t = synth.nf4_table()
    got = _gpu(dg, dev, codes, absmax, t, xb, N, K, B, launch=launch)
    assert_close(got, orc.gemv_nf4(codes, absmax, t, xb, N, K, B), TOL, f"{launch}")


# variant 33: (row groups G per workgroup, rows in flight + 100 * partial sums, grid); 0 is the default
ROWS_LAUNCHES = [(0, 0, 0), (0, 8, 0), (1, 4, 0), (1, 8, 1), (2, 4, 3), (3, 8, 5), (0, 4, 1), (0, 4, 4000),
                 (1, 4, 4000), (0, 8, 2), (0, 104, 0), (2, 204, 3), (1, 404, 0), (0, 208, 1), (3, 108, 0)]


@pytest.mark.parametrize("G,ahead,grid", ROWS_LAUNCHES)
@pytest.mark.parametrize("N,K,B", [(301, 8192, 64), (1000, 512, 32), (64, 4352, 64), (40, 6144, 128), (9, 28672, 64),
                                   (3, 32768, 128), (200, 2048, 256), (129, 14336, 32)])
def test_nf4_four_row_kernel(dg, dev, orc, N, K, B, G, ahead, grid):
    """The conflict-free table and four-row reduction: row groups per
    workgroup, rows in flight (whole groups of four, with streams whose row
    count is not a multiple of four or of 64), grids from one workgroup to
    more workgroups than rows."""
    S = (K + 2047) // 2048
    if G * S > 16:
        pytest.skip("more than 16 waves per workgroup")
    launch = dict(variant=33, unroll=ahead, grid=grid, block=G * S * 64)
    codes, absmax, xb = _operands(orc, 625, N, K, B)
    t = synth.nf4_table()
    got = _gpu(dg, dev, codes, absmax, t, xb, N, K, B, launch=launch)
    assert_close(got, orc.gemv_nf4(codes, absmax, t, xb, N, K, B), TOL, f"{launch}")


def test_nf4_four_row_kernel_rejects_bad_shapes(dg, dev, orc):
    codes, absmax, xb = _operands(orc, 630, 8, 8192, 64)
    for launch in (dict(variant=33, block=128), dict(variant=33, block=1280), dict(variant=33, unroll=2),
                   dict(variant=33, unroll=6), dict(variant=33, unroll=304), dict(variant=33, unroll=408)):
        with pytest.raises(dg.DGError):
            _gpu(dg, dev, codes, absmax, synth.nf4_table(), xb, 8, 8192, 64, launch=launch)


@pytest.mark.parametrize("N,K,B", [(1, 2048, 32), (17, 2048, 128), (33, 4096, 64), (300, 4096, 256), (70, 8192, 64),
                                   (5, 8192, 256), (1000, 4096, 32), (64, 8192, 128)])
@pytest.mark.parametrize("grid", [0, 1, 3])
def test_nf4_matrix_cores_match_oracle(dg, dev, orc, N, K, B, grid):
    """The matrix-core variant: K = 2048, 4096, 8192; block sizes from K/128 to
    K/16; ragged tiles; grids smaller than the tiles (workgroups loop)."""
    codes, absmax, xb = _operands(orc, 660 + K % 89, N, K, B)
    t = synth.nf4_table()
    got = _gpu(dg, dev, codes, absmax, t, xb, N, K, B, launch=dict(variant=32, grid=grid))
    assert_close(got, orc.gemv_nf4(codes, absmax, t, xb, N, K, B), TOL, f"mfma {N}x{K} B={B} grid={grid}")


@pytest.mark.parametrize("N,K,B", [(16, 1024, 64), (16, 14336, 64), (16, 2048, 256), (16, 8192, 32)])
def test_nf4_matrix_cores_refuse_other_shapes(dg, dev, orc, N, K, B):
    """K outside {2048, 4096, 8192}, a block longer than K/16 (256 > 2048/16)
    or shorter than K/128 (32 < 8192/128) is refused."""
    codes, absmax, xb = _operands(orc, 670, N, K, B)
    with pytest.raises(dg.DGError):
        _gpu(dg, dev, codes, absmax, synth.nf4_table(), xb, N, K, B, launch=dict(variant=32))


def test_nf4_matrix_cores_any_table_and_tiny_x(dg, dev, orc):
    """Unordered tables with repeats and a wide range; x with a tiny and a
    zero column stretch (one power-of-two scale for all of K)."""
    N, K, B = 45, 4096, 64
    g = np.random.default_rng(78)
    codes = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    absmax = np.abs(g.standard_normal((N, K // B))).astype(np.float32) * 3
    xf = g.standard_normal(K).astype(np.float32)
    xf[:512] *= 1e-3
    xf[512:640] = 0.0
    xb = (xf.view(np.uint32) >> 16).astype(np.uint16)   # truncation to bfloat16 bits (any bits are valid input)
    for t in (g.standard_normal(16).astype(np.float32) * 100, np.repeat(np.float32([0.5, -2.0]), 8),
              synth.nf4_table()):
        got = _gpu(dg, dev, codes, absmax, t, xb, N, K, B, launch=dict(variant=32))
        assert_close(got, orc.gemv_nf4(codes, absmax, t, xb, N, K, B), TOL, f"table {t[:3]}")


def test_nf4_any_table(dg, dev, orc):
    """The kernel takes any finite table: unordered, with repeats, wide range."""
    N, K, B = 90, 4096, 64
    g = np.random.default_rng(77)
    codes = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    absmax = np.abs(g.standard_normal((N, K // B))).astype(np.float32) * 3
    xb = synth.normal_bf16_bits((640, synth.KIND_X, 0, 0), (K,), 1.0)
    for t in (g.standard_normal(16).astype(np.float32) * 100, np.repeat(np.float32([0.5, -2.0]), 8),
              np.float32([1e-3 * (j - 8) for j in range(16)])):
        got = _gpu(dg, dev, codes, absmax, t, xb, N, K, B)
        assert_close(got, orc.gemv_nf4(codes, absmax, t, xb, N, K, B), TOL, f"table {t[:3]}")


def test_nf4_70b_mlp_shape_all_rows(dg, dev, orc):
    """28672 x 8192 with the default launch (the shape of the page's
    benchmark), operands quantised by the oracle; every row against it."""
    N, K, B = 28672, 8192, 64
    w = synth.normal_f32((7, synth.KIND_W, 0, 0), (N, K))
    table = synth.nf4_table()
    codes, absmax = orc.quantize_nf4(w, table, B, threads=0)
    del w
    xb = synth.normal_bf16_bits((7, synth.KIND_X, 0, 0), (K,), 1.0)
    got = _gpu(dg, dev, codes, absmax, table, xb, N, K, B)
    assert_close(got, orc.gemv_nf4(codes, absmax, table, xb, N, K, B, threads=0), TOL, "28672x8192 all rows")


def test_nf4_rejects_a_block_size_other_than_one_wave_per_unit(dg, dev, orc):
    codes, absmax, xb = _operands(orc, 630, 8, 8192, 64)
    with pytest.raises(dg.DGError):
        _gpu(dg, dev, codes, absmax, synth.nf4_table(), xb, 8, 8192, 64, launch=dict(variant=31, block=128))


def test_nf4_empty_and_zero_k(dg, dev):
    import torch
    t = torch.zeros(16, dtype=torch.float32, device=dev)
    c = torch.zeros(16, dtype=torch.uint8, device=dev)
    a = torch.zeros(16, dtype=torch.float32, device=dev)
    x = torch.zeros(8, dtype=torch.bfloat16, device=dev)
    y = torch.full((5,), 7.0, dtype=torch.float32, device=dev)
    dg.dg_gemv_nf4(c, a, t, x, y, N=0, K=256, B=64)        # nothing launched
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
    dg.dg_gemv_nf4(c, a, t, x, y, N=5, K=0, B=64)          # empty sums
    torch.cuda.synchronize()
    assert torch.all(y == 0.0)


def _gpu_quantize(dg, dev, w, table, B):
    import torch
    N, K = w.shape
    wt = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(dev)
    t = torch.from_numpy(np.ascontiguousarray(table, dtype=np.float32)).to(dev)
    codes = torch.full((N * K // 2,), 0xA5, dtype=torch.uint8, device=dev)
    absmax = torch.full((N * (K // B),), float("nan"), dtype=torch.float32, device=dev)
    dg.dg_quantize_nf4(wt, codes, absmax, t, N, K, B)
    torch.cuda.synchronize()
    return codes.cpu().numpy().reshape(N, K // 2), absmax.cpu().numpy().reshape(N, K // B)


@pytest.mark.parametrize("N,K,B", [(1, 32, 32), (3, 256, 64), (17, 4096, 128), (4, 14336, 256), (9, 2048, 64)])
def test_nf4_quantiser_bytes_match_oracle(dg, dev, orc, N, K, B):
    w = synth.normal_f32((650, synth.KIND_W, N, K), (N, K))
    for table in (synth.nf4_table(), np.float32([(j - 7) / 8 for j in range(16)])):
        c, a = _gpu_quantize(dg, dev, w, table, B)
        rc, ra = orc.quantize_nf4(w, table, B)
        assert np.array_equal(a, ra) and np.array_equal(c, rc)


def test_nf4_quantiser_ties_zeros_and_extremes(dg, dev, orc):
    """Values on exact midpoints of a dyadic table, all-zero blocks, the
    extreme levels and negative zero."""
    td = np.float32([(j - 7) / 8 for j in range(16)])
    mids = (td[:-1] + td[1:]) / 2
    K, B = 256, 32
    rows = [np.tile(np.concatenate([[1.0], mids, mids[:16 - 1], [-1.0]]).astype(np.float32), K // 32)[:K],
            np.zeros(K, np.float32), np.full(K, -0.0, np.float32),
            np.tile(np.float32([-3.0, 3.0] + [0.375] * 30), K // 32)]
    w = np.stack(rows).astype(np.float32)
    c, a = _gpu_quantize(dg, dev, w, td, B)
    rc, ra = orc.quantize_nf4(w, td, B)
    assert np.array_equal(a, ra) and np.array_equal(c, rc)
