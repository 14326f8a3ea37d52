"""Parity of dg_gemv_q4_0 (Q4_0 x Q8_1, M = 1..24) with the oracle (GPU).

Operands are quantised on the CPU by the oracle's quantisers from seeded
N(0, 1) draws, so no input comes from the GPU path; the GPU's own quantisers
are checked separately, byte for byte, in test_gpu_quantize.py.
"""
import functools
import json
import os

import numpy as np
import pytest

import synth
from tests._parity import assert_close

pytestmark = pytest.mark.gpu

TOL = 1e-3   # per-row floored relative error vs the oracle


@functools.lru_cache(maxsize=8)
def _weights(orc, cfg, N, K, copy):
    return orc.quantize_q4_0(synth.normal_f32((cfg, synth.KIND_W, copy, 0), (N, K)), threads=0)


def _operands(orc, cfg, N, K, M, copy=0, same_columns=False):
    Wq = _weights(orc, cfg, N, K, copy)
    cols = []
    for m in range(M):
        cols.append(synth.normal_f32((cfg, synth.KIND_X, copy, 0 if same_columns else m), (K,)))
    Xq = orc.quantize_q8_1(np.stack(cols))
    return Wq, Xq


def _gpu(dg, dev, Wq, Xq, N, K, M, launch=None):
    import torch
    W = torch.from_numpy(np.ascontiguousarray(Wq).reshape(-1)).to(dev)
    X = torch.from_numpy(np.ascontiguousarray(Xq).reshape(-1)).to(dev)
    Y = torch.full((max(M, 1), max(N, 1)), float("nan"), dtype=torch.float32, device=dev)
    dg.dg_gemv_q4_0(W, X, Y, N, K, M, launch=launch)
    torch.cuda.synchronize()
    return Y[:M, :N].cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("M", list(range(1, 25)))
def test_q4_0_every_column_count_small(dg, dev, orc, M):
    # K = 768: 12 block pairs per row, far from a full 64-pair step (ragged tail)
    N, K = 41, 768
    Wq, Xq = _operands(orc, 200 + M, N, K, M)
    got = _gpu(dg, dev, Wq, Xq, N, K, M)
    ref = orc.gemv_q4_0_q8_1(Wq, Xq, N, K, M)
    for m in range(M):
        assert_close(got[m], ref[m], TOL, f"M={M} column {m}")


@pytest.mark.parametrize("N,K", [(1, 256), (7, 4096), (70, 4352), (33, 8192), (64, 12288), (19, 14336), (5, 16384)])
@pytest.mark.parametrize("M", [1, 2, 5, 16, 24])
def test_q4_0_shapes_span_steps_and_tails(dg, dev, orc, N, K, M):
    Wq, Xq = _operands(orc, 210, N, K, M)
    got = _gpu(dg, dev, Wq, Xq, N, K, M)
    ref = orc.gemv_q4_0_q8_1(Wq, Xq, N, K, M)
    assert_close(got, ref, TOL, f"{N}x{K} M={M}")


VARIANTS = [
    dict(variant=11), dict(variant=11, grid=3, block=64), dict(variant=11, block=128),
    dict(variant=12, unroll=1), dict(variant=12, unroll=2), dict(variant=12, unroll=4), dict(variant=12, grid=2),
    dict(variant=13), dict(variant=13, grid=3, block=64), dict(variant=13, grid=5, block=192),
    dict(variant=13, block=128),
]


@pytest.mark.parametrize("launch", VARIANTS, ids=[str(v) for v in VARIANTS])
def test_q4_0_m1_variants(dg, dev, orc, launch):
    N, K = 301, 8192
    Wq, Xq = _operands(orc, 220, N, K, 1)
    got = _gpu(dg, dev, Wq, Xq, N, K, 1, launch=launch)
    assert_close(got[0], orc.gemv_q4_0_q8_1(Wq, Xq, N, K, 1)[0], TOL, str(launch))


@pytest.mark.parametrize("N,K", [(1, 256), (7, 4096), (70, 4352), (33, 8192), (64, 12288), (19, 14336),
                                 (5, 16384), (130, 2304)])
@pytest.mark.parametrize("launch", [dict(variant=15), dict(variant=15, unroll=2), dict(variant=15, unroll=4),
                                    dict(variant=15, grid=2, block=128), dict(variant=15, grid=1, block=64),
                                    dict(variant=15, unroll=2, grid=3, block=192)])
def test_q4_0_m1_units(dg, dev, orc, N, K, launch):
    """M = 1 with rows copied in units of 64 block pairs (ragged last units,
    several rows and units per wave)."""
    Wq, Xq = _operands(orc, 228, N, K, 1)
    got = _gpu(dg, dev, Wq, Xq, N, K, 1, launch=launch)
    assert_close(got[0], orc.gemv_q4_0_q8_1(Wq, Xq, N, K, 1)[0], TOL, f"{N}x{K} {launch}")


UNITS_FEW = [None, dict(variant=15), dict(variant=15, unroll=2), dict(variant=15, unroll=4),
             dict(variant=15, grid=2, block=128), dict(variant=15, grid=1, block=64),
             dict(variant=15, unroll=2, grid=3, block=192)]


@pytest.mark.parametrize("N,K,M", [(1, 256, 4), (7, 4096, 4), (70, 2304, 3), (33, 8192, 2), (130, 4352, 2),
                                   (301, 4096, 2), (64, 512, 3), (19, 16384, 1), (9, 4096, 8), (40, 1792, 6),
                                   (33, 8192, 4), (19, 14336, 2), (64, 12288, 2)])
@pytest.mark.parametrize("launch", UNITS_FEW, ids=[str(v) for v in UNITS_FEW])
def test_q4_0_units_few_columns(dg, dev, orc, N, K, M, launch):
    """Two to eight columns through the 64-pair units kernel (the weights of a
    pair are read and unpacked once for every column; M * ceil(K / 4096) <= 8)."""
    Wq, Xq = _operands(orc, 232, N, K, M)
    got = _gpu(dg, dev, Wq, Xq, N, K, M, launch=launch)
    assert_close(got, orc.gemv_q4_0_q8_1(Wq, Xq, N, K, M), TOL, f"{N}x{K} M={M} {launch}")


def test_q4_0_units_reject_too_many_columns(dg, dev, orc):
    """M * ceil(K / 4096) > 8 does not fit the units kernel's registers: an
    explicit request is an argument error, launching nothing."""
    Wq, Xq = _operands(orc, 233, 8, 8192, 5)
    with pytest.raises(dg.DGError):
        _gpu(dg, dev, Wq, Xq, 8, 8192, 5, launch=dict(variant=15))


@pytest.mark.parametrize("N,launch", [(300, dict(variant=13, grid=1, block=64)),
                                      (129, dict(variant=13, grid=1, block=64, unroll=3)),
                                      (1000, dict(variant=13, grid=2, block=128, unroll=4)),
                                      (64, dict(variant=13, grid=1, block=64)),
                                      (300, dict(variant=15, grid=1, block=64)),
                                      (1000, dict(variant=15, grid=2, block=128, unroll=4))])
@pytest.mark.parametrize("M", [1, 3])
def test_q4_0_m1_many_rows_per_wave(dg, dev, orc, N, launch, M):
    """One wave computing more than 64 rows: its results are stored 64 rows at
    a time, then the remainder (three columns: the units kernel only)."""
    if M > 1 and launch["variant"] != 15:
        pytest.skip("the LDS-row kernel takes one column")
    K = 512
    Wq, Xq = _operands(orc, 227, N, K, M)
    got = _gpu(dg, dev, Wq, Xq, N, K, M, launch=launch)
    assert_close(got, orc.gemv_q4_0_q8_1(Wq, Xq, N, K, M), TOL, f"{N} M={M} {launch}")


@pytest.mark.parametrize("N,K", [(1, 256), (7, 4096), (70, 4352), (33, 8192), (64, 12288), (130, 2304)])
@pytest.mark.parametrize("launch", [dict(variant=13), dict(variant=13, grid=2, block=128),
                                    dict(variant=13, unroll=2, grid=3, block=64),
                                    dict(variant=13, unroll=4, grid=2, block=64),
                                    dict(variant=13, unroll=3, grid=1, block=256)])
def test_q4_0_lds_row_copy_shapes(dg, dev, orc, N, K, launch):
    Wq, Xq = _operands(orc, 225, N, K, 1)
    got = _gpu(dg, dev, Wq, Xq, N, K, 1, launch=launch)
    assert_close(got[0], orc.gemv_q4_0_q8_1(Wq, Xq, N, K, 1)[0], TOL, f"{N}x{K} {launch}")


from tests._parity import MFMA_CONFIGS, mfma_max_columns, mfma_unroll  # noqa: E402

MFMA_TABLE = {c: mfma_max_columns(18, *c) for c in MFMA_CONFIGS}
_mfma_unroll = mfma_unroll
MFMA_CFGS = [dict(variant=14)] + [dict(variant=14, unroll=mfma_unroll(*c)) for c in MFMA_CONFIGS if MFMA_TABLE[c]]


def _mfma_supported(launch, M):
    u = launch.get("unroll", 0)
    if not u:
        return True
    return M <= MFMA_TABLE[(u // 10000, (u // 100) % 100, (u // 10) % 10, (u % 10) * 8)]


@pytest.mark.parametrize("launch", MFMA_CFGS, ids=[str(v) for v in MFMA_CFGS])
@pytest.mark.parametrize("N,K,M", [(37, 256, 2), (130, 4352, 7), (64, 8192, 16), (200, 2304, 17), (33, 12544, 24),
                                   (16, 512, 3), (1, 1024, 24), (700, 4096, 12), (90, 2560, 4), (50, 1792, 8),
                                   (45, 3328, 1)])
def test_q4_0_mfma_matches_oracle(dg, dev, orc, launch, N, K, M):
    if not _mfma_supported(launch, M):
        pytest.skip("configuration not built for this column count (LDS of one workgroup)")
    Wq, Xq = _operands(orc, 260, N, K, M)
    got = _gpu(dg, dev, Wq, Xq, N, K, M, launch=launch)
    assert_close(got, orc.gemv_q4_0_q8_1(Wq, Xq, N, K, M), TOL, f"mfma {launch} {N}x{K} M={M}")


@pytest.mark.parametrize("grid", [1, 3, 7])
@pytest.mark.parametrize("unroll", [0, 11611, 40221, 40131])
def test_q4_0_mfma_any_grid_covers_every_row_tile(dg, dev, orc, grid, unroll):
    """A grid smaller than the number of row-tile groups loops over them."""
    N, K, M = 333, 2304, 5
    Wq, Xq = _operands(orc, 265, N, K, M)
    launch = dict(variant=14, grid=grid, unroll=unroll)
    got = _gpu(dg, dev, Wq, Xq, N, K, M, launch=launch)
    assert_close(got, orc.gemv_q4_0_q8_1(Wq, Xq, N, K, M), TOL, str(launch))


@pytest.mark.parametrize("M,R", [(2, 1), (2, 2), (3, 4), (8, 1), (8, 2), (9, 1), (10, 1), (10, 2), (24, 1), (24, 2)])
def test_q4_0_lds_rows_per_wave(dg, dev, orc, M, R):
    N, K = 77, 4608
    Wq, Xq = _operands(orc, 230, N, K, M)
    got = _gpu(dg, dev, Wq, Xq, N, K, M, launch=dict(variant=12, unroll=R))
    assert_close(got, orc.gemv_q4_0_q8_1(Wq, Xq, N, K, M), TOL, f"M={M} R={R}")


def test_q4_0_70b_mlp_shape_all_rows(dg, dev, orc):
    """The 4-bit M = 1 decode shape, N = 28672, K = 8192: every row against the
    oracle (the output starts as NaN, so a row never written fails too)."""
    N, K = 28672, 8192
    Wq, Xq = _operands(orc, 2, N, K, 1)
    got = _gpu(dg, dev, Wq, Xq, N, K, 1)
    assert_close(got, orc.gemv_q4_0_q8_1(Wq, Xq, N, K, 1, threads=0), TOL, "28672x8192 all rows")


@pytest.mark.parametrize("N,K", [(4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336)])
@pytest.mark.parametrize("M", [1, 2, 4, 8, 12, 16, 24])
def test_q4_0_decoder_layer_shapes_all_rows(dg, dev, orc, N, K, M):
    Wq, Xq = _operands(orc, 3, N, K, M)
    got = _gpu(dg, dev, Wq, Xq, N, K, M)
    assert_close(got, orc.gemv_q4_0_q8_1(Wq, Xq, N, K, M, threads=0), TOL, f"{N}x{K} M={M}")


# Scales below the binary16 normal range (|w| ~ 1e-5 gives weight scales of
# about 1e-6, |x| ~ 1e-4 activation scales of about 1e-6): every kernel family
# keeps them, the matrix-core kernels included, which multiply the raw
# binary16 scales on the f16 matrix cores.
@pytest.mark.parametrize("M,launch", [(1, None), (3, None), (12, None), (24, None), (12, dict(variant=16)),
                                      (24, dict(variant=16))])
def test_q4_0_subnormal_scales(dg, dev, orc, M, launch):
    N, K = 300, 4096
    Wq = orc.quantize_q4_0(synth.normal_f32((900, synth.KIND_W, 0, 0), (N, K)) * np.float32(1e-5))
    cols = [synth.normal_f32((900, synth.KIND_X, 0, m), (K,)) * np.float32(1e-4) for m in range(M)]
    Xq = orc.quantize_q8_1(np.stack(cols))
    d_w = np.ascontiguousarray(Wq).reshape(N, K // 32, 18)[:, :, :2].copy().view(np.float16)
    d_x = np.ascontiguousarray(Xq).reshape(M, K // 32, 36)[:, :, :2].copy().view(np.float16)
    assert np.all(np.abs(d_w) < 2.0 ** -14) and np.all(np.abs(d_x) < 2.0 ** -14)
    assert np.count_nonzero(d_w) > 0 and np.count_nonzero(d_x) > 0
    got = _gpu(dg, dev, Wq, Xq, N, K, M, launch=launch)
    ref = orc.gemv_q4_0_q8_1(Wq, Xq, N, K, M)
    assert_close(got, ref, TOL, f"subnormal scales M={M} {launch}")


# The default kernel and configuration follow the column count, the row-tile
# count and the row length; these three shapes take every branch of that
# choice for every M.
@pytest.mark.parametrize("N,K", [(1024, 4096), (14336, 4096), (4096, 14336)])
@pytest.mark.parametrize("M", list(range(1, 25)))
def test_q4_0_default_launch_every_column_count(dg, dev, orc, N, K, M):
    Wq, Xq = _operands(orc, 3, N, K, M)
    got = _gpu(dg, dev, Wq, Xq, N, K, M)
    assert_close(got, orc.gemv_q4_0_q8_1(Wq, Xq, N, K, M, threads=0), TOL, f"{N}x{K} M={M}")


@pytest.mark.parametrize("M", [2, 13, 16, 24])
def test_q4_0_identical_columns_give_identical_outputs(dg, dev, orc, M):
    N, K = 300, 4096
    Wq, Xq = _operands(orc, 240, N, K, M, same_columns=True)
    got = _gpu(dg, dev, Wq, Xq, N, K, M)
    for m in range(1, M):
        assert np.array_equal(got[m], got[0])


def test_q4_0_overrides_beyond_kernel_limits_are_rejected(dg, dev):
    """Launch overrides a kernel cannot take (more threads than it was compiled
    for, a variant for another column count) return an argument error instead
    of launching."""
    import torch
    N, K = 64, 8192
    W = torch.zeros(N * K // 32 * 18, dtype=torch.uint8, device=dev)
    X = torch.zeros(24 * K // 32 * 36, dtype=torch.uint8, device=dev)
    Y = torch.zeros(24 * N, dtype=torch.float32, device=dev)
    for M, launch in ((1, dict(variant=11, block=512)), (1, dict(variant=13, block=1024)),
                      (2, dict(variant=11)), (2, dict(variant=13)), (1, dict(variant=12, block=128)),
                      (5, dict(variant=12, unroll=4)), (1, dict(variant=99)),
                      (4, dict(variant=14, unroll=124)), (4, dict(variant=14, unroll=21622)),
                      (4, dict(variant=14, unroll=10412)), (4, dict(variant=14, unroll=10461)),
                      (20, dict(variant=14, unroll=11611)), (20, dict(variant=14, unroll=10821)),
                      (5, dict(variant=15)), (1, dict(variant=15, block=512)), (1, dict(variant=15, unroll=5))):
        with pytest.raises(dg.DGError) as e:
            dg.dg_gemv_q4_0(W, X, Y, N, K, M, launch=launch)
        assert e.value.status == dg.DG_ERR_ARG, launch


def test_q4_0_worked_blocks_tiled(dg, dev):
    """The hand-worked blocks of tests/golden, each repeated 8 times along K
    (K = 256): y = 8 times the block's value, exact in fp32."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "q4_0_q8_1_worked.json")) as f:
        ex = json.load(f)["dot_examples"]
    for e in ex:
        w = np.frombuffer(bytes.fromhex(e["q4_0_block_hex"].replace(" ", "")), np.uint8)
        x = np.frombuffer(bytes.fromhex(e["q8_1_block_hex"].replace(" ", "")), np.uint8)
        got = _gpu(dg, dev, np.tile(w, 8), np.tile(x, 8), 1, 256, 1)
        assert got[0, 0] == 8 * e["y"], e["name"]


def test_q4_0_k_zero_and_empty(dg, dev):
    import torch
    W = torch.zeros(64, dtype=torch.uint8, device=dev)
    X = torch.zeros(64, dtype=torch.uint8, device=dev)
    Y = torch.full((3, 5), 9.0, dtype=torch.float32, device=dev)
    dg.dg_gemv_q4_0(W, X, Y, 5, 256, 0)      # M = 0: nothing written
    dg.dg_gemv_q4_0(W, X, Y, 0, 256, 3)      # N = 0: nothing written
    torch.cuda.synchronize()
    assert torch.all(Y == 9.0)
    dg.dg_gemv_q4_0(W, X, Y, 5, 0, 3)        # K = 0: empty sums
    torch.cuda.synchronize()
    assert torch.all(Y == 0.0)


def test_q4_0_deterministic(dg, dev, orc):
    N, K, M = 1000, 8192, 3
    Wq, Xq = _operands(orc, 250, N, K, M)
    a = _gpu(dg, dev, Wq, Xq, N, K, M)
    b = _gpu(dg, dev, Wq, Xq, N, K, M)
    assert np.array_equal(a, b)


# ---- the resident-activation matrix-core kernel (variant 16) ----
from tests._parity import RES_CFGS, res_default, res_runs, res_unroll  # noqa: E402

RES_LAUNCHES = [dict(variant=16)] + [dict(variant=16, unroll=res_unroll(*c)) for c in RES_CFGS]
RES_SHAPES = [(37, 4096, 2), (130, 8192, 7), (64, 4096, 16), (200, 4096, 17), (33, 4096, 24), (16, 4096, 3),
              (1, 4096, 24), (700, 4096, 12), (90, 8192, 4), (45, 4096, 1), (50, 12288, 8), (301, 2048, 5),
              (77, 14336, 4), (19, 1024, 9)]


def _res_expected(launch, N, M, K):
    u = launch.get("unroll", 0) or res_unroll(*res_default(18, N, M, K))
    return res_runs(18, u // 10000, (u // 100) % 100, M, K)


@pytest.mark.parametrize("launch", RES_LAUNCHES, ids=[str(v) for v in RES_LAUNCHES])
@pytest.mark.parametrize("N,K,M", RES_SHAPES)
def test_q4_0_res_matches_oracle(dg, dev, orc, launch, N, K, M):
    """Every built configuration on shapes with ragged row tiles and groups;
    configurations that cannot take a shape must be refused, not run."""
    Wq, Xq = _operands(orc, 270, N, K, M)
    if not _res_expected(launch, N, M, K):
        with pytest.raises(dg.DGError):
            _gpu(dg, dev, Wq, Xq, N, K, M, launch=launch)
        return
    got = _gpu(dg, dev, Wq, Xq, N, K, M, launch=launch)
    assert_close(got, orc.gemv_q4_0_q8_1(Wq, Xq, N, K, M), TOL, f"res {launch} {N}x{K} M={M}")


@pytest.mark.parametrize("grid", [1, 3, 7, 1000])
@pytest.mark.parametrize("unroll", [10820, 20420, 40120, 10430, 11620])
def test_q4_0_res_any_grid_covers_every_row_group(dg, dev, orc, grid, unroll):
    """Grids smaller than the row groups loop over them; larger grids leave
    workgroups without rows (they still meet every barrier)."""
    N, K, M = 333, 4096, 6
    Wq, Xq = _operands(orc, 275, N, K, M)
    launch = dict(variant=16, grid=grid, unroll=unroll)
    got = _gpu(dg, dev, Wq, Xq, N, K, M, launch=launch)
    assert_close(got, orc.gemv_q4_0_q8_1(Wq, Xq, N, K, M), TOL, str(launch))


@pytest.mark.parametrize("M", [2, 13, 16, 24])
def test_q4_0_res_identical_columns_give_identical_outputs(dg, dev, orc, M):
    N, K = 300, 4096
    Wq, Xq = _operands(orc, 240, N, K, M, same_columns=True)
    got = _gpu(dg, dev, Wq, Xq, N, K, M, launch=dict(variant=16, unroll=res_unroll(1, 4, 2)))
    for m in range(1, M):
        assert np.array_equal(got[m], got[0])
