"""Parity of dg_gemv_q8_0 (Q8_0 x Q8_1, M = 1..24) with the oracle (GPU).

Operands are quantised on the CPU by the oracle's quantisers from seeded
N(0, 1) draws; the GPU quantiser is checked byte for byte in
test_gpu_quantize.py.
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

# Matrix-core configurations built for Q8_0: (RT, KS, DEPTH, CB) -> the
# largest column count they serve (their LDS must fit one workgroup).
from tests._parity import MFMA_CONFIGS, mfma_max_columns  # noqa: E402

MFMA_TABLE = {c: c_max for c in MFMA_CONFIGS if (c_max := mfma_max_columns(34, *c))}


def _unroll(rt, ks, d, cb):
    return rt * 10000 + ks * 100 + d * 10 + cb // 8


@functools.lru_cache(maxsize=8)
def _weights(orc, cfg, N, K, copy):
    return orc.quantize_q8_0(synth.normal_f32((cfg, synth.KIND_W, copy, 0), (N, K)), threads=0)


def _operands(orc, cfg, N, K, M, same_columns=False):
    Wq = _weights(orc, cfg, N, K, 0)
    cols = [synth.normal_f32((cfg, synth.KIND_X, 0, 0 if same_columns else m), (K,)) for m in range(M)]
    return Wq, orc.quantize_q8_1(np.stack(cols))


def _gpu(dg, dev, Wq, Xq, N, K, M, launch=None):
    import torch
    W = torch.from_numpy(np.ascontiguousarray(Wq).reshape(-1)).to(dev)
    X = torch.from_numpy(np.ascontiguousarray(Xq).reshape(-1)).to(dev)
    Y = torch.full((max(M, 1), max(N, 1)), float("nan"), dtype=torch.float32, device=dev)
    dg.dg_gemv_q8_0(W, X, Y, N, K, M, launch=launch)
    torch.cuda.synchronize()
    return Y[:M, :N].cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("M", list(range(1, 25)))
def test_q8_0_every_column_count_small(dg, dev, orc, M):
    N, K = 41, 768
    Wq, Xq = _operands(orc, 400 + M, N, K, M)
    assert_close(_gpu(dg, dev, Wq, Xq, N, K, M), orc.gemv_q8_0_q8_1(Wq, Xq, N, K, M), TOL, f"M={M}")


@pytest.mark.parametrize("N,K", [(1, 256), (7, 4096), (70, 4352), (33, 8192), (64, 12288), (19, 14336),
                                 (5, 16384), (9, 20480)])
@pytest.mark.parametrize("M", [1, 2, 5, 16, 24])
def test_q8_0_shapes_span_steps_and_tails(dg, dev, orc, N, K, M):
    Wq, Xq = _operands(orc, 410, N, K, M)
    assert_close(_gpu(dg, dev, Wq, Xq, N, K, M), orc.gemv_q8_0_q8_1(Wq, Xq, N, K, M), TOL, f"{N}x{K} M={M}")


@pytest.mark.parametrize("N,K", [(1, 256), (130, 2304), (33, 8192), (19, 12544), (5, 16384)])
@pytest.mark.parametrize("launch", [dict(variant=21), dict(variant=21, grid=2, block=128),
                                    dict(variant=21, unroll=3, grid=3, block=64),
                                    dict(variant=21, unroll=4, grid=1, block=64),
                                    dict(variant=21, grid=1, block=64), dict(variant=22)])
def test_q8_0_m1_variants(dg, dev, orc, N, K, launch):
    Wq, Xq = _operands(orc, 420, N, K, 1)
    assert_close(_gpu(dg, dev, Wq, Xq, N, K, 1, launch=launch)[0], orc.gemv_q8_0_q8_1(Wq, Xq, N, K, 1)[0], TOL,
                 f"{N}x{K} {launch}")


@pytest.mark.parametrize("launch", [dict(variant=21, grid=1, block=64), dict(variant=23, grid=1, block=64),
                                    dict(variant=23, grid=1, block=128, unroll=4)])
def test_q8_0_m1_many_rows_per_wave(dg, dev, orc, launch):
    N, K = 300, 4352
    Wq, Xq = _operands(orc, 425, N, K, 1)
    got = _gpu(dg, dev, Wq, Xq, N, K, 1, launch=launch)
    assert_close(got[0], orc.gemv_q8_0_q8_1(Wq, Xq, N, K, 1)[0], TOL, f"300 rows {launch}")


@pytest.mark.parametrize("N,K", [(1, 256), (7, 4096), (70, 4352), (33, 8192), (64, 12288), (19, 14336),
                                 (5, 16384), (130, 2304)])
@pytest.mark.parametrize("launch", [dict(variant=23), dict(variant=23, unroll=2), dict(variant=23, unroll=4),
                                    dict(variant=23, grid=2, block=128), dict(variant=23, unroll=2, grid=3, block=192)])
def test_q8_0_m1_units(dg, dev, orc, N, K, launch):
    Wq, Xq = _operands(orc, 428, N, K, 1)
    got = _gpu(dg, dev, Wq, Xq, N, K, 1, launch=launch)
    assert_close(got[0], orc.gemv_q8_0_q8_1(Wq, Xq, N, K, 1)[0], TOL, f"{N}x{K} {launch}")


UNITS_FEW = [None, dict(variant=23), dict(variant=23, unroll=2), dict(variant=23, unroll=4),
             dict(variant=23, grid=2, block=128), dict(variant=23, unroll=2, grid=3, block=192)]


@pytest.mark.parametrize("N,K,M", [(1, 256, 4), (7, 4096, 4), (70, 2304, 3), (33, 8192, 2), (130, 4352, 2),
                                   (301, 4096, 2), (1000, 512, 3), (9, 4096, 8), (33, 8192, 4), (19, 14336, 2),
                                   (64, 12288, 2), (9, 4096, 9), (70, 2304, 10), (1000, 512, 9), (130, 4096, 10),
                                   (9, 4096, 11), (130, 4096, 12), (700, 2304, 12)])
@pytest.mark.parametrize("launch", UNITS_FEW, ids=[str(v) for v in UNITS_FEW])
def test_q8_0_units_few_columns(dg, dev, orc, N, K, M, launch):
    """Two to twelve columns through the 64-pair units kernel (M * ceil(K / 4096) <= 8, or up to twelve
    columns of rows of one unit, K <= 4096)."""
    Wq, Xq = _operands(orc, 432, N, K, M)
    got = _gpu(dg, dev, Wq, Xq, N, K, M, launch=launch)
    assert_close(got, orc.gemv_q8_0_q8_1(Wq, Xq, N, K, M), TOL, f"{N}x{K} M={M} {launch}")


MFMA_CFGS = [dict(variant=22)] + [dict(variant=22, unroll=_unroll(*c)) for c in MFMA_TABLE]


@pytest.mark.parametrize("launch", MFMA_CFGS, ids=[str(v) for v in MFMA_CFGS])
@pytest.mark.parametrize("N,K,M", [(37, 256, 2), (130, 4352, 7), (64, 8192, 16), (200, 2304, 17), (33, 12544, 24),
                                   (16, 512, 3), (700, 4096, 12), (45, 3328, 1)])
def test_q8_0_mfma_matches_oracle(dg, dev, orc, launch, N, K, M):
    u = launch.get("unroll", 0)
    if u and M > MFMA_TABLE[(u // 10000, (u // 100) % 100, (u // 10) % 10, (u % 10) * 8)]:
        pytest.skip("configuration not built for this column count (LDS of one workgroup)")
    Wq, Xq = _operands(orc, 430, N, K, M)
    assert_close(_gpu(dg, dev, Wq, Xq, N, K, M, launch=launch), orc.gemv_q8_0_q8_1(Wq, Xq, N, K, M), TOL,
                 f"mfma {launch} {N}x{K} M={M}")


def test_q8_0_70b_mlp_shape_all_rows(dg, dev, orc):
    N, K = 28672, 8192
    Wq, Xq = _operands(orc, 2, N, K, 1)
    got = _gpu(dg, dev, Wq, Xq, N, K, 1)
    assert_close(got, orc.gemv_q8_0_q8_1(Wq, Xq, N, K, 1, threads=0), TOL, "28672x8192 all rows")


@pytest.mark.parametrize("N,K", [(4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336)])
@pytest.mark.parametrize("M", [1, 2, 4, 8, 12, 16, 24])
def test_q8_0_decoder_layer_shapes_all_rows(dg, dev, orc, N, K, M):
    Wq, Xq = _operands(orc, 3, N, K, M)
    got = _gpu(dg, dev, Wq, Xq, N, K, M)
    assert_close(got, orc.gemv_q8_0_q8_1(Wq, Xq, N, K, M, threads=0), TOL, f"{N}x{K} M={M}")


# Scales below the binary16 normal range (|w| ~ 1e-5 gives weight scales of
# about 1e-6, |x| ~ 1e-4 activation scales of about 1e-6): every kernel family
# keeps them, the matrix-core kernels included, which multiply the raw
# binary16 scales on the f16 matrix cores.
@pytest.mark.parametrize("M,launch", [(1, None), (3, None), (12, None), (24, None), (12, dict(variant=24)),
                                      (24, dict(variant=24))])
def test_q8_0_subnormal_scales(dg, dev, orc, M, launch):
    N, K = 300, 4096
    Wq = orc.quantize_q8_0(synth.normal_f32((900, synth.KIND_W, 0, 0), (N, K)) * np.float32(1e-5))
    cols = [synth.normal_f32((900, synth.KIND_X, 0, m), (K,)) * np.float32(1e-4) for m in range(M)]
    Xq = orc.quantize_q8_1(np.stack(cols))
    d_w = np.ascontiguousarray(Wq).reshape(N, K // 32, 34)[:, :, :2].copy().view(np.float16)
    d_x = np.ascontiguousarray(Xq).reshape(M, K // 32, 36)[:, :, :2].copy().view(np.float16)
    assert np.all(np.abs(d_w) < 2.0 ** -14) and np.all(np.abs(d_x) < 2.0 ** -14)
    assert np.count_nonzero(d_w) > 0 and np.count_nonzero(d_x) > 0
    got = _gpu(dg, dev, Wq, Xq, N, K, M, launch=launch)
    ref = orc.gemv_q8_0_q8_1(Wq, Xq, N, K, M)
    assert_close(got, ref, TOL, f"subnormal scales M={M} {launch}")


# The default kernel and configuration follow the column count, the row-tile
# count and the row length; these three shapes take every branch of that
# choice for every M.
@pytest.mark.parametrize("N,K", [(1024, 4096), (14336, 4096), (4096, 14336)])
@pytest.mark.parametrize("M", list(range(1, 25)))
def test_q8_0_default_launch_every_column_count(dg, dev, orc, N, K, M):
    Wq, Xq = _operands(orc, 3, N, K, M)
    got = _gpu(dg, dev, Wq, Xq, N, K, M)
    assert_close(got, orc.gemv_q8_0_q8_1(Wq, Xq, N, K, M, threads=0), TOL, f"{N}x{K} M={M}")


@pytest.mark.parametrize("M", [2, 16, 24])
def test_q8_0_identical_columns_give_identical_outputs(dg, dev, orc, M):
    N, K = 300, 4096
    Wq, Xq = _operands(orc, 440, N, K, M, same_columns=True)
    got = _gpu(dg, dev, Wq, Xq, N, K, M)
    for m in range(1, M):
        assert np.array_equal(got[m], got[0])


def test_q8_0_worked_blocks_tiled(dg, dev):
    """The hand-worked blocks of tests/golden, each repeated 8 times along K
    (K = 256): y = 8 times the block's value, exact in fp32."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "q8_0_q8_1_worked.json")) as f:
        ex = json.load(f)["dot_examples"]
    for e in ex:
        w = np.frombuffer(bytes.fromhex(e["q8_0_block_hex"].replace(" ", "")), np.uint8)
        x = np.frombuffer(bytes.fromhex(e["q8_1_block_hex"].replace(" ", "")), np.uint8)
        for launch in (None, dict(variant=22)):
            got = _gpu(dg, dev, np.tile(w, 8), np.tile(x, 8), 1, 256, 1, launch=launch)
            assert got[0, 0] == 8 * e["y"], (e["name"], launch)


def test_q8_0_overrides_beyond_kernel_limits_are_rejected(dg, dev):
    import torch
    N, K = 64, 8192
    W = torch.zeros(N * K // 32 * 34, dtype=torch.uint8, device=dev)
    X = torch.zeros(24 * K // 32 * 36, dtype=torch.uint8, device=dev)
    Y = torch.zeros(24 * N, dtype=torch.float32, device=dev)
    for M, launch in ((1, dict(variant=21, block=512)), (2, dict(variant=21)), (1, dict(variant=12)),
                      (4, dict(variant=22, unroll=40421)), (20, dict(variant=22, unroll=11611)),
                      (4, dict(variant=22, block=256)), (1, dict(variant=99)), (5, dict(variant=23)),
                      (1, dict(variant=23, unroll=5))):
        with pytest.raises(dg.DGError) as e:
            dg.dg_gemv_q8_0(W, X, Y, N, K, M, launch=launch)
        assert e.value.status == dg.DG_ERR_ARG, launch
    # rows of one unit (K <= 4096) take at most twelve columns in the units kernel
    with pytest.raises(dg.DGError) as e:
        dg.dg_gemv_q8_0(W, X, Y, N, 4096, 13, launch=dict(variant=23))
    assert e.value.status == dg.DG_ERR_ARG


# ---- the resident-activation matrix-core kernel (variant 24) ----
from tests._parity import RES_CFGS, res_default, res_runs, res_unroll  # noqa: E402

RES_LAUNCHES = [dict(variant=24)] + [dict(variant=24, unroll=res_unroll(*c)) for c in RES_CFGS]


@pytest.mark.parametrize("launch", RES_LAUNCHES, ids=[str(v) for v in RES_LAUNCHES])
@pytest.mark.parametrize("N,K,M", [(37, 4096, 2), (130, 8192, 7), (64, 4096, 16), (200, 4096, 17), (33, 4096, 24),
                                   (700, 4096, 12), (45, 2048, 1), (50, 12288, 8), (77, 14336, 3)])
def test_q8_0_res_matches_oracle(dg, dev, orc, launch, N, K, M):
    Wq, Xq = _operands(orc, 440, N, K, M)
    u = launch.get("unroll", 0) or res_unroll(*res_default(34, N, M, K))
    if not res_runs(34, u // 10000, (u // 100) % 100, M, K):
        with pytest.raises(dg.DGError):
            _gpu(dg, dev, Wq, Xq, N, K, M, launch=launch)
        return
    assert_close(_gpu(dg, dev, Wq, Xq, N, K, M, launch=launch), orc.gemv_q8_0_q8_1(Wq, Xq, N, K, M), TOL,
                 f"res {launch} {N}x{K} M={M}")
