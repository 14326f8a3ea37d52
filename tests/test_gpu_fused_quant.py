"""dg_gemv_q4_0_f32: Q8_1 quantisation and the Q4_0 GEMV from float32
activations in one call (GPU).

The quantised columns it stores must equal the oracle's quantiser byte for
byte, and every row of Y must match the oracle's GEMV over those bytes, in
the default form (the quantiser's launch, then the GEMV's) and in the
one-launch form for one column (variant 13: the GEMV's workgroups quantise
the column themselves).
"""
import numpy as np
import pytest

import synth
from tests._parity import assert_close

pytestmark = pytest.mark.gpu

TOL = 1e-3


def _run(dg, dev, orc, cfg, N, K, M, store=True, scale=1.0, launch=None):
    import torch
    w = synth.normal_f32((cfg, synth.KIND_W, 0, 0), (N, K))
    Wq = orc.quantize_q4_0(w, threads=0)
    x = np.stack([synth.normal_f32((cfg, synth.KIND_X, 0, m), (K,)) for m in range(M)]) * np.float32(scale)
    Xq_ref = orc.quantize_q8_1(x)
    Wd = torch.from_numpy(np.ascontiguousarray(Wq).reshape(-1)).to(dev)
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    Y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    Xq = torch.full((M * (K // 32) * 36,), 0xA5, dtype=torch.uint8, device=dev) if store else None
    dg.dg_gemv_q4_0_f32(Wd, xd, Y, N, K, M, Xq=Xq, launch=launch)
    torch.cuda.synchronize()
    if store:
        assert np.array_equal(Xq.cpu().numpy(), Xq_ref.reshape(-1)), "Q8_1 bytes differ from the oracle's"
    ref = orc.gemv_q4_0_q8_1(Wq, Xq_ref, N, K, M, threads=0)
    assert_close(Y.cpu().numpy().astype(np.float64), ref, TOL, f"{N}x{K} M={M}")


ONE_LAUNCH = [None, dict(variant=13), dict(variant=13, grid=3, block=64), dict(variant=13, grid=768, unroll=3),
              dict(variant=13, grid=1, block=128, unroll=4)]


@pytest.mark.parametrize("launch", ONE_LAUNCH, ids=[str(v) for v in ONE_LAUNCH])
@pytest.mark.parametrize("N,K", [(1, 256), (7, 4096), (301, 8192), (70, 4352), (33, 16384), (28672, 8192),
                                 (4096, 4096)])
def test_one_column(dg, dev, orc, N, K, launch):
    _run(dg, dev, orc, 960, N, K, 1, launch=launch)


def test_one_launch_without_storing(dg, dev, orc):
    _run(dg, dev, orc, 961, 300, 4096, 1, store=False, launch=dict(variant=13))


def test_one_launch_rejects_what_it_cannot_take(dg, dev):
    import torch
    W = torch.zeros(64 * 24576 // 32 * 18, dtype=torch.uint8, device=dev)
    x = torch.zeros(2 * 24576, dtype=torch.float32, device=dev)
    Y = torch.zeros(2 * 64, dtype=torch.float32, device=dev)
    Xq = torch.zeros(2 * 24576 // 32 * 36, dtype=torch.uint8, device=dev)
    for N, K, M, launch in ((64, 4096, 2, dict(variant=13)), (64, 24576, 1, dict(variant=13)),
                            (64, 4096, 1, dict(variant=14)), (64, 4096, 1, dict(grid=4)),
                            (64, 4096, 1, dict(variant=13, block=512))):
        with pytest.raises(dg.DGError) as e:
            dg.dg_gemv_q4_0_f32(W, x, Y, N, K, M, Xq=Xq, launch=launch)
        assert e.value.status == dg.DG_ERR_ARG, (N, K, M, launch)


@pytest.mark.parametrize("N,K,M", [(300, 4096, 2), (77, 12288, 5), (4096, 14336, 24), (14336, 4096, 17)])
def test_several_columns(dg, dev, orc, N, K, M):
    _run(dg, dev, orc, 962, N, K, M)


def test_one_column_long_rows(dg, dev, orc):
    _run(dg, dev, orc, 963, 50, 24576, 1)


@pytest.mark.parametrize("launch", [None, dict(variant=13)])
@pytest.mark.parametrize("scale", [1e-30, 1e6])
def test_extreme_scales(dg, dev, orc, scale, launch):
    """Activation scales far below and above binary16's normal range, as the
    stored bytes (binary16 d and s, subnormal, zero or infinite) demand."""
    _run(dg, dev, orc, 964, 129, 2048, 1, scale=scale, launch=launch)


@pytest.mark.parametrize("launch", [None, dict(variant=13)])
def test_zero_activations(dg, dev, orc, launch):
    import torch
    N, K = 64, 2048
    Wq = orc.quantize_q4_0(synth.normal_f32((965, synth.KIND_W, 0, 0), (N, K)))
    x = np.zeros((1, K), dtype=np.float32)
    Y = torch.full((1, N), float("nan"), dtype=torch.float32, device=dev)
    Xq = torch.full((K // 32 * 36,), 0xA5, dtype=torch.uint8, device=dev)
    dg.dg_gemv_q4_0_f32(torch.from_numpy(Wq.reshape(-1)).to(dev), torch.from_numpy(x).to(dev), Y, N, K, 1, Xq=Xq,
                        launch=launch)
    torch.cuda.synchronize()
    assert np.array_equal(Xq.cpu().numpy(), orc.quantize_q8_1(x).reshape(-1))
    assert np.all(Y.cpu().numpy() == 0.0)
