"""Parity of dg_gemv_f16 / dg_gemv_bf16 with the fp64 oracle (GPU)."""
import numpy as np
import pytest

import synth
from tests._parity import assert_close

pytestmark = pytest.mark.gpu

TOL = 2e-3   # max floored relative error vs the fp64 oracle


def _upload(bits, dtype, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(dtype)


def _run(dg, dev, fmt, Wb, xb, N, K, ldw, launch=None):
    import torch
    wd = torch.float16 if fmt == "f16" else torch.bfloat16
    W = _upload(Wb, wd, dev)
    x = _upload(xb, wd, dev)
    y = torch.full((max(N, 1),), float("nan"), dtype=torch.float16 if fmt == "f16" else torch.float32, device=dev)
    fn = dg.dg_gemv_f16 if fmt == "f16" else dg.dg_gemv_bf16
    fn(W, x, y, N=N, K=K, ldw=ldw, launch=launch)
    torch.cuda.synchronize()
    return y[:N].float().cpu().numpy().astype(np.float64)


def _ref(orc, fmt, Wb, xb, N, K, ldw):
    fn = orc.gemv_f16 if fmt == "f16" else orc.gemv_bf16
    return fn(Wb, xb, N=N, K=K, ldw=ldw)


def _inputs(fmt, cfg, N, K, ldw=None, copy=0):
    ldw = K if ldw is None else ldw
    gen = synth.normal_f16_bits if fmt == "f16" else synth.normal_bf16_bits
    Wb = gen((cfg, synth.KIND_W, copy, 0), (N, ldw), 0.02)
    xb = gen((cfg, synth.KIND_X, copy, 0), (K,), 1.0)
    return Wb, xb


SHAPES = [(1, 8), (3, 24), (5, 520), (67, 1000), (130, 4096), (257, 4104), (64, 14336), (1000, 512)]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("N,K", SHAPES)
def test_dense_small_shapes(dg, dev, orc, fmt, N, K):
    Wb, xb = _inputs(fmt, 100, N, K)
    got = _run(dg, dev, fmt, Wb, xb, N, K, K)
    assert_close(got, _ref(orc, fmt, Wb, xb, N, K, K), TOL, f"{fmt} {N}x{K}")


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_dense_leading_dimension(dg, dev, orc, fmt):
    N, K, ldw = 33, 776, 800
    Wb, xb = _inputs(fmt, 101, N, K, ldw)
    Wb = Wb.copy()
    Wb[:, K:] = 0x7E00 if fmt == "f16" else 0x7FC0     # NaN padding must never be read
    got = _run(dg, dev, fmt, Wb, xb, N, K, ldw)
    assert np.all(np.isfinite(got))
    assert_close(got, _ref(orc, fmt, Wb, xb, N, K, ldw), TOL, "ldw")


VARIANTS = [
    dict(variant=1, unroll=1), dict(variant=1, unroll=2), dict(variant=1, unroll=4), dict(variant=1, unroll=8),
    dict(variant=2), dict(variant=3), dict(variant=4),
    dict(variant=1, grid=7, block=64), dict(variant=1, grid=3, block=1024), dict(variant=2, grid=5, block=128),
    dict(variant=1, unroll=102), dict(variant=1, unroll=304), dict(variant=1, unroll=108, block=128),
    dict(variant=1, unroll=301, grid=5, block=512), dict(variant=1, unroll=304, grid=2, block=1024),
]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("launch", VARIANTS, ids=[str(v) for v in VARIANTS])
def test_dense_variants_and_launch_shapes(dg, dev, orc, fmt, launch):
    N, K = 300, 4096 if launch.get("variant") == 2 else 2056
    Wb, xb = _inputs(fmt, 102, N, K)
    got = _run(dg, dev, fmt, Wb, xb, N, K, K, launch=launch)
    assert_close(got, _ref(orc, fmt, Wb, xb, N, K, K), TOL, str(launch))


def test_dense_invalid_overrides_are_rejected(dg, dev):
    import torch
    W = torch.zeros((8, 64), dtype=torch.float16, device=dev)
    x = torch.zeros(64, dtype=torch.float16, device=dev)
    y = torch.zeros(8, dtype=torch.float16, device=dev)
    for launch in (dict(variant=1, unroll=204), dict(variant=1, unroll=3), dict(variant=1, unroll=300, block=64),
                   dict(variant=2, unroll=16), dict(variant=9)):
        with pytest.raises(dg.DGError) as e:
            dg.dg_gemv_f16(W, x, y, launch=launch)
        assert e.value.status == dg.DG_ERR_ARG, launch


def test_dense_f16_full_size_all_rows(dg, dev, orc):
    """The fp16 decode shape, 4096 x 4096, every row against the oracle, plus the
    fp16 output rounding: within one binary16 ulp of the rounded oracle value."""
    N = K = 4096
    Wb, xb = _inputs("f16", 0, N, K)
    got = _run(dg, dev, "f16", Wb, xb, N, K, K)
    ref = _ref(orc, "f16", Wb, xb, N, K, K)
    assert_close(got, ref, TOL, "f16 4096x4096")
    ref16 = ref.astype(np.float16).view(np.int16).astype(np.int64)
    got16 = got.astype(np.float16).view(np.int16).astype(np.int64)
    assert np.max(np.abs(ref16 - got16)) <= 1


@pytest.mark.parametrize("N,K", [(4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336)])
def test_dense_bf16_decoder_layer_shapes(dg, dev, orc, N, K):
    Wb, xb = _inputs("bf16", 1, N, K)
    got = _run(dg, dev, "bf16", Wb, xb, N, K, K)
    assert_close(got, orc.gemv_bf16(Wb, xb, N=N, K=K, ldw=K, threads=0), TOL, f"bf16 {N}x{K}")


def test_dense_bf16_lm_head_all_rows(dg, dev, orc):
    N, K = 128256, 4096
    Wb, xb = _inputs("bf16", 4, N, K)
    got = _run(dg, dev, "bf16", Wb, xb, N, K, K)
    assert_close(got, orc.gemv_bf16(Wb, xb, N=N, K=K, ldw=K, threads=0), TOL, "lm-head all rows")


def test_dense_empty_and_k_zero(dg, dev):
    import torch
    W = torch.zeros((4, 8), dtype=torch.float16, device=dev)
    x = torch.zeros(8, dtype=torch.float16, device=dev)
    y = torch.full((4,), 7.0, dtype=torch.float16, device=dev)
    dg.dg_gemv_f16(W, x, y, N=0, K=8, ldw=8)            # nothing launched, nothing written
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
    dg.dg_gemv_f16(W, x, y, N=4, K=0, ldw=8)            # empty sums
    yb = torch.full((4,), 7.0, dtype=torch.float32, device=dev)
    dg.dg_gemv_bf16(W.view(torch.bfloat16), x.view(torch.bfloat16), yb, N=4, K=0, ldw=8)
    torch.cuda.synchronize()
    assert torch.all(y == 0) and torch.all(yb == 0)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_dense_invariants(dg, dev, fmt):
    """One-hot x selects a column exactly; scaling x by 2 scales y exactly;
    permuting rows permutes y exactly; two calls give identical bits."""
    N, K = 512, 4096
    Wb, xb = _inputs(fmt, 103, N, K)
    one = np.uint16(0x3C00 if fmt == "f16" else 0x3F80)
    for k in (0, 777, K - 1):
        e = np.zeros(K, dtype=np.uint16)
        e[k] = one
        got = _run(dg, dev, fmt, Wb, e, N, K, K)
        col = Wb[:, k].view(np.float16).astype(np.float64) if fmt == "f16" else \
            (Wb[:, k].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert np.array_equal(got, col)
    two = (xb.view(np.float16) * np.float16(2)).view(np.uint16) if fmt == "f16" else \
        synth.to_bf16_bits((xb.astype(np.uint32) << 16).view(np.float32) * np.float32(2))   # exact
    y1 = _run(dg, dev, fmt, Wb, xb, N, K, K)
    y2 = _run(dg, dev, fmt, Wb, two, N, K, K)
    assert np.array_equal(y2, 2 * y1)
    perm = np.random.default_rng(0).permutation(N)
    yp = _run(dg, dev, fmt, Wb[perm].copy(), xb, N, K, K)
    assert np.array_equal(yp, y1[perm])
    assert np.array_equal(_run(dg, dev, fmt, Wb, xb, N, K, K), y1)


def test_dense_f16_subnormal_weights_are_not_flushed(dg, dev):
    K = 1024
    W = np.arange(1, K + 1, dtype=np.uint32).astype(np.uint16).reshape(1, K)   # every positive subnormal
    x = np.full(K, 0x3C00, dtype=np.uint16)
    got = _run(dg, dev, "f16", W, x, 1, K, K)
    exact = sum(range(1, K + 1)) * 2.0 ** -24                                    # 31.25 ... in fp16 range
    assert abs(got[0] - exact) <= exact * 2 ** -10
