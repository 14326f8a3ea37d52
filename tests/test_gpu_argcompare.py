"""Parity of dg_argcompare_rows (argmax / argmin of float32, binary16 and
bfloat16 rows) with the oracle: bit-exact indices (GPU)."""
import json
import math
import os

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(x32, dtype):
    """float32 values -> the input array of that dtype (16-bit types as bit patterns)."""
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f16":
        return synth.to_f16_bits(x32)
    return synth.to_bf16_bits(x32)


def _gpu(dg, dev, a, dtype, op, C=None, ld=None):
    import torch
    R = a.shape[0]
    C = a.shape[1] if C is None else C
    ld = a.shape[1] if ld is None else ld
    if dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
        t = t.view(torch.float16 if dtype == "f16" else torch.bfloat16)
    idx = torch.full((R,), -1, dtype=torch.int64, device=dev)
    ws = torch.full((max(1, dg.dg_argmax_workspace_bytes(R, C)),), 0x5A, dtype=torch.uint8, device=dev)
    dg.dg_argcompare_rows(t, idx, op=op, R=R, C=C, ld=ld, ws=ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy()


def _parse(v):
    return {"-0": -0.0, "+0": 0.0, "nan": math.nan, "inf": math.inf, "-inf": -math.inf}.get(v, v) \
        if isinstance(v, str) else float(v)


def test_argcompare_hand_rows(dg, dev):
    with open(os.path.join(GOLDEN, "argcompare_rows.json")) as f:
        g = json.load(f)
    for r in g["f32_min_rows"]:
        x = np.array([[_parse(v) for v in r["x"]]], dtype=np.float32)
        assert _gpu(dg, dev, x, "f32", "min")[0] == r["idx"], r
    for r in g["bits_rows"]:
        bits = np.array([[int(b, 16) for b in r["bits"]]], dtype=np.uint16)
        assert _gpu(dg, dev, bits, r["dtype"], r["op"])[0] == r["idx"], r


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("op", ["max", "min"])
@pytest.mark.parametrize("R,C,ld", [(1, 1, 1), (3, 7, 7), (5, 1000, 1003), (2, 70001, 70008), (4, 128000, 128000),
                                    (33, 4104, 4112), (1, 16384 * 3 + 8, 16384 * 3 + 8)])
def test_argcompare_matches_oracle(dg, dev, orc, dtype, op, R, C, ld):
    x, _ = synth.argmax_logits(600 + R, R, ld)
    if op == "min":
        x = -x                                     # the planted duplicate maxima become duplicate minima
    a = _bits(x, dtype)
    got = _gpu(dg, dev, a, dtype, op, C=C, ld=ld)
    assert np.array_equal(got, orc.argcompare_rows(a, dtype, op, C=C, ld=ld))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("op", ["max", "min"])
def test_argcompare_heavy_ties_nan_and_signed_zero(dg, dev, orc, dtype, op):
    g = np.random.default_rng(61)
    R, C = 48, 5000
    x = (g.integers(0, 3, size=(R, C)) - 1).astype(np.float32)
    x[3, 4000] = np.nan
    x[4, [17, 4999]] = np.nan
    x[5, :] = -0.0
    x[5, 2500] = 0.0
    x[6, :] = 1.0
    x[6, [0, C - 1]] = 2.0 if op == "max" else 0.0
    a = _bits(x, dtype)
    assert np.array_equal(_gpu(dg, dev, a, dtype, op), orc.argcompare_rows(a, dtype, op))


@pytest.mark.parametrize("dtype,op,R,C", [("bf16", "max", 1, 128000), ("bf16", "max", 32, 128000),
                                          ("f16", "min", 32, 128000), ("f32", "min", 64, 1000000)])
def test_argcompare_census_shapes(dg, dev, orc, dtype, op, R, C):
    """The discussion's workloads: a 128K vocabulary row, 32 of them, and 64
    rows of a 1M-item output layer."""
    x, planted = synth.argmax_logits(700 + R, R, C)
    if op == "min":
        x = -x
    a = _bits(x, dtype)
    got = _gpu(dg, dev, a, dtype, op)
    assert np.array_equal(got, orc.argcompare_rows(a, dtype, op))
    for r, pos in planted.items():
        assert got[r] == pos[0]


def test_argmax_rows_is_argcompare_f32_max(dg, dev):
    import torch
    x, _ = synth.argmax_logits(710, 6, 33333)
    t = torch.from_numpy(x).to(dev)
    ws = torch.zeros(dg.dg_argmax_workspace_bytes(6, 33333), dtype=torch.uint8, device=dev)
    a = torch.empty(6, dtype=torch.int64, device=dev)
    dg.dg_argmax_rows(t, a, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy(), _gpu(dg, dev, x, "f32", "max"))
