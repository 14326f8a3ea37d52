"""Parity of dg_argmax_rows with the oracle: bit-exact indices (GPU)."""
import json
import math
import os

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _gpu_argmax(dg, dev, x, C=None, ld=None):
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    R = x.shape[0]
    C = x.shape[1] if C is None else C
    ld = x.shape[1] if ld is None else ld
    t = torch.from_numpy(x).to(dev)
    idx = torch.full((R,), -1, dtype=torch.int64, device=dev)
    ws = torch.zeros(max(1, dg.dg_argmax_workspace_bytes(R, C)), dtype=torch.uint8, device=dev)
    dg.dg_argmax_rows(t, idx, R=R, C=C, ld=ld, ws=ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy()


def _parse(v):
    return {"-0": -0.0, "+0": 0.0, "nan": math.nan, "inf": math.inf, "-inf": -math.inf}.get(v, v) \
        if isinstance(v, str) else float(v)


def test_argmax_hand_rows(dg, dev):
    with open(os.path.join(os.path.dirname(__file__), "golden", "argmax_rows.json")) as f:
        rows = json.load(f)["rows"]
    for r in rows:
        x = np.array([[_parse(v) for v in r["x"]]], dtype=np.float32)
        assert _gpu_argmax(dg, dev, x)[0] == r["idx"], r


@pytest.mark.parametrize("R,C", [(1, 1), (1, 5), (3, 1023), (2, 1024), (5, 4097), (8, 32000), (1, 50257),
                                 (32, 1000), (7, 65537), (1, 262144), (300, 3)])
def test_argmax_random_with_heavy_ties(dg, dev, orc, R, C):
    g = np.random.default_rng(R * 100003 + C)
    x = g.integers(0, 5, size=(R, C)).astype(np.float32)   # many equal maxima per row
    assert np.array_equal(_gpu_argmax(dg, dev, x), orc.argmax_rows(x))


def test_argmax_leading_dimension_and_unaligned_rows(dg, dev, orc):
    g = np.random.default_rng(5)
    R, C, ld = 9, 3001, 3003                                  # ld % 4 != 0: scalar path
    x = g.integers(0, 3, size=(R, ld)).astype(np.float32)
    x[:, C:] = 1e30
    assert np.array_equal(_gpu_argmax(dg, dev, x, C=C, ld=ld), orc.argmax_rows(x, C=C, ld=ld))
    R, C, ld = 6, 4000, 4096                                  # aligned rows, padding ignored
    x = g.integers(0, 3, size=(R, ld)).astype(np.float32)
    x[:, C:] = 1e30
    assert np.array_equal(_gpu_argmax(dg, dev, x, C=C, ld=ld), orc.argmax_rows(x, C=C, ld=ld))


def test_argmax_special_values(dg, dev, orc):
    C = 70000
    x = np.zeros((6, C), dtype=np.float32)
    x[0, :] = -0.0; x[0, 40000] = 0.0                         # -0 ties +0: index 0
    x[1, 5] = np.nan; x[1, 60000] = np.nan; x[1, 7] = np.inf  # first NaN
    x[2, :] = -np.inf                                          # all -inf: index 0
    x[3, 69999] = 1.0; x[3, 35000] = 1.0                       # duplicate in another chunk
    x[4, :] = np.float32(3.0); x[4, 0] = np.float32(2.0)       # max first at 1
    x[5, 12345] = np.inf; x[5, 54321] = np.inf
    got = _gpu_argmax(dg, dev, x)
    assert np.array_equal(got, orc.argmax_rows(x))
    assert got.tolist() == [0, 5, 0, 35000, 1, 12345]


@pytest.mark.parametrize("R,C", [(1, 128000), (32, 128000), (64, 1000000), (1, 128256)])
def test_argmax_workload_shapes_with_planted_ties(dg, dev, orc, R, C):
    x, planted = synth.argmax_logits(5, R, C)
    got = _gpu_argmax(dg, dev, x)
    ref = orc.argmax_rows(x)
    assert np.array_equal(got, ref)
    for r, pos in planted.items():
        assert got[r] == pos[0]


def test_argmax_workspace_contract(dg, dev):
    import torch
    x = torch.zeros((4, 5000), dtype=torch.float32, device=dev)
    idx = torch.zeros(4, dtype=torch.int64, device=dev)
    need = dg.dg_argmax_workspace_bytes(4, 5000)
    small = torch.empty(need - 8, dtype=torch.uint8, device=dev)
    with pytest.raises(dg.DGError) as e:
        dg.dg_argmax_rows(x, idx, ws=small)
    assert e.value.status == dg.DG_ERR_WORKSPACE


def test_argmax_workspace_contents_do_not_matter_and_it_is_reusable(dg, dev, orc):
    """One workspace, filled with garbage before the first call, serves calls of
    different shapes in a row."""
    import torch
    shapes = [(3, 70000), (1, 128000), (40, 5000), (2, 4), (7, 33333), (1, 1)]
    size = max(dg.dg_argmax_workspace_bytes(R, C) for R, C in shapes)
    ws = torch.full((size,), 0xAB, dtype=torch.uint8, device=dev)
    for i, (R, C) in enumerate(shapes * 2):
        x, _ = synth.argmax_logits(500 + i, R, C)
        idx = torch.full((R,), -1, dtype=torch.int64, device=dev)
        dg.dg_argmax_rows(torch.from_numpy(x).to(dev), idx, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), orc.argmax_rows(x)), (R, C)
