"""The GPU quantisers produce exactly the oracle's bytes (GPU)."""
import json
import os

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _gpu_q(dg, dev, a, kind):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    R, K = a.shape
    size = {"q8_1": 36, "q4_0": 18, "q8_0": 34}[kind]
    out = torch.zeros(R * (K // 32) * size, dtype=torch.uint8, device=dev)
    {"q8_1": dg.dg_quantize_q8_1, "q4_0": dg.dg_quantize_q4_0, "q8_0": dg.dg_quantize_q8_0}[kind](t, out, R, K)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _tricky(K):
    """Rows that exercise ties, zeros, sign, half-way codes and tiny scales."""
    j = np.arange(32, dtype=np.float32)
    rows = []
    rows.append(np.tile((j - 16) / 4, K // 32))                       # half-way Q4_0 codes
    rows.append(np.tile((16 - j) / 4, K // 32))
    z = np.zeros(K, np.float32); rows.append(z)                         # all-zero blocks
    t = np.zeros(K, np.float32); t[0::32] = -2; t[1::32] = 2; rows.append(t)  # magnitude ties
    rows.append(np.tile((j - 15.5) * 1e-6, K // 32))                    # tiny scales (binary16 subnormal d)
    h = np.tile(np.float32(127) * (j - 16) / 16 + 0.5, K // 32); rows.append(h)   # Q8_1 half-way cases
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("kind", ["q8_1", "q4_0", "q8_0"])
@pytest.mark.parametrize("R,K", [(1, 32), (3, 256), (17, 4096), (4, 14336)])
def test_quantiser_bytes_match_oracle(dg, dev, orc, kind, R, K):
    a = synth.normal_f32((300, synth.KIND_X, R, K), (R, K))
    a = np.concatenate([a, _tricky(K)])
    ref = {"q8_1": orc.quantize_q8_1, "q4_0": orc.quantize_q4_0, "q8_0": orc.quantize_q8_0}[kind](a).reshape(-1)
    got = _gpu_q(dg, dev, a, kind)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"


def test_quantiser_worked_blocks(dg, dev):
    with open(os.path.join(os.path.dirname(__file__), "golden", "q4_0_q8_1_worked.json")) as f:
        g = json.load(f)
    for e in g["q8_1_quantiser_examples"]:
        x = np.array(e["x"], dtype=np.float32).reshape(1, 32)
        assert bytes(_gpu_q(dg, dev, x, "q8_1")) == bytes.fromhex(e["block_hex"].replace(" ", "")), e["name"]
    j = np.arange(32)
    tie = np.zeros(32); tie[:2] = [-2, 2]
    xs = {"(j-16)/4 for j in 0..31": (j - 16) / 4, "(16-j)/4 for j in 0..31": (16 - j) / 4,
          "0 for j in 0..31": np.zeros(32), "[-2, 2, 0 x 30]": tie}
    for e in g["q4_0_quantiser_examples"]:
        x = xs[e["x"]].astype(np.float32).reshape(1, 32)
        assert bytes(_gpu_q(dg, dev, x, "q4_0")) == bytes.fromhex(e["block_hex"].replace(" ", "")), e["name"]

    with open(os.path.join(os.path.dirname(__file__), "golden", "q8_0_q8_1_worked.json")) as f:
        g8 = json.load(f)
    for e in g8["q8_0_quantiser_examples"]:
        x = np.array(e["x"], dtype=np.float32).reshape(1, 32)
        assert bytes(_gpu_q(dg, dev, x, "q8_0")) == bytes.fromhex(e["block_hex"].replace(" ", "")), e["name"]
