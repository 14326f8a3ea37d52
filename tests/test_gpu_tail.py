"""The greedy-decode tail: bf16 lm-head GEMV into fp32 logits, then argmax (GPU)."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def test_greedy_tail_lm_head_then_argmax(dg, dev, orc):
    import torch
    N, K = 128256, 4096
    Wb = synth.normal_bf16_bits((4, synth.KIND_W, 0, 0), (N, K), 0.02)
    xb = synth.normal_bf16_bits((4, synth.KIND_X, 0, 0), (K,), 1.0)
    W = torch.from_numpy(Wb.view(np.int16)).to(dev).view(torch.bfloat16)
    x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
    logits = torch.empty(N, dtype=torch.float32, device=dev)
    idx = torch.empty(1, dtype=torch.int64, device=dev)
    ws = torch.zeros(dg.dg_argmax_workspace_bytes(1, N), dtype=torch.uint8, device=dev)
    dg.dg_gemv_bf16(W, x, logits)
    dg.dg_argmax_rows(logits.view(1, N), idx, ws=ws)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    tok = int(idx.cpu().numpy()[0])
    # bit-exact against the oracle's argmax of the same logits
    assert tok == int(orc.argmax_rows(lg.reshape(1, N))[0])
    # against the fp64 logits of every row: the workload is seeded, so its top-2
    # gap must exceed twice the largest logit error, and then the token must be
    # the fp64 oracle's
    ref = orc.gemv_bf16(Wb, xb, N=N, K=K, ldw=K, threads=0)
    err = float(np.max(np.abs(lg.astype(np.float64) - ref)))
    order = np.argsort(-ref, kind="stable")
    gap = float(ref[order[0]] - ref[order[1]])
    print(f"[tail] token {tok}, top-2 gap {gap:.4g}, max logit error {err:.3g}")
    assert gap > 2 * err, f"top-2 gap {gap} within twice the logit error {err}"
    assert tok == int(order[0])


def _bf16_operands(dev, key, N, K, ldw=None):
    import torch
    ldw = K if ldw is None else ldw
    Wb = synth.normal_bf16_bits((key, synth.KIND_W, 0, 0), (N, ldw), 0.02)
    xb = synth.normal_bf16_bits((key, synth.KIND_X, 0, 0), (K,), 1.0)
    return Wb, xb


def _fused(dg, dev, Wb, xb, N, K, ldw, store_logits=True):
    import torch
    W = torch.from_numpy(Wb.view(np.int16)).to(dev).view(torch.bfloat16)
    x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.full((N,), float("nan"), dtype=torch.float32, device=dev) if store_logits else None
    idx = torch.full((1,), -1, dtype=torch.int64, device=dev)
    ws = torch.zeros(dg.dg_gemv_bf16_argmax_workspace_bytes(N, K), dtype=torch.uint8, device=dev)
    dg.dg_gemv_bf16_argmax(W, x, idx, y=y, N=N, K=K, ldw=ldw, ws=ws)
    torch.cuda.synchronize()
    return int(idx.cpu().numpy()[0]), (y.cpu().numpy() if store_logits else None)


def _two_calls(dg, dev, Wb, xb, N, K, ldw):
    import torch
    W = torch.from_numpy(Wb.view(np.int16)).to(dev).view(torch.bfloat16)
    x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.empty(N, dtype=torch.float32, device=dev)
    idx = torch.empty(1, dtype=torch.int64, device=dev)
    ws = torch.zeros(dg.dg_argmax_workspace_bytes(1, N), dtype=torch.uint8, device=dev)
    dg.dg_gemv_bf16(W, x, y, N=N, K=K, ldw=ldw)
    dg.dg_argmax_rows(y.view(1, N), idx, ws=ws)
    torch.cuda.synchronize()
    return int(idx.cpu().numpy()[0]), y.cpu().numpy()


@pytest.mark.parametrize("N,K,ldw", [(1, 8, 8), (7, 64, 72), (300, 1000, 1000), (5000, 4104, 4112),
                                     (70000, 512, 512), (128256, 4096, 4096)])
def test_fused_tail_equals_gemv_then_argmax(dg, dev, orc, N, K, ldw):
    """The fused call returns the same logits, bit for bit, and the token that
    the two-call path and the oracle's argmax of those logits give."""
    Wb, xb = _bf16_operands(dev, 800 + N % 97, N, K, ldw)
    tok, y = _fused(dg, dev, Wb, xb, N, K, ldw)
    tok2, y2 = _two_calls(dg, dev, Wb, xb, N, K, ldw)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    assert tok == tok2 == int(orc.argmax_rows(y.reshape(1, N))[0])
    tok3, _ = _fused(dg, dev, Wb, xb, N, K, ldw, store_logits=False)
    assert tok3 == tok


def test_fused_tail_ties_and_nan(dg, dev, orc):
    """Duplicated weight rows give bit-identical logits: the lowest index wins;
    a NaN weight makes its logit NaN, which wins, the first NaN first."""
    N, K = 9000, 256
    Wb, xb = _bf16_operands(dev, 810, N, K)
    Wb[[0, N - 1, 4321]] = 0x3F80              # rows of 1.0: the largest logits, tied
    xb = xb & np.uint16(0x7FFF)                # positive activations (sign bit cleared)
    tok, y = _fused(dg, dev, Wb, xb, N, K, K)
    assert y[0] == y[N - 1] == y[4321] and tok == 0
    Wb2 = Wb.copy()
    Wb2[[7000, 8000], 3] = 0x7FC0              # bfloat16 NaN
    tok, y = _fused(dg, dev, Wb2, xb, N, K, K)
    assert np.isnan(y[7000]) and tok == 7000 == int(orc.argmax_rows(y.reshape(1, N))[0])


def test_fused_tail_workspace_contents_do_not_matter(dg, dev, orc):
    """One garbage-filled workspace across calls of different sizes."""
    import torch
    ws = torch.full((dg.dg_gemv_bf16_argmax_workspace_bytes(128256, 4096),), 0xC3, dtype=torch.uint8, device=dev)
    idx = torch.empty(1, dtype=torch.int64, device=dev)
    for i, (N, K, scale) in enumerate([(50000, 512, 1.0), (3000, 256, 0.01), (128256, 4096, 0.001), (10, 64, 0.5)]):
        Wb = synth.normal_bf16_bits((820 + i, synth.KIND_W, 0, 0), (N, K), 0.02 * scale)
        xb = synth.normal_bf16_bits((820 + i, synth.KIND_X, 0, 0), (K,), 1.0)
        W = torch.from_numpy(Wb.view(np.int16)).to(dev).view(torch.bfloat16)
        x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
        y = torch.empty(N, dtype=torch.float32, device=dev)
        dg.dg_gemv_bf16_argmax(W, x, idx, y=y, ws=ws)
        torch.cuda.synchronize()
        assert int(idx.cpu().numpy()[0]) == int(orc.argmax_rows(y.cpu().numpy().reshape(1, N))[0]), (N, K)
