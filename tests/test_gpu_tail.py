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
    # against the fp64 logits: the same token whenever the top-2 gap exceeds twice
    # the largest logit error seen on the candidate rows
    top = np.argsort(-lg)[:16]
    ref_top = orc.gemv_bf16(Wb[top].copy(), xb, N=len(top), K=K, ldw=K)
    err = float(np.max(np.abs(lg[top] - ref_top)))
    order = np.argsort(-ref_top)
    gap = float(ref_top[order[0]] - ref_top[order[1]])
    print(f"[tail] token {tok}, top-2 gap {gap:.4g}, max logit error {err:.3g}")
    if gap > 2 * err:
        assert tok == int(top[order[0]])
