"""Library launches on a side stream and inside a captured HIP graph: every
replay (with eager work between replays) equals the eager result bit for bit (GPU)."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def test_side_stream_ordering(dg, dev):
    import torch
    N, K = 2048, 4096
    W = synth.gpu_normal((700, 0, 0, 0), (N, K), 0.02, torch.float16)
    x = synth.gpu_normal((700, 1, 0, 0), (K,), 1.0, torch.float16)
    y0 = torch.empty(N, dtype=torch.float16, device=dev)
    dg.dg_gemv_f16(W, x, y0)
    s = torch.cuda.Stream()
    y1 = torch.empty_like(y0)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        x2 = x * 2                                   # produced on the side stream
        dg.dg_gemv_f16(W, x2, y1)                    # must see x2 (same stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(y1.float(), (y0.float() * 2))


def test_graph_replays_match_eager(dg, dev):
    import torch
    N, K, Nq, Kq = 4096, 4096, 4096, 8192
    W = synth.gpu_normal((701, 0, 0, 0), (N, K), 0.02, torch.float16)
    x = synth.gpu_normal((701, 1, 0, 0), (K,), 1.0, torch.float16)
    w32 = synth.gpu_normal((701, 0, 1, 0), (Nq, Kq), 1.0, torch.float32)
    Wq = torch.empty(Nq * Kq // 32 * 18, dtype=torch.uint8, device=dev)
    dg.dg_quantize_q4_0(w32, Wq, Nq, Kq)
    xf = synth.gpu_normal((701, 1, 1, 0), (1, Kq), 1.0, torch.float32)
    Xq = torch.empty(Kq // 32 * 36, dtype=torch.uint8, device=dev)
    y = torch.empty(N, dtype=torch.float16, device=dev)
    yq = torch.empty(Nq, dtype=torch.float32, device=dev)
    idx = torch.empty(1, dtype=torch.int64, device=dev)
    ws = torch.zeros(dg.dg_argmax_workspace_bytes(1, Nq), dtype=torch.uint8, device=dev)

    def step():
        dg.dg_quantize_q8_1(xf, Xq, 1, Kq)
        dg.dg_gemv_f16(W, x, y)
        dg.dg_gemv_q4_0(Wq, Xq, yq, Nq, Kq, 1)
        dg.dg_argmax_rows(yq.view(1, Nq), idx, ws=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        # new inputs written eagerly between replays
        x.copy_(synth.gpu_normal((702, 1, rep, 0), (K,), 1.0, torch.float16))
        xf.copy_(synth.gpu_normal((702, 1, rep, 1), (1, Kq), 1.0, torch.float32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (y.clone(), yq.clone(), idx.clone(), Xq.clone())
        y.fill_(0); yq.fill_(0); idx.fill_(-1); Xq.fill_(0)
        step()
        torch.cuda.synchronize()
        assert torch.equal(got[3], Xq)
        assert torch.equal(got[0], y) and torch.equal(got[1], yq) and torch.equal(got[2], idx)
