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


def test_graph_replays_of_every_entry_point(dg, dev):
    """One captured graph holding a call of every computing entry point (the
    small-batch matrix-core and units paths of both quantised formats, the
    tiled Q4_0 path with and without K split over workgroups, NF4,
    the fp32-activation call, ArgCompare, the greedy tail and the
    no-allocation argmax, whose callers are exactly those that capture
    graphs): four replays with new inputs written eagerly in between, each
    equal bit for bit to an eager run of the same calls."""
    import torch
    K = 4096
    w32 = synth.gpu_normal((703, 0, 0, 0), (2048, K), 1.0, torch.float32)
    Wq4 = torch.empty(2048 * K // 32 * 18, dtype=torch.uint8, device=dev)
    Wq8 = torch.empty(2048 * K // 32 * 34, dtype=torch.uint8, device=dev)
    dg.dg_quantize_q4_0(w32, Wq4, 2048, K)
    dg.dg_quantize_q8_0(w32, Wq8, 2048, K)
    table = torch.from_numpy(np.asarray(synth.nf4_table(), np.float32)).to(dev)
    codes = torch.empty(2048 * K // 2, dtype=torch.uint8, device=dev)
    absmax = torch.empty(2048 * K // 64, dtype=torch.float32, device=dev)
    dg.dg_quantize_nf4(w32, codes, absmax, table, 2048, K, 64)
    Wb = synth.gpu_normal((703, 0, 1, 0), (20000, K), 0.02, torch.bfloat16)
    xf = synth.gpu_normal((703, 1, 0, 0), (16, K), 1.0, torch.float32)
    Xq = torch.empty(16 * K // 32 * 36, dtype=torch.uint8, device=dev)
    Xq1 = torch.empty(K // 32 * 36, dtype=torch.uint8, device=dev)
    xb = torch.empty(K, dtype=torch.bfloat16, device=dev)
    outs = dict(y16=torch.empty(16 * 2048, dtype=torch.float32, device=dev),
                y8=torch.empty(8 * 2048, dtype=torch.float32, device=dev),
                q8_16=torch.empty(16 * 2048, dtype=torch.float32, device=dev),
                q8_3=torch.empty(3 * 2048, dtype=torch.float32, device=dev),
                nf4=torch.empty(2048, dtype=torch.float32, device=dev),
                f32=torch.empty(2048, dtype=torch.float32, device=dev),
                logits=torch.empty(20000, dtype=torch.float32, device=dev),
                tok=torch.empty(1, dtype=torch.int64, device=dev),
                amin=torch.empty(16, dtype=torch.int64, device=dev),
                anoalloc=torch.empty(16, dtype=torch.int64, device=dev))
    Wt4 = torch.empty(dg.dg_q4_0_tiles_bytes(2048, K), dtype=torch.uint8, device=dev)
    dg.dg_repack_q4_0_tiles(Wq4, Wt4, 2048, K)
    ws_tiles = torch.zeros(1 << 22, dtype=torch.uint8, device=dev)
    Xq24 = torch.empty(24 * K // 32 * 36, dtype=torch.uint8, device=dev)
    outs.update(t16=torch.empty(16 * 2048, dtype=torch.float32, device=dev),
                t24=torch.empty(24 * 2048, dtype=torch.float32, device=dev))
    ws_tail = torch.zeros(dg.dg_gemv_bf16_argmax_workspace_bytes(20000, K), dtype=torch.uint8, device=dev)
    ws_arg = torch.zeros(dg.dg_argmax_workspace_bytes(16, K), dtype=torch.uint8, device=dev)

    def step():
        dg.dg_quantize_q8_1(xf, Xq, 16, K)
        xb.copy_(xf[0].to(torch.bfloat16))
        dg.dg_gemv_q4_0(Wq4, Xq, outs["y16"], 2048, K, 16)     # matrix cores
        dg.dg_gemv_q4_0(Wq4, Xq, outs["y8"], 2048, K, 8)       # matrix cores, eight columns
        dg.dg_gemv_q4_0_tiles(Wt4, Xq, outs["t16"], 2048, K, 16, ws=ws_tiles)    # tiled copy
        dg.dg_quantize_q8_1(xf.repeat(2, 1)[:24].contiguous(), Xq24, 24, K)
        dg.dg_gemv_q4_0_tiles(Wt4, Xq24, outs["t24"], 2048, K, 24, ws=ws_tiles,      # K split: tickets
                              launch=dict(unroll=2 * 1000000 + 2 * 10000 + 4 * 100 + 2))
        dg.dg_gemv_q8_0(Wq8, Xq, outs["q8_16"], 2048, K, 16)
        dg.dg_gemv_q8_0(Wq8, Xq, outs["q8_3"], 2048, K, 3)     # units
        dg.dg_gemv_nf4(codes, absmax, table, xb, outs["nf4"], N=2048, K=K, B=64)
        dg.dg_gemv_q4_0_f32(Wq4, xf[0].contiguous(), outs["f32"], 2048, K, 1, Xq=Xq1)
        dg.dg_gemv_bf16_argmax(Wb, xb, outs["tok"], y=outs["logits"], N=20000, K=K, ws=ws_tail)
        dg.dg_argcompare_rows(xf, outs["amin"], op="min", ws=ws_arg)
        dg.dg_argmax_rows_noalloc(xf, outs["anoalloc"])

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
        xf.copy_(synth.gpu_normal((704, 1, rep, 0), (16, K), 1.0, torch.float32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in outs.items()}
        for v in outs.values():
            v.fill_(-1)
        step()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(got[k], v), f"replay {rep}: {k} differs from the eager call"
