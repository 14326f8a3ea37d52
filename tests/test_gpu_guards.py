"""Guard regions around every buffer a call writes (GPU).

Each output (and each caller workspace) is a view into a larger device buffer
whose GUARD bytes before and after the view hold a sentinel byte.  After the
call the sentinel must be intact on both sides: no kernel wrote outside what
the header says it writes.  The outputs are also checked against the oracle,
so every element inside the view was written.  Shapes are ragged on purpose
(rows not a multiple of any tile or row group, column counts of every kernel
family the default dispatch picks), since a tail is where a stray store would
land.
"""
import numpy as np
import pytest

import synth
from tests._parity import assert_close

pytestmark = pytest.mark.gpu

GUARD = 4096          # bytes on each side of every view
SENTINEL = 0xA5


class Guarded:
    """A device view of `count` elements of `dtype` with sentinel bytes around it."""

    def __init__(self, dev, count, dtype):
        import torch
        self.torch = torch
        esize = torch.empty((), dtype=dtype).element_size()
        self.nbytes = count * esize
        self.buf = torch.full((GUARD + self.nbytes + GUARD,), SENTINEL, dtype=torch.uint8, device=dev)
        self.view = self.buf[GUARD:GUARD + self.nbytes].view(dtype)

    def assert_guards(self, what):
        self.torch.cuda.synchronize()
        before = self.buf[:GUARD].cpu().numpy()
        after = self.buf[GUARD + self.nbytes:].cpu().numpy()
        bad_b = np.flatnonzero(before != SENTINEL)
        bad_a = np.flatnonzero(after != SENTINEL)
        assert bad_b.size == 0, f"{what}: {bad_b.size} bytes written before the output (first at -{GUARD - bad_b[-1]})"
        assert bad_a.size == 0, f"{what}: {bad_a.size} bytes written after the output (first at +{bad_a[0]})"


def _dev_u8(dev, a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).reshape(-1).view(np.uint8)).to(dev)


def _dev_bits(dev, bits, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).reshape(-1).view(np.int16)).to(dev).view(dtype)


# --------------------------------------------------------------------------
# dense
# --------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("variant", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("N,K", [(1003, 4104), (77, 520)])
def test_dense_output_guards(dg, dev, orc, fmt, variant, N, K):
    import torch
    gen = synth.normal_f16_bits if fmt == "f16" else synth.normal_bf16_bits
    wd = torch.float16 if fmt == "f16" else torch.bfloat16
    Wb = gen((900, synth.KIND_W, 0, 0), (N, K), 0.02)
    xb = gen((900, synth.KIND_X, 0, 0), (K,), 1.0)
    y = Guarded(dev, N, torch.float16 if fmt == "f16" else torch.float32)
    fn = dg.dg_gemv_f16 if fmt == "f16" else dg.dg_gemv_bf16
    launch = dict(variant=variant) if variant else None
    try:
        fn(_dev_bits(dev, Wb, wd), _dev_bits(dev, xb, wd), y.view, N=N, K=K, ldw=K, launch=launch)
    except dg.DGError:
        pytest.skip("this dense variant does not take the shape")
    y.assert_guards(f"gemv_{fmt} {N}x{K} variant {variant}")
    ref = (orc.gemv_f16 if fmt == "f16" else orc.gemv_bf16)(Wb, xb, N=N, K=K, ldw=K)
    assert_close(y.view.float().cpu().numpy(), ref, 2e-3, f"gemv_{fmt}")


# --------------------------------------------------------------------------
# Q4_0 / Q8_0 x Q8_1: shapes and column counts that take every kernel family
# of the default dispatch (M = 1 row kernels, units, dot4 LDS, resident and
# streaming matrix cores)
# --------------------------------------------------------------------------

QUANT_CASES = [(1003, 4096, 1), (16400, 2048, 1), (1003, 4096, 3), (2051, 4096, 4), (1003, 4096, 2),
               (1003, 4096, 9), (2051, 4096, 5), (8200, 4096, 12), (2051, 4096, 17), (1003, 8192, 24)]


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("N,K,M", QUANT_CASES)
def test_quantised_gemv_output_guards(dg, dev, orc, fmt, N, K, M):
    quant = orc.quantize_q4_0 if fmt == "q4_0" else orc.quantize_q8_0
    gemv = orc.gemv_q4_0_q8_1 if fmt == "q4_0" else orc.gemv_q8_0_q8_1
    Wq = quant(synth.normal_f32((901, synth.KIND_W, 0, 0), (N, K)), threads=0)
    Xq = orc.quantize_q8_1(np.stack([synth.normal_f32((901, synth.KIND_X, 0, m), (K,)) for m in range(M)]))
    import torch
    Y = Guarded(dev, M * N, torch.float32)
    (dg.dg_gemv_q4_0 if fmt == "q4_0" else dg.dg_gemv_q8_0)(_dev_u8(dev, Wq), _dev_u8(dev, Xq), Y.view, N, K, M)
    Y.assert_guards(f"{fmt} {N}x{K} M={M}")
    assert_close(Y.view.cpu().numpy().reshape(M, N), gemv(Wq, Xq, N, K, M, threads=0), 1e-3, f"{fmt} M={M}")


@pytest.mark.parametrize("N,K,M,launch", [(1003, 4096, 3, None), (1003, 4096, 16, None), (2051, 4096, 17, None),
                                          (1003, 14336, 16, None), (300, 5888, 24, dict(unroll=3040402))])
def test_tiled_q4_0_output_workspace_and_weight_guards(dg, dev, orc, N, K, M, launch):
    """The tiled copy, the outputs and the workspace (its ticket counters and
    partial sums, K split over workgroups in the last two cases) stay within
    their extents on ragged shapes; the counters end at zero."""
    import torch
    Wq = orc.quantize_q4_0(synth.normal_f32((906, synth.KIND_W, 0, 0), (N, K)), threads=0)
    Xq = orc.quantize_q8_1(np.stack([synth.normal_f32((906, synth.KIND_X, 0, m), (K,)) for m in range(M)]))
    Wt = Guarded(dev, dg.dg_q4_0_tiles_bytes(N, K), torch.uint8)
    dg.dg_repack_q4_0_tiles(_dev_u8(dev, Wq), Wt.view, N, K)
    Wt.assert_guards(f"tiles {N}x{K} Wt")
    need = max(dg.dg_gemv_q4_0_tiles_workspace_bytes(N, K, M), 1 << 20)
    ws = Guarded(dev, need, torch.uint8)
    ws.view.zero_()
    Y = Guarded(dev, M * N, torch.float32)
    dg.dg_gemv_q4_0_tiles(Wt.view, _dev_u8(dev, Xq), Y.view, N, K, M, ws=ws.view, launch=launch)
    Y.assert_guards(f"tiles {N}x{K} M={M} Y")
    ws.assert_guards(f"tiles {N}x{K} M={M} ws")
    assert not torch.any(ws.view[:64 * 1024] != 0).item()
    assert_close(Y.view.cpu().numpy().reshape(M, N), orc.gemv_q4_0_q8_1(Wq, Xq, N, K, M, threads=0), 1e-3,
                 f"tiles M={M}")


@pytest.mark.parametrize("N,K,M,launch", [(1003, 4096, 1, None), (1003, 4096, 5, None), (2051, 8192, 1, dict(variant=13))])
def test_fp32_activation_gemv_output_and_workspace_guards(dg, dev, orc, N, K, M, launch):
    import torch
    Wq = orc.quantize_q4_0(synth.normal_f32((902, synth.KIND_W, 0, 0), (N, K)), threads=0)
    x = np.stack([synth.normal_f32((902, synth.KIND_X, 0, m), (K,)) for m in range(M)]).astype(np.float32)
    Y = Guarded(dev, M * N, torch.float32)
    Xq = Guarded(dev, M * (K // 32) * 36, torch.uint8)
    dg.dg_gemv_q4_0_f32(_dev_u8(dev, Wq), torch.from_numpy(x.reshape(-1)).to(dev), Y.view, N, K, M,
                        Xq=Xq.view, launch=launch)
    Y.assert_guards(f"q4_0_f32 {N}x{K} M={M} Y")
    Xq.assert_guards(f"q4_0_f32 {N}x{K} M={M} Xq")
    Xq_ref = orc.quantize_q8_1(x)
    assert_close(Y.view.cpu().numpy().reshape(M, N), orc.gemv_q4_0_q8_1(Wq, Xq_ref, N, K, M, threads=0), 1e-3,
                 "q4_0_f32")


# --------------------------------------------------------------------------
# NF4
# --------------------------------------------------------------------------

@pytest.mark.parametrize("launch", [None, dict(variant=31), dict(variant=32)])
@pytest.mark.parametrize("N,K", [(1003, 4096), (77, 8192)])
def test_nf4_output_guards(dg, dev, orc, launch, N, K):
    import torch
    B = 64
    table = synth.nf4_table()
    codes, absmax = orc.quantize_nf4(synth.normal_f32((903, synth.KIND_W, 0, 0), (N, K)), table, B, threads=0)
    xb = synth.normal_bf16_bits((903, synth.KIND_X, 0, 0), (K,), 1.0)
    y = Guarded(dev, N, torch.float32)
    dg.dg_gemv_nf4(_dev_u8(dev, codes), torch.from_numpy(np.ascontiguousarray(absmax, np.float32).reshape(-1)).to(dev),
                   torch.from_numpy(np.asarray(table, np.float32)).to(dev), _dev_bits(dev, xb, torch.bfloat16),
                   y.view, N=N, K=K, B=B, launch=launch)
    y.assert_guards(f"nf4 {N}x{K} {launch}")
    assert_close(y.view.cpu().numpy(), orc.gemv_nf4(codes, absmax, table, xb, N, K, B, threads=0), 1e-3, "nf4")


# --------------------------------------------------------------------------
# quantisers
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["q8_1", "q4_0", "q8_0", "nf4"])
def test_quantiser_output_guards(dg, dev, orc, kind):
    import torch
    R, K, B = 37, 544, 32
    w = synth.normal_f32((904, synth.KIND_W, 0, 0), (R, K))
    wd = torch.from_numpy(w.reshape(-1)).to(dev)
    if kind == "nf4":
        table = synth.nf4_table()
        codes = Guarded(dev, R * K // 2, torch.uint8)
        absmax = Guarded(dev, R * (K // B), torch.float32)
        dg.dg_quantize_nf4(wd, codes.view, absmax.view, torch.from_numpy(np.asarray(table, np.float32)).to(dev),
                           R, K, B)
        codes.assert_guards("nf4 codes")
        absmax.assert_guards("nf4 absmax")
        c_ref, a_ref = orc.quantize_nf4(w, table, B)
        assert np.array_equal(codes.view.cpu().numpy(), np.asarray(c_ref).reshape(-1))
        assert np.array_equal(absmax.view.cpu().numpy().view(np.uint32),
                              np.asarray(a_ref, np.float32).reshape(-1).view(np.uint32))
        return
    bb = {"q8_1": 36, "q4_0": 18, "q8_0": 34}[kind]
    out = Guarded(dev, R * (K // 32) * bb, torch.uint8)
    getattr(dg, f"dg_quantize_{kind}")(wd, out.view, R, K)
    out.assert_guards(kind)
    ref = getattr(orc, f"quantize_{kind}")(w)
    assert np.array_equal(out.view.cpu().numpy(), np.asarray(ref).reshape(-1))


# --------------------------------------------------------------------------
# argmax, ArgCompare, the greedy tail
# --------------------------------------------------------------------------

@pytest.mark.parametrize("R,C", [(1, 128001), (5, 1001), (3, 70000)])
def test_argmax_index_and_workspace_guards(dg, dev, orc, R, C):
    import torch
    x = synth.normal_f32((905, synth.KIND_X, 0, 0), (R, C))
    xd = torch.from_numpy(x).to(dev)
    idx = Guarded(dev, R, torch.int64)
    ws = Guarded(dev, dg.dg_argmax_workspace_bytes(R, C), torch.uint8)
    dg.dg_argmax_rows(xd, idx.view, ws=ws.view)
    idx.assert_guards("argmax idx")
    ws.assert_guards("argmax workspace")
    assert np.array_equal(idx.view.cpu().numpy(), orc.argmax_rows(x))
    idx2 = Guarded(dev, R, torch.int64)
    dg.dg_argmax_rows_noalloc(xd, idx2.view)
    idx2.assert_guards("argmax_noalloc idx")
    assert np.array_equal(idx2.view.cpu().numpy(), orc.argmax_rows(x))
    bits = synth.normal_bf16_bits((905, synth.KIND_X, 1, 0), (R, C), 1.0)
    idx3 = Guarded(dev, R, torch.int64)
    ws3 = Guarded(dev, dg.dg_argmax_workspace_bytes(R, C), torch.uint8)
    dg.dg_argcompare_rows(_dev_bits(dev, bits, torch.bfloat16).view(R, C), idx3.view, op="min", ws=ws3.view)
    idx3.assert_guards("argcompare idx")
    ws3.assert_guards("argcompare workspace")
    assert np.array_equal(idx3.view.cpu().numpy(), orc.argcompare_rows(bits, "bf16", "min"))


@pytest.mark.parametrize("keep_logits", [True, False])
def test_greedy_tail_guards(dg, dev, orc, keep_logits):
    import torch
    N, K = 20011, 1024
    Wb = synth.normal_bf16_bits((906, synth.KIND_W, 0, 0), (N, K), 0.02)
    xb = synth.normal_bf16_bits((906, synth.KIND_X, 0, 0), (K,), 1.0)
    idx = Guarded(dev, 1, torch.int64)
    y = Guarded(dev, N, torch.float32) if keep_logits else None
    ws = Guarded(dev, dg.dg_gemv_bf16_argmax_workspace_bytes(N, K), torch.uint8)
    dg.dg_gemv_bf16_argmax(_dev_bits(dev, Wb, torch.bfloat16), _dev_bits(dev, xb, torch.bfloat16), idx.view,
                           y=y.view if y else None, N=N, K=K, ws=ws.view)
    idx.assert_guards("tail token")
    ws.assert_guards("tail workspace")
    ref = orc.gemv_bf16(Wb, xb, N=N, K=K)
    if y is not None:
        y.assert_guards("tail logits")
        assert_close(y.view.cpu().numpy(), ref, 2e-3, "tail logits")
    # the token is the argmax of the logits the GPU computed (bit-exact rule)
    logits = torch.empty(N, dtype=torch.float32, device=dev)
    dg.dg_gemv_bf16(_dev_bits(dev, Wb, torch.bfloat16), _dev_bits(dev, xb, torch.bfloat16), logits, N=N, K=K)
    torch.cuda.synchronize()
    assert int(idx.view.cpu()[0]) == int(orc.argmax_rows(logits.cpu().numpy().reshape(1, N))[0])
