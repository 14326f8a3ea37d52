"""Parity of the 16-row-tile paths (dg_repack_q4_0_tiles / dg_repack_q8_0_tiles,
then dg_gemv_q4_0_tiles / dg_gemv_q8_0_tiles, M = 1..24) with the oracle (GPU).

The rearrangements are checked byte for byte against the layouts written out
below with numpy indexing (permutations of the row-major bytes, independent
of the library); the GEMVs against the oracle's Q4_0 / Q8_0 x Q8_1 products
of the row-major bytes, on operands quantised on the CPU by the oracle's
quantisers.
"""
import functools

import numpy as np
import pytest

import synth
from tests._parity import assert_close

pytestmark = pytest.mark.gpu

TOL = 1e-3   # per-row floored relative error vs the oracle
TICKET_BYTES = 64 * 1024   # the workspace's ticket counters (include/decodegemv.h)

# (RT, KW, D) configurations the library builds; unroll = CS*100000000 +
# KP*1000000 + RT*10000 + KW*100 + D
BUILT = [(1, 4, 2), (1, 4, 4), (1, 8, 2), (1, 8, 4), (1, 16, 2), (2, 4, 2), (2, 4, 4), (2, 2, 4), (2, 8, 2),
         (4, 1, 4), (4, 2, 2), (4, 2, 4), (4, 4, 2), (4, 4, 4)]
FORMATS = ["q4_0", "q8_0"]


def built(fmt, cfg, M):
    """Q8_0 with 24 columns in 16-wave workgroups four groups deep would spill: not built."""
    return not (fmt == "q8_0" and M > 16 and cfg[0] * cfg[1] == 16 and cfg[2] == 4)


def unroll(kp, rt, kw, d, cs=0):
    return cs * 100000000 + kp * 1000000 + rt * 10000 + kw * 100 + d


def tiled_layout_q8(Wq, N, K):
    """The tiled bytes of row-major Q8_0 bytes Wq [N][K/32*34], by indexing
    (codes and scales unchanged)."""
    nb = K // 32
    S = K // 256
    T = (N + 15) // 16
    pad = np.zeros((T * 16, nb, 34), dtype=np.uint8)
    pad[:N] = np.asarray(Wq, dtype=np.uint8).reshape(N, nb, 34)
    b = pad.reshape(T, 16, S, 8, 34)
    # code dword d = g + 4q of block i = 2h + e  ->  [t, n, s, h, e, q, g, byte]
    codes = b[..., 2:].reshape(T, 16, S, 4, 2, 2, 4, 4)
    out = np.zeros((T, S, 4352), dtype=np.uint8)
    # bytes 1024h + (16g + n)*16 + 8e + 4q + byte
    out[:, :, :4096] = codes.transpose(0, 2, 3, 6, 1, 4, 5, 7).reshape(T, S, 4096)
    out[:, :, 4096:] = b[..., :2].transpose(0, 2, 1, 3, 4).reshape(T, S, 256)
    return out.reshape(-1)


def tiled_layout(Wq, N, K):
    """The tiled bytes of row-major Q4_0 bytes Wq [N][K/32*18], by indexing:
    each 4-bit code q is stored as q XOR 8, the two's-complement nibble of q - 8."""
    nb = K // 32
    S = K // 256
    T = (N + 15) // 16
    blocks = np.asarray(Wq, dtype=np.uint8).reshape(N, nb, 18)
    pad = np.zeros((T * 16, nb, 18), dtype=np.uint8)
    pad[:N] = blocks
    pad[:N, :, 2:] ^= 0x88   # codes as signed nibbles q - 8 (padding rows: 0)
    # [T, 16 rows, S, 8 blocks, 18]
    b = pad.reshape(T, 16, S, 8, 18)
    codes = b[..., 2:].reshape(T, 16, S, 8, 4, 4)            # [t, n, s, i, g, byte]
    scales = b[..., :2]                                       # [t, n, s, i, 2]
    out = np.zeros((T, S, 2304), dtype=np.uint8)
    # bytes h*1024 + (16g + n)*16 + 4j + byte = code dword g of row n, block 4h + j
    c = codes.reshape(T, 16, S, 2, 4, 4, 4)                   # [t, n, s, h, j, g, byte]
    c = c.transpose(0, 2, 3, 5, 1, 4, 6)                      # [t, s, h, g, n, j, byte]
    out[:, :, :2048] = c.reshape(T, S, 2048)
    out[:, :, 2048:] = scales.transpose(0, 2, 1, 3, 4).reshape(T, S, 256)
    return out.reshape(-1)


@functools.lru_cache(maxsize=8)
def _weights(orc, fmt, cfg, N, K):
    w = synth.normal_f32((cfg, synth.KIND_W, 0, 0), (N, K))
    return (orc.quantize_q4_0 if fmt == "q4_0" else orc.quantize_q8_0)(w, threads=0)


def _operands(orc, fmt, cfg, N, K, M, same_columns=False):
    Wq = _weights(orc, fmt, cfg, N, K)
    cols = [synth.normal_f32((cfg, synth.KIND_X, 0, 0 if same_columns else m), (K,)) for m in range(M)]
    return Wq, orc.quantize_q8_1(np.stack(cols))


def _ref(orc, fmt, Wq, Xq, N, K, M, threads=1):
    return (orc.gemv_q4_0_q8_1 if fmt == "q4_0" else orc.gemv_q8_0_q8_1)(Wq, Xq, N, K, M, threads=threads)


def _tiles(dg, dev, fmt, Wq, N, K):
    import torch
    W = torch.from_numpy(np.ascontiguousarray(Wq).reshape(-1)).to(dev)
    nbytes = (dg.dg_q4_0_tiles_bytes if fmt == "q4_0" else dg.dg_q8_0_tiles_bytes)(N, K)
    Wt = torch.full((max(nbytes, 16),), 0xA5, dtype=torch.uint8, device=dev)
    (dg.dg_repack_q4_0_tiles if fmt == "q4_0" else dg.dg_repack_q8_0_tiles)(W, Wt, N, K)
    return Wt


def _gpu(dg, dev, fmt, Wt, Xq, N, K, M, launch=None, ws=None):
    import torch
    X = torch.from_numpy(np.ascontiguousarray(Xq).reshape(-1)).to(dev)
    Y = torch.full((max(M, 1), max(N, 1)), float("nan"), dtype=torch.float32, device=dev)
    if ws is None:   # the default launch's workspace, and room for every override at the small shapes
        need = (dg.dg_gemv_q4_0_tiles_workspace_bytes if fmt == "q4_0" else dg.dg_gemv_q8_0_tiles_workspace_bytes)
        ws = torch.zeros(max(need(N, K, M), 1 << 23), dtype=torch.uint8, device=dev)
    (dg.dg_gemv_q4_0_tiles if fmt == "q4_0" else dg.dg_gemv_q8_0_tiles)(Wt, X, Y, N, K, M, ws=ws, launch=launch)
    torch.cuda.synchronize()
    return Y[:M, :N].cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("N,K", [(1, 256), (16, 256), (41, 768), (300, 4096), (33, 14336)])
def test_tiles_repack_matches_layout(dg, dev, orc, fmt, N, K):
    Wq = _weights(orc, fmt, 600, N, K)
    Wt = _tiles(dg, dev, fmt, Wq, N, K)
    import torch
    torch.cuda.synchronize()
    got = Wt.cpu().numpy()
    ref = (tiled_layout if fmt == "q4_0" else tiled_layout_q8)(Wq, N, K)
    assert (dg.dg_q4_0_tiles_bytes if fmt == "q4_0" else dg.dg_q8_0_tiles_bytes)(N, K) == ref.size
    assert np.array_equal(got[:ref.size], ref)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M", list(range(1, 25)))
def test_tiles_every_column_count_small(dg, dev, orc, fmt, M):
    N, K = 41, 768   # three tiles (the last ragged), three groups of 8 blocks
    Wq, Xq = _operands(orc, fmt, 610 + M, N, K, M)
    got = _gpu(dg, dev, fmt, _tiles(dg, dev, fmt, Wq, N, K), Xq, N, K, M)
    assert_close(got, _ref(orc, fmt, Wq, Xq, N, K, M), TOL, f"{fmt} M={M}")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("cfg", BUILT, ids=[str(c) for c in BUILT])
@pytest.mark.parametrize("kp", [1, 2, 3, 5])
@pytest.mark.parametrize("M", [3, 16, 20])
def test_tiles_every_configuration(dg, dev, orc, fmt, cfg, kp, M):
    """Every built (RT, KW, D) with K split over 1..5 workgroups: ragged row
    groups (N = 200: 13 tiles), parts of K that do not divide evenly (K =
    5888: 23 groups of 8 blocks) and waves without a part."""
    N, K = 200, 5888
    Wq, Xq = _operands(orc, fmt, 620, N, K, M)
    Wt = _tiles(dg, dev, fmt, Wq, N, K)
    if not built(fmt, cfg, M):
        with pytest.raises(dg.DGError):
            _gpu(dg, dev, fmt, Wt, Xq, N, K, M, launch=dict(unroll=unroll(kp, *cfg)))
        return
    got = _gpu(dg, dev, fmt, Wt, Xq, N, K, M, launch=dict(unroll=unroll(kp, *cfg)))
    assert_close(got, _ref(orc, fmt, Wq, Xq, N, K, M), TOL, f"{fmt} {cfg} KP={kp} M={M}")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("cfg", [(1, 8, 2), (2, 4, 2), (4, 2, 4)], ids=str)
@pytest.mark.parametrize("cs", [2, 3, 5, 8])
@pytest.mark.parametrize("kp", [1, 3])
@pytest.mark.parametrize("M", [3, 9, 16, 17, 24])
def test_tiles_column_slices(dg, dev, orc, fmt, cfg, cs, kp, M):
    """Columns split over CS workgroups per row group and K range (ceil(M /
    CS) each, the last slice shorter), K in 1 or 3 ranges: units padded to
    whole blocks of 8 (N = 200), a K that leaves waves without a part (23
    groups of 8 blocks).  A split that would leave a slice empty is an
    argument error."""
    N, K = 200, 5888
    Wq, Xq = _operands(orc, fmt, 650 + M, N, K, M)
    Wt = _tiles(dg, dev, fmt, Wq, N, K)
    if (cs - 1) * -(-M // cs) >= M:
        with pytest.raises(dg.DGError):
            _gpu(dg, dev, fmt, Wt, Xq, N, K, M, launch=dict(unroll=unroll(kp, *cfg, cs=cs)))
        return
    got = _gpu(dg, dev, fmt, Wt, Xq, N, K, M, launch=dict(unroll=unroll(kp, *cfg, cs=cs)))
    assert_close(got, _ref(orc, fmt, Wq, Xq, N, K, M), TOL, f"{fmt} {cfg} CS={cs} KP={kp} M={M}")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("cfg,kp,cs", [((1, 8, 2), 2, 1), ((2, 2, 4), 3, 1), ((4, 4, 2), 1, 2), ((4, 2, 2), 2, 2)],
                         ids=str)
@pytest.mark.parametrize("M", [5, 16, 24])
def test_tiles_prologue_orders_give_identical_bits(dg, dev, orc, fmt, cfg, kp, cs, M):
    """The weight loads of the first groups issued after the column copies
    have landed (the default) or before (D + 10): the same arithmetic in the
    same order, so the same bits."""
    N, K = 200, 5888
    Wq, Xq = _operands(orc, fmt, 670 + M, N, K, M)
    Wt = _tiles(dg, dev, fmt, Wq, N, K)
    a = _gpu(dg, dev, fmt, Wt, Xq, N, K, M, launch=dict(unroll=unroll(kp, *cfg, cs=cs)))
    rt, kw, d = cfg
    b = _gpu(dg, dev, fmt, Wt, Xq, N, K, M, launch=dict(unroll=unroll(kp, rt, kw, d + 10, cs=cs)))
    assert np.array_equal(a, b)
    assert_close(a, _ref(orc, fmt, Wq, Xq, N, K, M), TOL, f"{fmt} {cfg} KP={kp} CS={cs} M={M}")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("cs,M", [(2, 10), (2, 16), (2, 17), (3, 24), (3, 20)])
def test_tiles_column_slices_long_rows(dg, dev, orc, fmt, cs, M):
    """A 4096 x 14336 matrix, whose columns fit a workgroup's LDS only in
    slices, with no workspace."""
    N, K = 4096, 14336
    Wq, Xq = _operands(orc, fmt, 660 + M, N, K, M)
    got = _gpu(dg, dev, fmt, _tiles(dg, dev, fmt, Wq, N, K), Xq, N, K, M,
               launch=dict(unroll=unroll(1, 2, 4, 2, cs=cs)))
    assert_close(got, _ref(orc, fmt, Wq, Xq, N, K, M, threads=0), TOL, f"{fmt} CS={cs} M={M}")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("N,K", [(4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336)])
@pytest.mark.parametrize("M", [1, 2, 4, 8, 12, 16, 17, 24])
def test_tiles_decoder_layer_shapes_all_rows(dg, dev, orc, fmt, N, K, M):
    Wq, Xq = _operands(orc, fmt, 3, N, K, M)
    got = _gpu(dg, dev, fmt, _tiles(dg, dev, fmt, Wq, N, K), Xq, N, K, M)
    assert_close(got, _ref(orc, fmt, Wq, Xq, N, K, M, threads=0), TOL, f"{fmt} {N}x{K} M={M}")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M", [1, 16, 24])
def test_tiles_subnormal_scales(dg, dev, orc, fmt, M):
    N, K = 300, 4096
    w = synth.normal_f32((901, synth.KIND_W, 0, 0), (N, K)) * np.float32(1e-5)
    Wq = (orc.quantize_q4_0 if fmt == "q4_0" else orc.quantize_q8_0)(w)
    cols = [synth.normal_f32((901, synth.KIND_X, 0, m), (K,)) * np.float32(1e-4) for m in range(M)]
    Xq = orc.quantize_q8_1(np.stack(cols))
    got = _gpu(dg, dev, fmt, _tiles(dg, dev, fmt, Wq, N, K), Xq, N, K, M)
    assert_close(got, _ref(orc, fmt, Wq, Xq, N, K, M, threads=0), TOL, f"{fmt} M={M}")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M", [2, 16, 24])
def test_tiles_identical_columns_give_identical_outputs(dg, dev, orc, fmt, M):
    N, K = 300, 4096
    Wq, Xq = _operands(orc, fmt, 630, N, K, M, same_columns=True)
    got = _gpu(dg, dev, fmt, _tiles(dg, dev, fmt, Wq, N, K), Xq, N, K, M)
    for m in range(1, M):
        assert np.array_equal(got[m], got[0])


def test_tiles_workspace_left_zero_and_calls_repeat_bit_for_bit(dg, dev, orc):
    """K split over workgroups: the ticket counters are zero after every call,
    repeated calls give identical bits, and calls of other shapes and the
    other format on the same workspace in between change nothing."""
    import torch
    N, K, M = 4096, 14336, 24
    need = dg.dg_gemv_q8_0_tiles_workspace_bytes(N, K, M)
    assert need > 0   # Q8_0 splits K at this shape by default
    ws = torch.zeros(8 << 20, dtype=torch.uint8, device=dev)
    Wq, Xq = _operands(orc, "q8_0", 640, N, K, M)
    Wt = _tiles(dg, dev, "q8_0", Wq, N, K)
    a = _gpu(dg, dev, "q8_0", Wt, Xq, N, K, M, ws=ws)
    assert not torch.any(ws[:TICKET_BYTES] != 0).item()
    b = _gpu(dg, dev, "q8_0", Wt, Xq, N, K, M, ws=ws)
    assert np.array_equal(a, b)
    assert_close(a, _ref(orc, "q8_0", Wq, Xq, N, K, M, threads=0), TOL, "first call")
    n2, k2, m2 = 1000, 14336, 5   # K split eight ways: its partial sums cover more of the workspace
    for fmt in FORMATS:
        Wq2, Xq2 = _operands(orc, fmt, 641, n2, k2, m2)
        Wt2 = _tiles(dg, dev, fmt, Wq2, n2, k2)
        ref2 = _ref(orc, fmt, Wq2, Xq2, n2, k2, m2, threads=0)
        for u in (unroll(8, 4, 2, 2), unroll(4, 2, 4, 2, cs=2)):   # the second: a counter per row group and slice
            c = _gpu(dg, dev, fmt, Wt2, Xq2, n2, k2, m2, ws=ws, launch=dict(unroll=u))
            assert_close(c, ref2, TOL, f"{fmt} smaller second call {u}")
            assert not torch.any(ws[:TICKET_BYTES] != 0).item()
    d = _gpu(dg, dev, "q8_0", Wt, Xq, N, K, M, ws=ws)   # the first shape again, after the others' partial sums
    assert np.array_equal(a, d)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("N", [1, 17])
@pytest.mark.parametrize("M", [1, 5, 24])
def test_tiles_one_group_of_k(dg, dev, orc, fmt, N, M):
    """K = 256: one group of 8 blocks per row tile, so every wave but the
    first of a workgroup has no part; the defaults slice the columns here."""
    K = 256
    Wq, Xq = _operands(orc, fmt, 680 + M, N, K, M)
    got = _gpu(dg, dev, fmt, _tiles(dg, dev, fmt, Wq, N, K), Xq, N, K, M)
    assert_close(got, _ref(orc, fmt, Wq, Xq, N, K, M), TOL, f"{fmt} N={N} M={M}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_tiles_empty_sums_and_empty_shapes(dg, dev, fmt):
    """K = 0 writes zeros; N = 0 or M = 0 launch nothing and touch nothing."""
    import torch
    lib = dg.raw()
    gemv = lib.dg_gemv_q4_0_tiles if fmt == "q4_0" else lib.dg_gemv_q8_0_tiles
    Y = torch.full((5 * 33,), float("nan"), dtype=torch.float32, device=dev)
    assert gemv(None, None, Y.data_ptr(), 33, 0, 5, None, 0, None) == 0
    torch.cuda.synchronize()
    assert not torch.any(Y != 0).item()
    Y.fill_(float("nan"))
    assert gemv(None, None, Y.data_ptr(), 0, 4096, 5, None, 0, None) == 0
    assert gemv(None, None, Y.data_ptr(), 33, 4096, 0, None, 0, None) == 0
    torch.cuda.synchronize()
    assert torch.isnan(Y).all().item()


def test_tiles_argument_errors(dg, dev):
    import torch
    N, K, M = 64, 28672, 24   # Q4_0 splits K at this shape by default
    lib = dg.raw()
    Wt = torch.zeros(dg.dg_q4_0_tiles_bytes(N, K), dtype=torch.uint8, device=dev)
    X = torch.zeros(M * K // 32 * 36, dtype=torch.uint8, device=dev)
    Y = torch.zeros(M * N, dtype=torch.float32, device=dev)
    need = dg.dg_gemv_q4_0_tiles_workspace_bytes(N, K, M)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    P = lambda t: t.data_ptr()   # noqa: E731
    assert lib.dg_gemv_q4_0_tiles(P(Wt), P(X), P(Y), N, K, M, P(ws), need - 1, None) == 4   # DG_ERR_WORKSPACE
    assert lib.dg_gemv_q4_0_tiles(P(Wt), P(X), P(Y), N, K, M, None, 0, None) == 4
    assert lib.dg_gemv_q4_0_tiles(P(Wt), P(X), P(Y), N, 4000, M, P(ws), need, None) == 3     # DG_ERR_SHAPE
    assert lib.dg_gemv_q4_0_tiles(P(Wt), P(X), P(Y), N, K, 25, P(ws), need, None) == 3
    for bad in (unroll(2, 3, 3, 3),          # not built
                unroll(1, 2, 4, 2, cs=9),    # more slices than allowed
                unroll(1, 2, 4, 2, cs=3),    # 8 columns of rows this long do not fit the LDS
                unroll(4, 4, 2, 2, cs=2)):   # the default here: fits
        cfg = dg.dg_launch(0, 0, 0, bad)
        rc = lib.dg_gemv_q4_0_tiles_ex(P(Wt), P(X), P(Y), N, K, M, P(ws), need, cfg, None)
        assert rc == (0 if bad == unroll(4, 4, 2, 2, cs=2) else 6), bad   # DG_ERR_ARG
    cfg = dg.dg_launch(0, 0, 0, unroll(8, 4, 2, 2))   # K in 8 ranges, no slices: more workspace than the default's
    assert lib.dg_gemv_q4_0_tiles_ex(P(Wt), P(X), P(Y), N, K, M, P(ws), need, cfg, None) == 4
    for m, bad in ((2, unroll(1, 2, 4, 2, cs=3)), (1, unroll(1, 2, 4, 2, cs=2))):   # an empty slice
        cfg = dg.dg_launch(0, 0, 0, bad)
        assert lib.dg_gemv_q4_0_tiles_ex(P(Wt), P(X), P(Y), N, K, m, P(ws), need, cfg, None) == 6
    torch.cuda.synchronize()
