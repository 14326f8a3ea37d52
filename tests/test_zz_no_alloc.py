"""dg_argmax_rows_noalloc through the C ABI against dg_argmax_rows (GPU).

The no-allocation argmax keeps its chunk keys in the library's fixed
per-device array; its indices must equal the workspace call's bit for bit,
on two calls in a row (the second smaller, so stale keys of the first call
sit in the array), and on the planted-tie workload shapes.
"""
import ctypes

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _raw_noalloc(dg, x, idx, R, C, ld):
    import torch
    lib = dg.raw()
    st = lib.dg_argmax_rows_noalloc(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(idx.data_ptr()), R, C, ld,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, st


def _reference(dg, x, R, C, ld):
    import torch
    idx = torch.full((R,), -1, dtype=torch.int64, device=x.device)
    ws = torch.full((max(8, dg.dg_argmax_workspace_bytes(R, C)),), 0x5A, dtype=torch.uint8, device=x.device)
    dg.dg_argmax_rows(x, idx, R=R, C=C, ld=ld, ws=ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy()


@pytest.mark.parametrize("first,second", [((64, 1000000, 1000000), (3, 5000, 5003)),
                                          ((32, 128000, 128000), (1, 128256, 128256)),
                                          ((1, 128256, 128256), (1, 1, 1))])
def test_noalloc_argmax_equals_workspace_call_twice(dg, dev, orc, first, second):
    import torch
    for i, (R, C, ld) in enumerate((first, second)):
        vals, _ = synth.argmax_logits(950 + i, R, ld)
        x = torch.from_numpy(vals).to(dev)
        idx = torch.full((R,), -1, dtype=torch.int64, device=dev)
        _raw_noalloc(dg, x, idx, R, C, ld)
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        assert np.array_equal(got, _reference(dg, x, R, C, ld)), (R, C, ld)
        assert np.array_equal(got, orc.argmax_rows(vals, C=C, ld=ld)), (R, C, ld)


def test_noalloc_argmax_rejects_too_many_keys(dg, dev):
    import torch
    from tests.test_abi import noalloc_max_rows
    C = 1 << 20
    rmax = noalloc_max_rows(dg.raw(), C, dg.DG_ARGMAX_SCRATCH_BYTES)
    x = torch.zeros(8, dtype=torch.float32, device=dev)
    idx = torch.full((1,), -7, dtype=torch.int64, device=dev)
    lib = dg.raw()
    st = lib.dg_argmax_rows_noalloc(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(idx.data_ptr()), rmax + 1, C, C,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == dg.DG_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert int(idx[0]) == -7
