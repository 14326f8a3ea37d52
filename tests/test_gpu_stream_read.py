"""dg_stream_read reads every byte exactly once: the wrapping sum of its
per-workgroup partials equals the oracle's wrapping word sum (GPU)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _total(parts):
    return int(parts.cpu().numpy().view(np.uint32).astype(np.uint64).sum() % 2**32)


def _run(dg, dev, buf, nbytes, **kw):
    import torch
    grid = kw.get("grid_blocks") or dg.DG_READ_DEFAULT_GRID
    # one spare entry past the grid, poisoned: the probe must not write it
    parts = torch.full((grid + 1,), -1, dtype=torch.int32, device=dev)
    dg.dg_stream_read(buf, parts[:grid], nbytes=nbytes, **kw)
    torch.cuda.synchronize()
    assert int(parts[grid]) == -1
    return _total(parts[:grid])


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 1 << 20, (64 << 20) + 48])
@pytest.mark.parametrize("launch", [dict(flags=1), dict(flags=0), dict(flags=2), dict(flags=3),
                                    dict(grid_blocks=1, block_threads=64), dict(grid_blocks=7, block_threads=1024),
                                    dict(grid_blocks=4096, block_threads=512, flags=3),
                                    dict(grid_blocks=3, block_threads=192, flags=1), dict(flags=5),
                                    dict(grid_blocks=9, block_threads=128, flags=4), dict(flags=9), dict(flags=17),
                                    dict(grid_blocks=5, block_threads=256, flags=8),
                                    dict(grid_blocks=65537, block_threads=256, flags=17),
                                    dict(grid_blocks=11, block_threads=256, flags=33),
                                    dict(grid_blocks=6, block_threads=384, flags=33 | 8 | (5 << 8)),
                                    dict(grid_blocks=3000, block_threads=128, flags=1 | 32 | (4 << 8)),
                                    dict(flags=1 | (1 << 8)), dict(grid_blocks=300, block_threads=64, flags=(15 << 8))])
def test_stream_checksum_matches_oracle(dg, dev, orc, nbytes, launch):
    import torch
    g = np.random.default_rng(nbytes)
    words = g.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to(dev)
    assert _run(dg, dev, buf, nbytes, **launch) == orc.checksum_u32(words)


def test_stream_partials_overwrite_and_cover_every_workgroup(dg, dev, orc):
    """Every one of the G partials is written (stale values are overwritten),
    whether or not its workgroup had bytes to read."""
    import torch
    words = np.arange(1 << 16, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to(dev)
    for grid in (0, 3, 5000):
        g = grid or dg.DG_READ_DEFAULT_GRID
        parts = torch.full((g,), 12345, dtype=torch.int32, device=dev)
        dg.dg_stream_read(buf, parts, grid_blocks=grid, block_threads=256)
        dg.dg_stream_read(buf, parts, grid_blocks=grid, block_threads=256)
        torch.cuda.synchronize()
        assert _total(parts) == orc.checksum_u32(words), grid
        if g == 5000:   # 64 Ki words read by 8 KiB wave steps: most workgroups have nothing to read
            assert int((parts == 0).sum()) > 0


def test_stream_full_size_closed_form(dg, dev):
    """The ceiling workload, an 8 GiB buffer (32 x the 256 MiB last-level cache),
    filled with w_i = i: the wrapping sum has the closed form n(n-1)/2 mod 2^32."""
    import torch
    n = (8 << 30) // 4
    buf = torch.arange(n, dtype=torch.int32, device=dev)    # 0 .. 2^31 - 1
    expect = (n * (n - 1) // 2) % 2**32
    for flags in (0, 1, 2, 3, 5, 9, 17):
        assert _run(dg, dev, buf, n * 4, flags=flags) == expect
    # one-shot grids: every wave reads one chunk (8, 4 and 2 KiB per wave)
    for flags, chunk in ((1, 8192), (9, 4096), (17, 2048)):
        grid = n * 4 // (4 * chunk)
        assert _run(dg, dev, buf, n * 4, flags=flags, grid_blocks=grid, block_threads=256) == expect
    # capped residency, and half the waves of each workgroup reading
    for flags, block, waves in ((1 | (5 << 8), 128, 2), (17 | (4 << 8), 512, 8), (1 | 32 | (5 << 8), 256, 2)):
        grid = n * 4 // (waves * (2048 if flags & 16 else 8192))
        assert _run(dg, dev, buf, n * 4, flags=flags, grid_blocks=grid, block_threads=block) == expect
    del buf
    torch.cuda.empty_cache()
