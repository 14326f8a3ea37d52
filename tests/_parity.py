"""Helpers shared by the GPU parity tests (no arithmetic of the method here)."""
import numpy as np


def floored_rel_err(got, ref, floor_frac=1e-3):
    """Per-element |got - ref| / max(|ref|, floor_frac * rms(ref)).

    A strict relative error is unstable for rows whose exact value is near 0
    (an fp32 sum of thousands of terms carries an absolute error of about
    1e-7..1e-5 however small its result is), so the denominator is floored at
    floor_frac times the root-mean-square of the reference.  A single dropped
    or wrong term is still orders of magnitude above the bound.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    den = np.maximum(np.abs(ref), floor_frac * rms)
    den = np.where(den == 0, 1.0, den)
    return np.abs(got - ref) / den


def assert_close(got, ref, tol, what=""):
    err = floored_rel_err(got, ref)
    worst = int(np.argmax(err)) if err.size else 0
    assert err.size == 0 or err.max() <= tol, (
        f"{what}: max floored relative error {err.max():.3e} > {tol} at {worst}: "
        f"got {np.asarray(got).reshape(-1)[worst]!r} ref {np.asarray(ref).reshape(-1)[worst]!r}")
    return float(err.max()) if err.size else 0.0


# Configurations of the resident-activation matrix-core kernel the library
# builds: (RT row tiles, KS parts of K, P chunks in flight); launch override
# unroll = RT*10000 + KS*100 + P*10.  A configuration runs a shape when K/32
# is a multiple of 8*KS and the workgroup's LDS fits (160 KiB on gfx950):
# the M activation columns (36-byte blocks, odd number of 16-byte slots per
# column), one transpose buffer per wave and the partial sums of the upper K
# parts.
RES_CFGS = [(1, 16, 2), (2, 8, 2), (4, 4, 2), (1, 8, 2), (2, 4, 2), (4, 2, 2), (8, 1, 2), (1, 4, 2), (2, 2, 2),
            (4, 1, 2), (1, 8, 3), (2, 4, 3), (1, 4, 3)]
LDS_PER_WORKGROUP = 160 * 1024


def res_unroll(rt, ks, p):
    return rt * 10000 + ks * 100 + p * 10


def res_runs(block_bytes, rt, ks, M, K):
    nblk = K // 32
    if nblk % (8 * ks) or M < 1 or M > 32:
        return False
    nt = 1 if M <= 16 else 2
    if nt == 2 and rt * ks == 16 and (block_bytes == 34 or rt > 1):
        return False   # not built: it would spill
    g = 8 * block_bytes // 16
    buf = -(-16 * g // 64) * 1024
    cstr = ((nblk * 36 // 16) | 1) * 16
    lds = M * cstr + rt * ks * buf + rt * (ks - 1) * nt * 1024
    return lds <= LDS_PER_WORKGROUP


def res_default(block_bytes, N, M, K):
    """The configuration the library picks when no override is given: four row
    tiles per workgroup for more than 512 tiles (K in two parts for Q4_0, whole
    for Q8_0), else one tile with K in eight parts; one tile with K in four
    parts when that does not fit."""
    tiles = (N + 15) // 16
    cfg = ((4, 1 if block_bytes == 34 else 2, 2) if tiles > 512 else (1, 8, 2))
    if not res_runs(block_bytes, cfg[0], cfg[1], M, K):
        cfg = (1, 4, 2)
    return cfg
