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


# Configurations of the streaming matrix-core kernel the library builds:
# (RT row tiles, KS parts of K, DEPTH chunks staged, CB blocks per chunk);
# launch override unroll = RT*10000 + KS*100 + DEPTH*10 + CB/8.  Which column
# counts each serves follows from its LDS (one stage: every wave's 16 weight
# rows of a chunk, rows padded to an odd number of 16-byte slots, and the
# activation chunks of MP >= M columns; MP = 4, 8, 16 or 24) and the limits
# the library applies against register spills (12- and 16-wave workgroups up
# to 24 columns, 16 parts of K up to 16, Q8_0 at 16 waves up to 16).
MFMA_CONFIGS = [(1, 16, 1, 8), (2, 8, 1, 8), (4, 4, 2, 8), (1, 12, 1, 8), (3, 4, 1, 8), (1, 8, 1, 8), (1, 8, 2, 8),
                (2, 4, 2, 8), (4, 2, 2, 8), (8, 1, 2, 8), (4, 1, 2, 8), (4, 1, 3, 8), (2, 2, 2, 8), (1, 4, 2, 8),
                (1, 4, 3, 8), (1, 4, 4, 8), (1, 4, 5, 8), (2, 2, 3, 8), (2, 2, 4, 8)]


def mfma_unroll(rt, ks, d, cb):
    return rt * 10000 + ks * 100 + d * 10 + cb // 8


def mfma_builds(block_bytes, rt, ks, depth, cb, mp):
    w = rt * ks
    nt = (mp + 15) // 16
    wrow = (cb * block_bytes // 16) | 1
    cw = (16 * wrow + 63) // 64
    acol = (cb * 36 // 16) | 1
    apart = mp * acol
    ca = (apart + 63) // 64 if rt == 1 else (ks * apart + w * 64 - 1) // (w * 64)
    stage = w * cw * 1024 + ca * w * 1024
    lds = max(depth * stage, w * nt * 4 * 64 * 4)
    return (lds <= LDS_PER_WORKGROUP and (cw + ca) * (depth - 1) <= 63 and (w < 12 or mp <= 24)
            and (ks < 16 or mp <= 16) and (w < 16 or mp <= 16 or block_bytes == 18))


def mfma_max_columns(block_bytes, rt, ks, depth, cb):
    """The largest column count the configuration takes (0: not built)."""
    best = 0
    for mp in (4, 8, 16, 24):
        if mfma_builds(block_bytes, rt, ks, depth, cb, mp):
            best = mp
    return best
