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
