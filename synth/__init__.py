"""Seeded synthetic inputs for the decode GEMV path.

This module is the one thing the GPU tests, the oracle checks and the benchmark
share.  It only draws random numbers and encodes them into the operand formats
(binary16 / bfloat16 bit patterns, float32); it holds none of the method's
arithmetic -- no products, no sums, no quantisation, no reductions.

Recipe (the workloads of the pages, with synthetic values):
  * dense weights  W ~ N(0, 0.02) (0.02 is the standard deviation), activations
    x ~ N(0, 1), drawn in float32 and rounded to nearest-even into binary16 or
    bfloat16;
  * weights to be quantised to Q4_0 and activations to be quantised to Q8_1
    are N(0, 1) float32 (the quantisers live in the library and in the oracle);
  * argmax logits are uniform(-10, 10) float32, with exact duplicate maxima
    planted in about 1% of the rows (at least one row);
  * weights to be quantised to NF4 are N(0, 1) float32 with bfloat16
    activations x ~ N(0, 1), and the 16-level code table both sides receive
    is ``nf4_table()``.

Every stream comes from numpy's PCG64 seeded with
``SeedSequence([0xD6, config, kind, copy, column])``; ``kind`` is 0 for weights,
1 for activations and 2 for tie positions.  ``gpu_*`` helpers draw the large
benchmark operands directly in device memory with a seeded torch generator
(same distributions, a different stream).
"""
from __future__ import annotations

import math

import numpy as np

ROOT_SEED = 0xD6
KIND_W, KIND_X, KIND_TIES = 0, 1, 2


def rng(config: int, kind: int, copy: int = 0, column: int = 0) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([ROOT_SEED, config, kind, copy, column])))


def normal_f32(key, shape, std: float = 1.0) -> np.ndarray:
    g = rng(*key)
    return g.standard_normal(shape, dtype=np.float32) * np.float32(std)


def to_f16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> binary16 bit patterns, round to nearest even (numpy's cast)."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)   # no wrap for finite u
    return r.astype(np.uint16)


def normal_f16_bits(key, shape, std: float = 1.0) -> np.ndarray:
    return to_f16_bits(normal_f32(key, shape, std))


def normal_bf16_bits(key, shape, std: float = 1.0) -> np.ndarray:
    return to_bf16_bits(normal_f32(key, shape, std))


def uniform_f32(key, shape, lo: float, hi: float) -> np.ndarray:
    g = rng(*key)
    return g.uniform(lo, hi, size=shape).astype(np.float32)


def argmax_logits(config: int, R: int, C: int, copy: int = 0, tie_fraction: float = 0.01,
                  lo: float = -10.0, hi: float = 10.0):
    """uniform(lo, hi) float32 [R][C] with planted exact duplicate maxima.

    max(1, ceil(tie_fraction * R)) rows are chosen by seed.  In each chosen row a
    value above ``hi`` is written at 2 to 4 positions (so it is the row maximum
    by construction); the first chosen row (when C >= 2) uses positions 0 and
    C-1.  Returns (logits, planted) where planted maps row -> sorted positions.
    """
    x = uniform_f32((config, KIND_X, copy, 0), (R, C), lo, hi)
    g = rng(config, KIND_TIES, copy, 0)
    n_rows = max(1, math.ceil(tie_fraction * R)) if R > 0 else 0
    rows = g.choice(R, size=min(n_rows, R), replace=False) if R > 0 else []
    planted = {}
    for i, r in enumerate(sorted(int(v) for v in rows)):
        val = np.float32(hi + 1.0 + float(g.uniform(0.0, 1.0)))
        if C == 1:
            pos = [0]
        elif i == 0:
            pos = [0, C - 1]
        else:
            k = int(g.integers(2, 5))
            pos = sorted(set(int(p) for p in g.choice(C, size=min(k, C), replace=False)))
        x[r, pos] = val
        planted[r] = pos
    return x, planted


# ---- device-side draws for the benchmark's large operands --------------------

def gpu_generator(config: int, kind: int, copy: int = 0, column: int = 0):
    import torch
    seed = int(np.random.SeedSequence([ROOT_SEED, config, kind, copy, column]).generate_state(1)[0])
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return g


def gpu_normal(key, shape, std: float, dtype):
    """N(0, std) drawn in float32 on the device, then cast (round to nearest even)."""
    import torch
    g = gpu_generator(*key)
    t = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t if dtype == torch.float32 else t.to(dtype)


def gpu_uniform(key, shape, lo: float, hi: float):
    import torch
    g = gpu_generator(*key)
    t = torch.rand(shape, generator=g, device="cuda", dtype=torch.float32)
    return t.mul_(hi - lo).add_(lo)


def nf4_table() -> np.ndarray:
    """The 16-entry code table of the NF4 workload, float32, increasing.

    An input of both the library and the oracle (the kernel takes its table as
    an argument, as the bitsandbytes kernel takes its quant_map), not part of
    the method's arithmetic.  It is a NormalFloat table in the manner of QLoRA
    (Dettmers et al., 2023, "4-bit NormalFloat Quantization"): levels at
    standard-normal quantiles of evenly spaced probabilities, eight on the
    non-negative side and seven on the negative side of an exact zero,
    normalised so that the extremes are -1 and 1.  The outermost probability
    is 1 - (1/32 + 1/30)/2; the positive levels are the quantiles at 8 evenly
    spaced probabilities from there down to 1/2 (exclusive), the negative ones
    at 7.  This reading is not claimed to match any library's table bit for
    bit; the kernel works with any increasing table.
    """
    from statistics import NormalDist
    inv = NormalDist().inv_cdf
    p_hi = 1.0 - (1.0 / 32.0 + 1.0 / 30.0) / 2.0
    pos = [inv(p_hi + (0.5 - p_hi) * i / 8.0) for i in range(8)]    # p_hi .. just above 1/2
    neg = [-inv(p_hi + (0.5 - p_hi) * i / 7.0) for i in range(7)]
    top = inv(p_hi)
    levels = sorted([v / top for v in pos] + [0.0] + [v / top for v in neg])
    return np.array(levels, dtype=np.float32)
