"""Rounding primitives of the oracle, written from the IEEE-754 definitions.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np


def bf16_rne(x) -> np.ndarray:
    """Round float32 values to bfloat16 (8-bit significand), nearest, ties to even.

    Returned as float32 values that are exactly representable in bfloat16. NaN stays NaN;
    values beyond the largest bfloat16 round to +-inf as IEEE rounding prescribes.
    """
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    out = r.astype(np.uint32).view(np.float32)
    return np.where(np.isnan(f), np.float32(np.nan), out).astype(np.float32)


def round_storage(x, act: str) -> np.ndarray:
    """Round float64 values once to the activation storage type 'bf16' or 'f32' (nearest even).

    Returned as float32 values.
    """
    if act == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    if act == "bf16":
        return bf16_from_f64(x)
    raise ValueError(act)


def bf16_from_f64(x) -> np.ndarray:
    """Correctly round float64 values straight to bfloat16 (single rounding, ties to even)."""
    x = np.asarray(x, dtype=np.float64)
    r = bf16_rne(x.astype(np.float32)).astype(np.float64)  # candidate, may be off by one step
    # Neighbours of the candidate in the bfloat16 grid.
    r32 = r.astype(np.float32)
    up = _bf16_next(r32, +1).astype(np.float64)
    dn = _bf16_next(r32, -1).astype(np.float64)
    best = r.copy()
    for cand in (up, dn):
        d_best = np.abs(x - best)
        d_c = np.abs(x - cand)
        closer = d_c < d_best
        tie = (d_c == d_best) & (cand != best)
        even_c = (_bf16_bits(cand.astype(np.float32)) & 1) == 0
        best = np.where(closer | (tie & even_c), cand, best)
    return np.where(np.isfinite(x), best, r).astype(np.float32)


def _bf16_bits(f32) -> np.ndarray:
    return (np.asarray(f32, np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint32)


def _bf16_next(f32, direction: int) -> np.ndarray:
    """Adjacent bfloat16 value toward +inf (direction=+1) or -inf (-1), finite inputs."""
    b = _bf16_bits(f32).astype(np.int64)
    neg = (b & 0x8000) != 0
    mag = b & 0x7FFF
    # Moving toward +inf increases the magnitude of positives and decreases that of negatives.
    grow = (~neg) if direction > 0 else neg
    mag_new = np.where(grow, mag + 1, mag - 1)
    # Crossing zero: -0 toward +inf is the smallest positive, +0 toward -inf the smallest negative.
    cross = mag == 0
    sign_new = np.where(cross, 0 if direction > 0 else 0x8000, b & 0x8000)
    mag_new = np.where(cross, 1, mag_new)
    bits = (sign_new | mag_new).astype(np.uint32) << np.uint32(16)
    return bits.view(np.float32)


def two_sum(a, b):
    """Knuth's TwoSum on float64: s + e == a + b exactly, s = fl(a + b)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    s = a + b
    bp = s - a
    ap = s - bp
    e = (a - ap) + (b - bp)
    return s, e


def f32_round_sum(hi, lo) -> np.ndarray:
    """Correctly round the exact value ``hi + lo`` to float32 (nearest, ties to even).

    ``hi`` and ``lo`` are float64 with ``hi = fl64(hi + lo)`` (as produced by ``two_sum``).
    Rounding ``hi`` alone is right unless ``hi`` lies exactly halfway between two float32
    numbers and ``lo`` is non-zero; then the sign of ``lo`` picks the neighbour.
    """
    hi = np.asarray(hi, np.float64)
    lo = np.asarray(lo, np.float64)
    r = hi.astype(np.float32)
    r64 = r.astype(np.float64)
    # The float32 neighbour of r on the side where hi lies.
    toward = np.where(hi > r64, np.float32(np.inf), np.float32(-np.inf)).astype(np.float32)
    nb = np.nextafter(r, toward)
    on_mid = (hi != r64) & (hi == (r64 + nb.astype(np.float64)) / 2.0)
    lower = np.minimum(r, nb)
    upper = np.maximum(r, nb)
    fixed = np.where(lo > 0, upper, np.where(lo < 0, lower, r))
    return np.where(on_mid & np.isfinite(hi), fixed, r).astype(np.float32)
