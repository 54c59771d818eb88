"""Pins of the oracle's rounding primitives against exact rational arithmetic and torch."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import numeric


def frac_round(fr: Fraction, mant_bits: int, emin: int) -> Fraction:
    """Brute force: round a rational to a binary format with ``mant_bits`` significand bits
    (implicit bit included) and minimum normal exponent ``emin``, nearest, ties to even."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)  # subnormals share the minimum exponent
    scale = Fraction(2) ** (e - (mant_bits - 1))
    m = a / scale
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * scale


def to_f32_exact(fr):
    return frac_round(fr, 24, -126)


def to_bf16_exact(fr):
    return frac_round(fr, 8, -126)


def test_bf16_rne_matches_torch_conversion():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(1e3),
        rng.standard_normal(2000).astype(np.float32) * np.float32(1e-38),
        np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, np.inf, -np.inf], np.float32),
    ])
    # Exact ties: low 16 bits == 0x8000, with even and odd kept parts.
    ties = (np.arange(1, 2000, dtype=np.uint32) << np.uint32(16) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    got = numeric.bf16_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.isnan(numeric.bf16_rne(np.array([np.nan], np.float32)))[0]


def test_bf16_from_f64_is_single_correct_rounding():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(3000) * np.exp(rng.uniform(-20, 20, 3000))
    # Values that a float32 double rounding would get wrong: just above a bf16 midpoint by
    # less than a float32 ulp.
    base = np.float32(1.0) + np.float32(2.0 ** -8)  # midpoint between 1 and 1 + 2^-7
    x = np.concatenate([x, [float(base) + 2.0 ** -40, float(base) - 2.0 ** -40, float(base)]])
    got = numeric.bf16_from_f64(x)
    for xi, gi in zip(x, got):
        assert Fraction(float(gi)) == to_bf16_exact(Fraction(float(xi))), xi
    assert got[-3] == np.float32(1.0078125) and got[-2] == np.float32(1.0) and got[-1] == np.float32(1.0)


def test_f32_round_sum_exact():
    rng = np.random.default_rng(3)
    z = rng.standard_normal(4000).astype(np.float32)
    p = (rng.standard_normal(4000).astype(np.float32) * np.float32(1e-8)).astype(np.float64)
    # Constructed midpoints: z + half a float32 ulp, nudged by +-2^-70 below float64 precision.
    zc = np.float32(1.5)
    half = 2.0 ** -24
    z = np.concatenate([z, [zc, zc, zc, zc]]).astype(np.float32)
    p = np.concatenate([p, [half + 2.0 ** -70, half - 2.0 ** -70, half, -half]])
    hi, lo = numeric.two_sum(z.astype(np.float64), p)
    got = numeric.f32_round_sum(hi, lo)
    for zi, pi, gi in zip(z, p, got):
        assert Fraction(float(gi)) == to_f32_exact(Fraction(float(zi)) + Fraction(float(pi)))
    # The nudged midpoints must round apart; a plain float64-then-float32 rounding would not.
    assert got[-4] == np.nextafter(zc, np.float32(2)) and got[-3] == zc and got[-2] == zc
