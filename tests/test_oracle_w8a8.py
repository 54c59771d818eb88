"""Pins of the oracle's W8A8 path: per-row activation quantisation, the integer-accumulated
projection and the W8A8 block."""
import math
from fractions import Fraction

import numpy as np

from oracle import dit, quant
from test_oracle_block import _micro, brute_block
from test_oracle_numeric import to_bf16_exact, to_f32_exact

F32_OVERFLOW = Fraction(2) ** 128


def _half_even(fr: Fraction) -> int:
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def brute_quant_row(row):
    """Exact-arithmetic per-row activation quantisation of float32 inputs (Python floats)."""
    a = max(abs(Fraction(float(v))) for v in row)
    if a == 0:
        return [0] * len(row), 0.0
    inv = to_f32_exact(Fraction(127) / a)
    if abs(inv) >= F32_OVERFLOW:
        return [0] * len(row), 0.0
    s = to_f32_exact(a / 127)
    q = [max(-127, min(127, _half_even(to_f32_exact(Fraction(float(v)) * inv)))) for v in row]
    return q, float(s)


def test_quant_rows_brute_force_and_properties():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((10, 48)).astype(np.float32) * 3
    x[2] = 0.0                                       # all-zero row
    x[3] = np.float32(1e-45)                          # 127 / a overflows: dead row
    x[4] = 0.0
    x[4, 9] = -2.5                                    # one non-zero entry
    x[5] = np.linspace(-1, 1, 48).astype(np.float32)  # ties of the float32 product are possible
    x[6] = np.float32(1e-39) * np.arange(48)          # subnormal inputs, finite inverse
    x[7, :3] = [np.float32(6e4), np.float32(-6e4), np.float32(1.0)]
    q, s = quant.quant_act_rows(x)
    assert q.dtype == np.int8 and s.dtype == np.float32
    for r in range(x.shape[0]):
        bq, bs = brute_quant_row(x[r])
        assert float(s[r]) == bs, r
        assert list(q[r]) == bq, r
    assert not np.any(q == -128)
    assert s[2] == 0 and s[3] == 0 and not q[2].any() and not q[3].any()
    assert q[4, 9] == -127 and np.count_nonzero(q[4]) == 1
    live = s != 0
    assert np.all(np.abs(q[live].astype(int)).max(axis=1) == 127)
    # Reconstruction: at most half a step, plus the rounding of the inverse and the product.
    err = np.abs(quant.dequant(q, s) - x.astype(np.float64))
    step = s.astype(np.float64)[:, None]
    assert np.all(err[live] <= step[live] * (0.5 + 256 * 2.0 ** -24))


def test_int8_matmul_is_exact_integer_sum():
    rng = np.random.default_rng(22)
    qa = rng.integers(-127, 128, (5, 70)).astype(np.int8)
    qw = rng.integers(-127, 128, (6, 70)).astype(np.int8)
    qa[0] = 127
    qw[0] = -127  # the extreme product, summed over k
    sa = rng.random(5).astype(np.float32)
    sw = rng.random(6).astype(np.float32)
    got = quant.int8_matmul(qa, sa, qw, sw)
    for r in range(5):
        for c in range(6):
            acc = sum(int(a) * int(b) for a, b in zip(qa[r], qw[c]))
            exact = Fraction(float(sa[r])) * Fraction(float(sw[c])) * acc
            assert abs(Fraction(float(got[r, c])) - exact) <= abs(exact) * Fraction(1, 2 ** 51), (r, c)
    assert quant.int8_matmul(qa[:1], np.ones(1, np.float32), qw[:1], np.ones(1, np.float32))[0, 0] == -127 * 127 * 70


def brute_w8a8_row(row):
    """Storage rounding to bfloat16, then the brute-force quantise-dequantise of one row."""
    stored = [float(to_bf16_exact(Fraction(float(v)))) for v in row]
    q, s = brute_quant_row(stored)
    return [s * c for c in q]


def test_w8a8_block_matches_brute_force():
    """The oracle's W8A8 block against the loop-level block with the quantisation applied to the
    four projection inputs (normalised input, attention output, second normalised input and the
    SwiGLU product), each written out independently."""
    x, w, mod, geom, nh = _micro(seed=7)
    ref = brute_block(x, w, mod, geom, nh, act_quant=brute_w8a8_row)
    got = dit.block_forward(x, w, mod, geom, nh, act_quant=quant.w8a8_act("bf16"))
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)
    plain = dit.block_forward(x, w, mod, geom, nh)
    e = np.linalg.norm(got - plain) / np.linalg.norm(plain - x)
    assert 1e-4 < e < 0.1  # the quantisation is visible and small


def test_w8a8_hook_sees_the_four_projection_inputs():
    x, w, mod, geom, nh = _micro(seed=8)
    seen = []

    def hook(a):
        seen.append(np.array(a))
        return a
    plain = dit.block_forward(x, w, mod, geom, nh)
    np.testing.assert_array_equal(dit.block_forward(x, w, mod, geom, nh, act_quant=hook), plain)
    n, d = x.shape
    f = w["gate"].shape[0]
    assert [a.shape for a in seen] == [(n, d), (n, d), (n, d), (n, f)]
    # The first is the modulated normalisation of the block input, written out per row.
    shift1, scale1 = mod[0], mod[1]
    for i in range(n):
        r = 1.0 / math.sqrt(sum(v * v for v in x[i]) / d + 1e-6)
        np.testing.assert_allclose(seen[0][i], x[i] * r * (1 + scale1) + shift1, rtol=1e-12, atol=1e-14)
