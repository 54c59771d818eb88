"""Pins of the oracle's sampler, token reduction and int8 packing."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import quant, sampler, tokred
from oracle.geometry import Geometry
from test_oracle_numeric import to_f32_exact, to_bf16_exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- schedule and reuse
def test_fresh_counts_printed_on_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "fresh_counts.json")))
    s = g["n_steps"]
    for r, count in g["fresh_by_reuse"].items():
        assert sum(sampler.is_fresh(i, s, int(r)) for i in range(s)) == count
    # The first and the last step always evaluate the DiT.
    for r in (1, 2, 3, 4, 7):
        assert sampler.is_fresh(0, s, r) and sampler.is_fresh(s - 1, s, r)


def test_sigma_grid():
    for s in (1, 4, 20, 50):
        sg = sampler.sigma_grid(s)
        assert sg[0] == 1.0 and sg[-1] == 0.0 and len(sg) == s + 1
        assert np.all(np.diff(sg) < 0)
        total = sum(float(sampler.sigma_delta(sg[i], sg[i + 1])) for i in range(s))
        assert abs(total + 1.0) < 1e-6
    np.testing.assert_array_equal(sampler.sigma_grid(4), [1.0, 0.75, 0.5, 0.25, 0.0])
    assert sampler.sigma_grid(20)[1] == np.float32(0.95)


# ---------------------------------------------------------------- Euler
def test_euler_is_correctly_rounded():
    rng = np.random.default_rng(7)
    z = rng.standard_normal(3000).astype(np.float32)
    v = rng.standard_normal(3000).astype(np.float32)
    for delta in (np.float32(-0.05), np.float32(-0.25), np.float32(-0.0500001)):
        got = sampler.euler_update(z, delta, v)
        for zi, vi, gi in zip(z[:600], v[:600], got[:600]):
            exact = Fraction(float(zi)) + Fraction(float(delta)) * Fraction(float(vi))
            assert Fraction(float(gi)) == to_f32_exact(exact)


def test_euler_same_sigma_is_noop_and_zero_velocity():
    rng = np.random.default_rng(8)
    z = rng.standard_normal(1000).astype(np.float32)
    v = rng.standard_normal(1000).astype(np.float32)
    d = sampler.sigma_delta(0.35, 0.35)
    assert d == 0
    np.testing.assert_array_equal(sampler.euler_update(z, d, v).view(np.uint32), z.view(np.uint32))
    np.testing.assert_array_equal(sampler.euler_update(z, np.float32(-0.1), np.zeros(1000)), z)


# ---------------------------------------------------------------- token reduction
def brute_merge_index(g: Geometry):
    """(t, y, m) -> merged row, and its two source rows, from nested loops."""
    out = []
    for t in range(g.frames):
        for y in range(g.grid_h):
            for m in range(g.grid_w // 2):
                src0 = (t * g.grid_h + y) * g.grid_w + 2 * m
                out.append((src0, src0 + 1))
    return out


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_merge_unmerge(act):
    g = Geometry(2, 3, 6, 4, 5)
    rng = np.random.default_rng(9)
    x = rng.standard_normal((g.n_tokens, 8)).astype(np.float32)
    if act == "bf16":
        x = to_bf16_values(x)
    xm = tokred.merge(x, g, act)
    assert xm.shape == (g.n_tokens - g.n_video // 2, 8)
    for p, (a, b) in enumerate(brute_merge_index(g)):
        for c in range(8):
            mean = (Fraction(float(x[a, c])) + Fraction(float(x[b, c]))) / 2
            want = to_bf16_exact(mean) if act == "bf16" else to_f32_exact(mean)
            assert Fraction(float(xm[p, c])) == want
    np.testing.assert_array_equal(xm[g.n_video // 2:], x[g.n_video:])
    # unmerge then merge is the identity on any merged input.
    np.testing.assert_array_equal(tokred.merge(tokred.unmerge(xm, g), g, act), xm)
    # merge then unmerge is the identity on pair-constant inputs.
    xpc = tokred.unmerge(xm, g)
    np.testing.assert_array_equal(tokred.unmerge(tokred.merge(xpc, g, act), g), xpc)


def test_merge_counts():
    assert Geometry(6, 32, 32, 256, 512).as_merged().n_video == 3072
    assert Geometry(6, 30, 54, 256, 512).as_merged().n_video == 4860
    with pytest.raises(ValueError):
        Geometry(1, 3, 5, 0, 0).as_merged()


def to_bf16_values(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).float().numpy()


# ---------------------------------------------------------------- int8 packing
def brute_pack_row(row):
    """Exact-arithmetic packing of one row (bfloat16 inputs as Python floats)."""
    a = max(abs(Fraction(float(w))) for w in row)
    if a == 0:
        return [0] * len(row), 0.0
    s = to_bf16_exact(to_f32_exact(a / 127))
    if s == 0:
        return [0] * len(row), 0.0
    q = []
    for w in row:
        quot = to_f32_exact(Fraction(float(w)) / s)
        fl = quot.numerator // quot.denominator
        rem = quot - fl
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
            fl += 1
        q.append(max(-127, min(127, fl)))
    return q, float(s)


def test_pack_int8_brute_force_and_properties():
    rng = np.random.default_rng(10)
    w = to_bf16_values(rng.standard_normal((12, 40)).astype(np.float32) * 0.02)
    w[3] = 0.0  # all-zero row
    w[4] = to_bf16_values(np.full(40, 1e-40, np.float32))  # scale underflows to 0
    w[5, 7] = to_bf16_values(np.array([-3.0], np.float32))[0]  # single large negative
    w[6] = to_bf16_values(np.linspace(-1, 1, 40).astype(np.float32))
    q, s = quant.pack_int8(w)
    assert q.dtype == np.int8 and s.dtype == np.float32
    for r in range(w.shape[0]):
        bq, bs = brute_pack_row(w[r])
        assert s[r] == bs, r
        assert list(q[r]) == bq, r
    assert np.all(np.abs(q.astype(int)) <= 127) and not np.any(q == -128)
    nz = s != 0
    assert np.all(np.abs(q[nz].astype(int)).max(axis=1) == 127)
    assert s[3] == 0 and s[4] == 0 and not q[3].any() and not q[4].any()
    # Reconstruction error at most half a step.
    err = np.abs(quant.dequant(q, s) - w.astype(np.float64))
    assert np.all(err <= s.astype(np.float64)[:, None] / 2 + 1e-30)
    # Scales are bfloat16 values.
    np.testing.assert_array_equal(to_bf16_values(s), s)


# ---------------------------------------------------------------- denoise chain structure
def test_denoise_step_with_identity_dit():
    """All gates 0 make every block the identity: v is the rounded state itself."""
    from synth import TINY, block_weights, modulation, initial_state, text_rows
    w = TINY.replace(n_blocks=1)
    geom = Geometry(w.frames, w.grid_h, w.grid_w, w.n_audio, w.n_text)
    blocks = [block_weights(w, 0)]
    mods = [modulation(w, 0, 0)]
    mods[0][2] = 0
    mods[0][5] = 0
    z = initial_state(w)
    c = text_rows(w)
    for act in ("f32", "bf16"):
        z1, v = sampler.denoise_step(z, c, None, blocks, mods, geom, w.n_heads, act, 0, 20, 1, 1.0, 0.95)
        vr = z if act == "f32" else to_bf16_values(z)
        np.testing.assert_array_equal(v, vr)
        np.testing.assert_array_equal(z1, sampler.euler_update(z, np.float32(0.95) - np.float32(1.0), vr))


def test_reused_step_uses_cache_only():
    from synth import TINY, block_weights, modulation, initial_state, text_rows
    w = TINY
    geom = Geometry(w.frames, w.grid_h, w.grid_w, w.n_audio, w.n_text)
    z = initial_state(w)
    cache = np.random.default_rng(1).standard_normal(z.shape).astype(np.float32)
    # Step 1 of 20 with reuse 2 is not fresh: blocks are never touched (None would fail).
    z1, v = sampler.denoise_step(z, text_rows(w), cache, None, None, geom, w.n_heads, "f32", 1, 20, 2, 0.95, 0.9)
    np.testing.assert_array_equal(v, cache)
    np.testing.assert_array_equal(z1, sampler.euler_update(z, sampler.sigma_delta(0.95, 0.9), cache))
