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


# ---------------------------------------------------------------- schedule and sampler variants
def test_sigma_schedules():
    for s in (1, 4, 7, 20):
        np.testing.assert_array_equal(sampler.sigma_schedule("linear", s), sampler.sigma_grid(s))
        np.testing.assert_array_equal(sampler.sigma_schedule("power", s, 1.0), sampler.sigma_grid(s))
        for kind, p in (("power", 2.0), ("power", 3.0), ("power", 0.5), ("linear_terminal", 29)):
            g = sampler.sigma_schedule(kind, s, p)
            assert len(g) == s + 1 and g[0] == 1.0 and g[-1] == 0.0 and np.all(np.diff(g) < 0)
    # Dyadic grids are exact: quadratic and cubic warps at S = 4.
    np.testing.assert_array_equal(sampler.sigma_schedule("power", 4, 2.0), [1, 9 / 16, 1 / 4, 1 / 16, 0])
    np.testing.assert_array_equal(sampler.sigma_schedule("power", 4, 3.0), [1, 27 / 64, 1 / 8, 1 / 64, 0])
    # A few-step run on the 20-step linear base: 1, .95, .9, .85, then the terminal 0.
    g = sampler.sigma_schedule("linear_terminal", 4, 20)
    np.testing.assert_array_equal(g[:4], sampler.sigma_grid(20)[:4])
    assert g[4] == 0.0
    with pytest.raises(ValueError):
        sampler.sigma_schedule("linear_terminal", 8, 4)


def test_velocity_extrapolation():
    assert sampler.extrapolation_weight(0.625, 0.75, 1.0) == np.float32(0.5)
    assert sampler.extrapolation_weight(0.75, 0.75, 1.0) == 0
    rng = np.random.default_rng(11)
    va = rng.standard_normal(500).astype(np.float32)
    vb = rng.standard_normal(500).astype(np.float32)
    # w = 0 holds, equal velocities extrapolate to themselves.
    np.testing.assert_array_equal(sampler.extrapolate_velocity(va, vb, 0.0), va)
    np.testing.assert_array_equal(sampler.extrapolate_velocity(va, va, 0.37), va)
    # One rounding of the exact w * float32(va - vb) + va.
    w = np.float32(0.3718)
    got = sampler.extrapolate_velocity(va, vb, w)
    for a, b, g in zip(va[:200], vb[:200], got[:200]):
        dd = np.float32(a) - np.float32(b)
        exact = Fraction(float(w)) * Fraction(float(dd)) + Fraction(float(a))
        assert Fraction(float(g)) == to_f32_exact(exact)
    # A velocity linear in sigma (dyadic values) is reproduced exactly.
    A = np.float32(0.375) * np.arange(-8, 8, dtype=np.float32)
    Bv = np.float32(1.25) * np.arange(16, dtype=np.float32)
    v_at = lambda sg: A + Bv * np.float32(sg)
    w = sampler.extrapolation_weight(0.5, 0.75, 1.0)
    np.testing.assert_array_equal(sampler.extrapolate_velocity(v_at(0.75), v_at(1.0), w), v_at(0.5))


def test_cond_rows_brute_force():
    g = Geometry(5, 3, 4, 7, 9)
    for cf, cl in ((0, 0), (1, 0), (0, 1), (1, 1), (2, 3), (5, 0)):
        m = sampler.cond_rows(g, cf, cl)
        assert m.shape == (g.n_video + g.n_audio,)
        for r in range(g.n_video + g.n_audio):
            t = r // (g.grid_h * g.grid_w)
            expect = r < g.n_video and (t < cf or t >= g.frames - cl)
            assert bool(m[r]) == expect
        assert m.sum() == min(cf + cl, g.frames) * g.grid_h * g.grid_w


def _tiny_chain_setup():
    from synth import TINY, block_weights, modulation, initial_state, text_rows
    w = TINY.replace(n_blocks=4)
    geom = Geometry(w.frames, w.grid_h, w.grid_w, w.n_audio, w.n_text)
    blocks = [block_weights(w, b) for b in range(w.n_blocks)]
    mods = [modulation(w, 0, b) for b in range(w.n_blocks)]
    return w, geom, blocks, mods, initial_state(w), text_rows(w)


def test_fixed_condition_rows_are_held():
    w, geom, blocks, mods, z, c = _tiny_chain_setup()
    plain = sampler.denoise_step_full(z, c, None, blocks, mods, geom, w.n_heads, "f32", 0, 4, 1, 1.0, 0.75)
    held = sampler.denoise_step_full(z, c, None, blocks, mods, geom, w.n_heads, "f32", 0, 4, 1, 1.0, 0.75,
                                     cond_first=1)
    fixed = sampler.cond_rows(geom, 1, 0)
    assert fixed.any() and not fixed.all()
    np.testing.assert_array_equal(held[0][fixed], z[fixed])
    np.testing.assert_array_equal(held[0][~fixed], plain[0][~fixed])
    np.testing.assert_array_equal(held[1], plain[1])  # the DiT saw the same input


def test_core_reuse_closed_forms():
    w, geom, blocks, mods, z, c = _tiny_chain_setup()
    x0 = np.concatenate([z, c]).astype(np.float64)
    # Core fresh on every step is the plain stack, and its delta is what the core blocks add.
    plain = sampler.dit_eval(x0, blocks, mods, geom, w.n_heads, "f32")
    out, delta = sampler.dit_eval(x0, blocks, mods, geom, w.n_heads, "f32", core=(1, 2, True, None))
    np.testing.assert_array_equal(out, plain)
    x1 = dit_block(x0, blocks[0], mods[0], geom, w.n_heads)
    x3 = dit_block(dit_block(x1, blocks[1], mods[1], geom, w.n_heads), blocks[2], mods[2], geom, w.n_heads)
    np.testing.assert_allclose(delta, x3 - x1, rtol=0, atol=0)
    # Outer blocks that are the identity (zero gates): a reused core adds the kept delta to the
    # current input, whatever it is.
    idm = [m.copy() for m in mods]
    for b in (0, 3):
        idm[b][2] = 0
        idm[b][5] = 0
    _, d_kept = sampler.dit_eval(x0, blocks, idm, geom, w.n_heads, "f32", core=(1, 2, True, None))
    x_other = x0 * 0.5 + 0.25
    out2, d2 = sampler.dit_eval(x_other, blocks, idm, geom, w.n_heads, "f32", core=(1, 2, False, d_kept))
    np.testing.assert_array_equal(out2, x_other + d_kept)
    np.testing.assert_array_equal(d2, d_kept)
    # Through the step: core period 2 at step 1 of 4 reuses, step 2 refreshes.
    zs, v, _, dk = sampler.denoise_step_full(z, c, None, blocks, mods, geom, w.n_heads, "f32", 0, 4, 1,
                                             1.0, 0.75, core=(2, 1, 2, None))
    z2, v2, _, dk2 = sampler.denoise_step_full(zs, c, v, blocks, mods, geom, w.n_heads, "f32", 1, 4, 1,
                                               0.75, 0.5, core=(2, 1, 2, dk))
    np.testing.assert_array_equal(dk2, dk)
    xin = np.concatenate([zs, c]).astype(np.float64)
    front = dit_block(xin, blocks[0], mods[0], geom, w.n_heads)
    tail = dit_block(front + dk, blocks[3], mods[3], geom, w.n_heads)
    np.testing.assert_array_equal(v2, tail[: geom.n_video + geom.n_audio].astype(np.float32))


def dit_block(x, wts, mod, geom, n_heads):
    from oracle import dit
    return dit.block_forward(x, wts, mod, geom, n_heads)
