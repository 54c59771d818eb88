"""Pins of the oracle's block arithmetic: closed forms, invariants and loop-level brute force."""
import math

import numpy as np
import pytest

from oracle import dit
from oracle.geometry import Geometry


# ---------------------------------------------------------------- modulated RMSNorm
def test_rmsnorm_closed_forms():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 48))
    zero = np.zeros(48)
    y = dit.rms_norm_mod(x, zero, zero)
    ms = np.mean(x * x, axis=1)
    # With shift = scale = 0 the output has mean square ms / (ms + eps) exactly.
    np.testing.assert_allclose(np.mean(y * y, axis=1), ms / (ms + 1e-6), rtol=1e-13)
    # scale = -1 wipes the normalised part: the output is the shift.
    shift = rng.standard_normal(48)
    np.testing.assert_array_equal(dit.rms_norm_mod(x, shift, -np.ones(48)), np.broadcast_to(shift, x.shape))
    # A constant row c maps to c / sqrt(c^2 + eps).
    c = 0.37
    yc = dit.rms_norm_mod(np.full((1, 48), c), zero, zero)
    np.testing.assert_allclose(yc, c / math.sqrt(c * c + 1e-6), rtol=1e-14)
    # (1 + scale) multiplies, shift adds, per channel.
    sc = rng.standard_normal(48)
    np.testing.assert_allclose(dit.rms_norm_mod(x, shift, sc), y * (1 + sc) + shift, rtol=1e-13)


# ---------------------------------------------------------------- 3D RoPE
def _one_head_unit(dh, i):
    z = np.zeros((1, dh))
    z[0, i] = 1.0
    return z


@pytest.mark.parametrize("dh", [64, 128])
def test_rope_frequencies_at_fixed_points(dh):
    """Within a chunk of size D, pair k = 0 turns by pos, k = D/8 by pos/10, k = D/4 by pos/100."""
    chunks = dit.rope_chunks(dh)
    assert [c[2] for c in chunks] == [dh // 4, 3 * dh // 8, 3 * dh // 8]
    for axis, off, size in chunks:
        for k, omega in ((0, 1.0), (size // 8, 0.1), (size // 4, 0.01)):
            if (size // 8) * 8 != size and k == size // 8:
                continue
            pos = np.zeros((1, 3))
            pos[0, axis] = 7.0
            z = _one_head_unit(dh, off + 2 * k)
            r = dit.rope(z, pos, np.array([True]), 1)
            want = np.zeros(dh)
            want[off + 2 * k] = math.cos(7.0 * omega)
            want[off + 2 * k + 1] = math.sin(7.0 * omega)
            np.testing.assert_allclose(r[0], want, atol=1e-14)


def test_rope_axis_assignment_and_identity():
    dh, nh = 64, 2
    rng = np.random.default_rng(1)
    z = rng.standard_normal((5, nh * dh))
    zero = np.zeros((5, 3))
    np.testing.assert_array_equal(dit.rope(z, zero, np.ones(5, bool), nh), z)
    # A position on one axis moves only that axis' chunk.
    for axis, off, size in dit.rope_chunks(dh):
        pos = np.zeros((5, 3))
        pos[:, axis] = 3.0
        r = dit.rope(z, pos, np.ones(5, bool), nh)
        moved = np.zeros(dh, bool)
        moved[off:off + size] = True
        moved = np.tile(moved, nh)
        np.testing.assert_array_equal(r[:, ~moved], z[:, ~moved])
        assert np.all(np.abs(r[:, moved] - z[:, moved]).max(axis=0) > 0)
    # Unrotated rows pass through.
    pos = rng.uniform(0, 9, (5, 3))
    rot = np.array([True, False, True, False, False])
    r = dit.rope(z, pos, rot, nh)
    np.testing.assert_array_equal(r[~rot], z[~rot])


def test_rope_norm_and_relative_position():
    dh, nh = 128, 3
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, nh * dh))
    k = rng.standard_normal((1, nh * dh))
    p1, p2 = np.array([[2.0, 5.0, 7.5]]), np.array([[1.0, 3.0, 4.0]])
    shift = np.array([[3.0, -2.0, 10.5]])
    on = np.array([True])
    rq = dit.rope(q, p1, on, nh)
    # Each pair keeps its norm.
    np.testing.assert_allclose(np.hypot(rq[0, 0::2], rq[0, 1::2]), np.hypot(q[0, 0::2], q[0, 1::2]), rtol=1e-13)
    # <R(p1) q, R(p2) k> depends only on p1 - p2, per head.
    a = dit.rope(q, p1, on, nh) * dit.rope(k, p2, on, nh)
    b = dit.rope(q, p1 + shift, on, nh) * dit.rope(k, p2 + shift, on, nh)
    for h in range(nh):
        sl = slice(h * dh, (h + 1) * dh)
        assert abs(a[0, sl].sum() - b[0, sl].sum()) < 1e-10


def test_positions_layout():
    g = Geometry(2, 3, 4, 5, 6)
    pos, rot = g.positions()
    assert pos.shape == (24 + 11, 3) and rot.sum() == 24
    for t in range(2):
        for y in range(3):
            for x in range(4):
                assert tuple(pos[(t * 3 + y) * 4 + x]) == (t, y, x)
    gm = g.as_merged()
    pos, rot = gm.positions()
    assert gm.n_video == 12 and rot.sum() == 12 and len(pos) == 23
    for t in range(2):
        for y in range(3):
            for m in range(2):
                assert tuple(pos[(t * 3 + y) * 2 + m]) == (t, y, 2 * m + 0.5)


# ---------------------------------------------------------------- attention
def brute_attention(q, k, v, nh):
    m, d = q.shape
    n = k.shape[0]
    dh = d // nh
    out = np.zeros((m, d))
    for h in range(nh):
        for i in range(m):
            logits = []
            for j in range(n):
                s = 0.0
                for c in range(dh):
                    s += q[i, h * dh + c] * k[j, h * dh + c]
                logits.append(s / math.sqrt(dh))
            mx = max(logits)
            w = [math.exp(l - mx) for l in logits]
            tot = sum(w)
            for c in range(dh):
                out[i, h * dh + c] = sum(w[j] * v[j, h * dh + c] for j in range(n)) / tot
    return out


def test_attention_brute_force_and_invariants():
    rng = np.random.default_rng(3)
    nh, dh, n, m = 2, 8, 11, 5
    q = rng.standard_normal((m, nh * dh)) * 2
    k = rng.standard_normal((n, nh * dh)) * 2
    v = rng.standard_normal((n, nh * dh))
    np.testing.assert_allclose(dit.attention(q, k, v, nh), brute_attention(q, k, v, nh), rtol=1e-12, atol=1e-13)
    # Rows of P sum to one: V == 1 gives O == 1.
    np.testing.assert_allclose(dit.attention(q, k, np.ones_like(v), nh), 1.0, rtol=1e-14)
    # Identical keys give the mean of V.
    kk = np.tile(k[:1], (n, 1))
    np.testing.assert_allclose(dit.attention(q, kk, v, nh), np.tile(v.mean(0), (m, 1)), rtol=1e-12)
    # Jointly permuting key and value rows changes nothing.
    perm = rng.permutation(n)
    np.testing.assert_allclose(dit.attention(q, k[perm], v[perm], nh), dit.attention(q, k, v, nh), rtol=1e-12)
    # Huge logits do not overflow (max subtraction).
    assert np.all(np.isfinite(dit.attention(q * 1e3, k * 1e3, v, nh)))


def test_silu_values():
    np.testing.assert_allclose(dit.silu(np.array([0.0, 1.0, -1.0, 40.0, -40.0])),
                               [0.0, 0.7310585786300049, -0.2689414213699951, 40.0, -40.0 * math.exp(-40.0)],
                               rtol=1e-12, atol=1e-30)


# ---------------------------------------------------------------- whole block
def brute_block(x, w, mod, geom, nh, act_quant=None):
    """Loop-level block from the stated definitions (no shared code with the oracle).
    act_quant, if given, maps one projection-input row to its quantised values."""
    aq = act_quant or (lambda row: row)
    n, d = x.shape
    dh = d // nh
    f = w["gate"].shape[0]
    shift1, scale1, gate1, shift2, scale2, gate2 = mod

    def norm(row, shift, scale):
        ms = sum(v * v for v in row) / d
        r = 1.0 / math.sqrt(ms + 1e-6)
        return [row[c] * r * (1 + scale[c]) + shift[c] for c in range(d)]

    def matvec(wm, vec):
        return [sum(wm[o][c] * vec[c] for c in range(len(vec))) for o in range(len(wm))]

    # positions
    coords = []
    for t in range(geom.frames):
        for yy in range(geom.grid_h):
            for xx in range(geom.grid_w):
                coords.append((t, yy, xx))
    sizes = [dh // 4, 3 * dh // 8, dh - dh // 4 - 3 * dh // 8]

    def rot(vec, i):
        if i >= len(coords):
            return vec
        out = list(vec)
        for h in range(nh):
            base = h * dh
            for a in range(3):
                for kk in range(sizes[a] // 2):
                    ang = coords[i][a] * 10000.0 ** (-2.0 * kk / sizes[a])
                    j = base + 2 * kk
                    p, r_ = vec[j], vec[j + 1]
                    out[j] = p * math.cos(ang) - r_ * math.sin(ang)
                    out[j + 1] = p * math.sin(ang) + r_ * math.cos(ang)
                base += sizes[a]
        return out

    ys = [aq(norm(list(x[i]), shift1, scale1)) for i in range(n)]
    wq, wk, wv = w["qkv"][:d], w["qkv"][d:2 * d], w["qkv"][2 * d:]
    qs = [rot(matvec(wq, ys[i]), i) for i in range(n)]
    ks = [rot(matvec(wk, ys[i]), i) for i in range(n)]
    vs = [matvec(wv, ys[i]) for i in range(n)]
    att = brute_attention(np.array(qs), np.array(ks), np.array(vs), nh)
    out = np.zeros((n, d))
    for i in range(n):
        ao = matvec(w["out"], aq(list(att[i])))
        x1 = [x[i, c] + gate1[c] * ao[c] for c in range(d)]
        y2 = aq(norm(x1, shift2, scale2))
        g = matvec(w["gate"], y2)
        u = matvec(w["up"], y2)
        hmid = aq([g[j] / (1 + math.exp(-g[j])) * u[j] for j in range(f)])
        mo = matvec(w["down"], hmid)
        out[i] = [x1[c] + gate2[c] * mo[c] for c in range(d)]
    return out


def _micro(seed=4, d=16, nh=2, f=24, geom=Geometry(1, 2, 4, 2, 3)):
    rng = np.random.default_rng(seed)
    n = geom.n_tokens
    x = rng.standard_normal((n, d))
    w = {"qkv": rng.standard_normal((3 * d, d)) * 0.4, "out": rng.standard_normal((d, d)) * 0.3,
         "gate": rng.standard_normal((f, d)) * 0.3, "up": rng.standard_normal((f, d)) * 0.3,
         "down": rng.standard_normal((d, f)) * 0.3}
    mod = rng.standard_normal((6, d)) * 0.2
    mod[2] += 1
    mod[5] += 1
    return x, w, mod, geom, nh


def test_block_matches_brute_force():
    x, w, mod, geom, nh = _micro()
    ref = brute_block(x, w, mod, geom, nh)
    got = dit.block_forward(x, w, mod, geom, nh)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)
    # Sampled rows equal the corresponding full-output rows.
    rows = np.array([0, 3, 8, 12])
    np.testing.assert_allclose(dit.block_forward(x, w, mod, geom, nh, rows=rows), got[rows], rtol=1e-13)


def test_block_zero_gates_is_identity_and_zero_wo():
    x, w, mod, geom, nh = _micro(seed=5)
    m0 = mod.copy()
    m0[2] = 0.0
    m0[5] = 0.0
    np.testing.assert_array_equal(dit.block_forward(x, w, m0, geom, nh), x)
    w0 = dict(w, out=np.zeros_like(w["out"]))
    m1 = mod.copy()
    m1[5] = 0.0
    np.testing.assert_array_equal(dit.block_forward(x, w0, m1, geom, nh), x)


def test_block_flops_formula():
    # 2*N*d*(3d + d + 2F + F) + 4*N^2*d for the 6912-token, d = 6144, F = 24576 block.
    assert dit.block_flops(6912, 6144, 24576) == pytest.approx(9.5236e12, rel=1e-4)
