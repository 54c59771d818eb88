"""Pins of where the oracle's block loop reduces tokens, and of core reuse inside that loop.

Reading pinned (jdon.com, "330亿参数是什么概念"; siami.tw, "速度與品質的可調旋鈕" control
table, row "Token 縮減": horizontal video tokens are merged in the middle blocks): with token
reduction over blocks tf..tl (0-based, inclusive), blocks 0..tf-1 run on the full sequence, the
video pairs are merged right before block tf, blocks tf..tl run on the merged sequence, and the
pairs are written back right before block tl+1 (or after the last block when tl is the last).

The expected results here are built as an explicit composition -- a list of the operations in
order, taken from ranges -- not by a loop that checks block indices, so that an off-by-one in
``sampler.dit_eval`` (merging after block tf, unmerging before tl or after tl+1, skipping the
final unmerge) fails.
"""
import numpy as np
import pytest

from oracle import dit, sampler, tokred
from oracle.geometry import Geometry

GEOM = Geometry(1, 2, 4, 2, 3)  # 8 video (4 merged), 2 audio, 3 text tokens


def plan(n_blocks, tf, tl):
    """The operations of one evaluation, in order: ('block', b, merged), ('merge',), ('unmerge',)."""
    if tf < 0:
        return [("block", b, False) for b in range(n_blocks)]
    return ([("block", b, False) for b in range(0, tf)] + [("merge",)] +
            [("block", b, True) for b in range(tf, tl + 1)] + [("unmerge",)] +
            [("block", b, False) for b in range(tl + 1, n_blocks)])


def run_plan(ops, x, block_fn, act):
    g = GEOM
    for op in ops:
        if op[0] == "merge":
            x, g = tokred.merge(x, g, act), g.as_merged()
        elif op[0] == "unmerge":
            x, g = tokred.unmerge(x, g.as_unmerged()), g.as_unmerged()
        else:
            assert g.merged == op[2]
            x = block_fn(op[1], x, g)
    return x


def fake_block(b, x, g):
    """A block that is not pair-preserving: every row gets its own, block-dependent change."""
    n = x.shape[0]
    assert n == g.n_tokens
    ramp = np.arange(n, dtype=np.float64)[:, None] * 0.01 + np.arange(x.shape[1])[None, :] * 0.001
    return 1.25 * x + (b + 1) * ramp + (0.5 if g.merged else 0.0)


CASES = [(-1, -1), (0, 5), (0, 0), (2, 2), (1, 4), (3, 5), (5, 5), (0, 4), (1, 5)]


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("tf,tl", CASES)
def test_reduction_placement_against_explicit_plan(monkeypatch, act, tf, tl):
    n_blocks = 6
    log = []

    def recorded(x, w, mod, g, n_heads, rows=None, act_quant=None):
        log.append(("block", w["id"], g.merged))
        return fake_block(w["id"], np.asarray(x, np.float64), g)

    monkeypatch.setattr(dit, "block_forward", recorded)
    x0 = np.random.default_rng(3).standard_normal((GEOM.n_tokens, 4))
    if act == "bf16":
        from oracle.numeric import round_storage
        x0 = round_storage(x0, "bf16").astype(np.float64)
    blocks = [{"id": b} for b in range(n_blocks)]
    got = sampler.dit_eval(x0, blocks, [None] * n_blocks, GEOM, 1, act, tf, tl)
    ops = plan(n_blocks, tf, tl)
    assert log == [op for op in ops if op[0] == "block"]
    want = run_plan(ops, x0, fake_block, act)
    np.testing.assert_array_equal(got, want)


def _micro_stack(n_blocks, live, seed=11, d=16, nh=2, f=24):
    """Random micro blocks; every block except `live` has zero gates (is the identity)."""
    rng = np.random.default_rng(seed)
    blocks, mods = [], []
    for b in range(n_blocks):
        blocks.append({"qkv": rng.standard_normal((3 * d, d)) * 0.4, "out": rng.standard_normal((d, d)) * 0.3,
                       "gate": rng.standard_normal((f, d)) * 0.3, "up": rng.standard_normal((f, d)) * 0.3,
                       "down": rng.standard_normal((d, f)) * 0.3})
        m = rng.standard_normal((6, d)) * 0.2
        m[2] += 1
        m[5] += 1
        if b != live:
            m[2] = 0.0
            m[5] = 0.0
        mods.append(m)
    return blocks, mods, nh


def pair_constant(x, g):
    v = x[: g.n_video]
    return bool(np.all(v[0::2] == v[1::2]))


@pytest.mark.parametrize("tf,tl", [(1, 3), (0, 4), (2, 2), (4, 4)])
def test_single_live_block_runs_in_the_right_geometry(tf, tl):
    """Real blocks, all but one with zero gates: the output tells which geometry the live block
    ran in. Live block before the range: its own output, then merge and unmerge. Inside: merge,
    the block on the merged sequence (the audio and text rows see fewer keys), unmerge. After:
    merge, unmerge, then the block. The video rows come out pair-constant exactly when the live
    block lies at or before the last reduced block."""
    n_blocks = 5
    x0 = np.random.default_rng(5).standard_normal((GEOM.n_tokens, 16))
    for live in range(n_blocks):
        blocks, mods, nh = _micro_stack(n_blocks, live)
        got = sampler.dit_eval(x0, blocks, mods, GEOM, nh, "f32", tf, tl)
        run = lambda x, g: dit.block_forward(x, blocks[live], mods[live], g, nh)
        mg = GEOM.as_merged()
        if live < tf:
            want = tokred.unmerge(tokred.merge(run(x0, GEOM), GEOM, "f32"), GEOM)
        elif live <= tl:
            want = tokred.unmerge(run(tokred.merge(x0, GEOM, "f32"), mg), GEOM)
        else:
            want = run(tokred.unmerge(tokred.merge(x0, GEOM, "f32"), GEOM), GEOM)
        np.testing.assert_array_equal(got, want)
        assert pair_constant(got, GEOM) == (live <= tl)
        # The three placements give different results (the check above could not pass by luck).
        alt = run(x0, GEOM)
        assert not np.array_equal(got, alt)


def test_core_reuse_with_token_reduction():
    """Core inside the reduced range: the kept change has the merged row count; a reused core
    adds it to the merged activations. Straddling a reduction boundary is rejected."""
    n_blocks = 6
    rng = np.random.default_rng(9)
    blocks, mods, nh = _micro_stack(n_blocks, live=-1)
    for m in mods:  # all blocks live
        m[2] = 1.0 + 0.1 * rng.standard_normal(m.shape[1])
        m[5] = 1.0 + 0.1 * rng.standard_normal(m.shape[1])
    x0 = np.random.default_rng(6).standard_normal((GEOM.n_tokens, 16))
    tf, tl = 1, 4
    mg = GEOM.as_merged()
    blk = lambda b, x, g: dit.block_forward(x, blocks[b], mods[b], g, nh)
    # Fresh core 2..3 inside 1..4: identical to the plain reduced stack; delta over the core.
    plain = sampler.dit_eval(x0, blocks, mods, GEOM, nh, "f32", tf, tl)
    out, delta = sampler.dit_eval(x0, blocks, mods, GEOM, nh, "f32", tf, tl, core=(2, 3, True, None))
    np.testing.assert_array_equal(out, plain)
    xm = blk(1, tokred.merge(blk(0, x0, GEOM), GEOM, "f32"), mg)
    np.testing.assert_array_equal(delta, blk(3, blk(2, xm, mg), mg) - xm)
    assert delta.shape == (mg.n_tokens, 16)
    # Reused core: the merged activations before block 2 plus the kept change, then block 4.
    out2, d2 = sampler.dit_eval(x0, blocks, mods, GEOM, nh, "f32", tf, tl, core=(2, 3, False, delta * 0.5))
    want = blk(5, tokred.unmerge(blk(4, xm + delta * 0.5, mg), GEOM), GEOM)
    np.testing.assert_array_equal(out2, want)
    np.testing.assert_array_equal(d2, delta * 0.5)
    # A core wholly before the range keeps an unmerged change.
    _, d3 = sampler.dit_eval(x0, blocks, mods, GEOM, nh, "f32", 2, 4, core=(0, 1, True, None))
    assert d3.shape == (GEOM.n_tokens, 16)
    # Straddling cores are rejected.
    for core in ((0, 1), (4, 5), (0, 5)):
        with pytest.raises(ValueError):
            sampler.dit_eval(x0, blocks, mods, GEOM, nh, "f32", tf, tl, core=(*core, True, None))
