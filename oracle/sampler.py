"""Denoising schedule, whole-velocity reuse and the flow-matching Euler step (test
infrastructure only).

Pages: siami.tw, "速度與品質的可調旋鈕" control table -- ``--steps`` names the number of real
denoising passes, and whole-denoiser reuse 1 / 2 / 3 gives 20 / 11 / 8 fresh DiT evaluations
at 20 steps; the same section says the few-step schedule is a linear base grid with one
terminal endpoint. siami.tw, "技術亮點 › 1." lists the schedule as its own module. Readings
taken where the pages are silent:

* sigma grid: ``sigma_i = float32(1 - i/S)``, i = 0..S (linear from 1 to 0);
* step i is fresh iff ``i % reuse == 0`` or ``i == S - 1`` (this reproduces the printed
  20 / 11 / 8 counts; so does the end-aligned variant, so the choice is a convention);
* the state z holds the video and audio rows in float32; text rows are fixed conditioning:
  never updated and fed unchanged to every evaluation;
* a fresh evaluation feeds ``[round_act(z); c]`` through the blocks, merging video pairs before
  block ``tr_first`` and unmerging before block ``tr_last + 1`` (or after the last block); the
  velocity v is the output's video+audio rows rounded to the activation storage type, and it
  is kept for the following reused steps;
* Euler: ``delta = float32(sigma_{i+1}) - float32(sigma_i)`` in float32, then
  ``z <- float32(z + delta * v)`` rounded once (nearest, ties to even) from the exact value.

Variants the pages name (readings where they give no formula):

* schedules (mobbang.com / jdon.com list linear spacing, quadratic, cubic and power warps; the
  siami.tw control-table section says the few-step runs settled on a linear base grid with a
  single terminal endpoint): ``power`` is ``(1 - i/S)^p`` (p = 2, 3: quadratic, cubic), and
  ``linear_terminal`` takes the first S points of the linear grid of a longer base count B
  (``1 - i/B``, i < S) and then one terminal step to 0;
* linear velocity extrapolation instead of holding the last fresh velocity (same list): on a
  reused step, with v_a, v_b the last two fresh velocities taken at sigma_a, sigma_b,
  ``v = v_a + w (v_a - v_b)``, ``w = (sigma - sigma_a) / (sigma_a - sigma_b)`` (float32), computed
  as ``fmaf(w, float32(v_a - v_b), v_a)``; w = 0 is the plain hold;
* fixed condition rows (siami.tw, "專業音訊": first/last-frame conditioning with fixed condition
  rows in the DiT): the video rows of the first ``cond_first`` and the last ``cond_last`` latent
  frames are conditioning; the DiT sees them like any other row, the update leaves them as
  they are;
* core reuse (siami.tw control table, ``--core-reuse``, exclusive with whole-velocity reuse):
  every step runs the outer blocks; the core blocks ``core_first..core_last`` run only on steps
  that are fresh for the core period k (the same rule as whole reuse), where the change they
  make to the activations, ``delta = x_after - x_before``, is kept; on the other steps the core
  is replaced by ``x + delta``. Core reuse combines with token reduction (the pages make it
  exclusive only with whole-velocity reuse): the core then lies wholly inside the reduced
  blocks, and its change is kept in the merged geometry, or wholly outside them.
"""
from __future__ import annotations

import numpy as np

from . import dit, tokred
from .geometry import Geometry
from .numeric import f32_round_sum, round_storage, two_sum


def sigma_grid(n_steps: int) -> np.ndarray:
    """float32 [S+1]: sigma_i = 1 - i/S."""
    i = np.arange(n_steps + 1, dtype=np.float64)
    return (1.0 - i / n_steps).astype(np.float32)


def sigma_schedule(kind: str, n_steps: int, param: float = 1.0) -> np.ndarray:
    """float32 [S+1] sigma grids, each value computed in float64 and rounded once.

    'linear': 1 - i/S. 'power': (1 - i/S)^param. 'linear_terminal': 1 - i/param for i < S
    (param = base count B >= S), then 0.
    """
    i = np.arange(n_steps + 1, dtype=np.float64)
    if kind == "linear":
        g = 1.0 - i / n_steps
    elif kind == "power":
        g = (1.0 - i / n_steps) ** np.float64(param)
    elif kind == "linear_terminal":
        if param < n_steps:
            raise ValueError("base count below the step count")
        g = 1.0 - i / np.float64(param)
        g[-1] = 0.0
    else:
        raise ValueError(kind)
    return g.astype(np.float32)


def fma_f32(a, b, c) -> np.ndarray:
    """float32(a * b + c) rounded once from the exact value (a, b, c float32)."""
    p = np.asarray(a, np.float32).astype(np.float64) * np.asarray(b, np.float32).astype(np.float64)
    hi, lo = two_sum(np.asarray(c, np.float32).astype(np.float64), p)
    return f32_round_sum(hi, lo)


def extrapolation_weight(sigma: float, sigma_a: float, sigma_b: float) -> np.float32:
    """w = (sigma - sigma_a) / (sigma_a - sigma_b) from float32 sigmas, rounded once to float32."""
    sa, sb, sg = (np.float64(np.float32(t)) for t in (sigma_a, sigma_b, sigma))
    return np.float32((sg - sa) / (sa - sb))


def extrapolate_velocity(v_a, v_b, w) -> np.ndarray:
    """fmaf(w, float32(v_a - v_b), v_a): the velocity extrapolated linearly in sigma."""
    d = np.asarray(v_a, np.float32) - np.asarray(v_b, np.float32)  # IEEE float32 subtraction
    return fma_f32(np.float32(w), d, v_a)


def cond_rows(geom: Geometry, cond_first: int, cond_last: int) -> np.ndarray:
    """bool [n_video + n_audio]: True for the state rows of the fixed conditioning frames."""
    per_frame = geom.grid_h * geom.grid_w
    t = np.arange(geom.n_video + geom.n_audio) // per_frame
    video = np.arange(geom.n_video + geom.n_audio) < geom.n_video
    return video & ((t < cond_first) | (t >= geom.frames - cond_last))


def is_fresh(step: int, n_steps: int, reuse: int) -> bool:
    if reuse < 1 or not (0 <= step < n_steps):
        raise ValueError("bad step/reuse")
    return step % reuse == 0 or step == n_steps - 1


def sigma_delta(sigma: float, sigma_next: float) -> np.float32:
    return np.float32(np.float32(sigma_next) - np.float32(sigma))


def euler_update(z, delta, v) -> np.ndarray:
    """float32(z + delta * v) rounded once from the exact value.

    z float32, delta float32, v float32 or bfloat16 values: delta*v is exact in float64
    (at most 24 + 24 significand bits), TwoSum recovers the exact sum, and it is rounded once.
    """
    z = np.asarray(z, np.float32).astype(np.float64)
    p = np.float64(np.float32(delta)) * np.asarray(v, np.float32).astype(np.float64)
    hi, lo = two_sum(z, p)
    return f32_round_sum(hi, lo)


def dit_eval(x0, blocks, mods, geom: Geometry, n_heads: int, act: str,
             tr_first: int = -1, tr_last: int = -1, core=None, act_quant=None):
    """Run the block stack on x0 [N, d] with optional token reduction; float64 output [N, d].

    act_quant: passed to every block (the W8A8 activation hook of dit.block_forward).

    core: None, or (first, last, fresh, delta): with fresh the core blocks run and
    ``x_after - x_before`` is returned as the new delta; otherwise they are replaced by
    ``x + delta``. With token reduction the core lies wholly inside the reduced range (its
    delta then has the merged row count) or wholly outside it. Returns x, or (x, delta) when
    core is given.
    """
    x = np.asarray(x0, np.float64)
    g = geom
    n_blocks = len(blocks)
    if core is not None and tr_first >= 0:
        first, last = core[0], core[1]
        inside = tr_first <= first and last <= tr_last
        if not (inside or last < tr_first or first > tr_last):
            raise ValueError("the core blocks straddle a token-reduction boundary")
    delta_out = None
    b = 0
    while b < n_blocks:
        if b == tr_first:
            x = tokred.merge(x, g, act)
            g = g.as_merged()
        if b == tr_last + 1 and g.merged:
            x = tokred.unmerge(x, g.as_unmerged())
            g = g.as_unmerged()
        if core is not None and b == core[0]:
            first, last, fresh, delta = core
            x_in = x
            if fresh:
                for bb in range(first, last + 1):
                    x = dit.block_forward(x, blocks[bb], mods[bb], g, n_heads, act_quant=act_quant)
                delta_out = x - x_in
            else:
                x = x_in + np.asarray(delta, np.float64)
                delta_out = np.asarray(delta, np.float64)
            b = last + 1
            continue
        x = dit.block_forward(x, blocks[b], mods[b], g, n_heads, act_quant=act_quant)
        b += 1
    if g.merged:
        x = tokred.unmerge(x, g.as_unmerged())
    return x if core is None else (x, delta_out)


def denoise_step_full(z, c, v_cache, blocks, mods, geom: Geometry, n_heads: int, act: str,
                      step: int, n_steps: int, reuse: int, sigma: float, sigma_next: float,
                      tr_first: int = -1, tr_last: int = -1, cond_first: int = 0,
                      cond_last: int = 0, v_prev=None, extrap: float = 0.0, core=None,
                      act_quant=None):
    """One sampler step with every variant. Returns (z_next, v_cache, v_prev, core_delta).

    z [Nv+Na, d] float32; c [Nt, d] text rows (values of the act type); v_cache, v_prev: the
    last two fresh velocities (v_prev may be None while extrap is 0); core: None or
    (k, first, last, delta) with delta the kept core change (ignored on core-fresh steps).
    """
    n_state = geom.n_video + geom.n_audio
    core_delta = None
    if is_fresh(step, n_steps, reuse):
        x0 = np.concatenate([round_storage(z, act).astype(np.float64),
                             np.asarray(c, np.float64)], axis=0)
        if core is None:
            out = dit_eval(x0, blocks, mods, geom, n_heads, act, tr_first, tr_last, act_quant=act_quant)
        else:
            k, first, last, delta = core
            out, core_delta = dit_eval(x0, blocks, mods, geom, n_heads, act, tr_first, tr_last,
                                       core=(first, last, is_fresh(step, n_steps, k), delta),
                                       act_quant=act_quant)
        v_prev_next = v_cache
        v = round_storage(out[:n_state], act)
        v_cache_next = v
    else:
        v_cache_next, v_prev_next = v_cache, v_prev
        v = np.asarray(v_cache, np.float32)
        if extrap != 0:
            v = extrapolate_velocity(v_cache, v_prev, extrap)
    z_next = euler_update(z, sigma_delta(sigma, sigma_next), v)
    fixed = cond_rows(geom, cond_first, cond_last)
    z_next[fixed] = np.asarray(z, np.float32)[fixed]
    return z_next, v_cache_next, v_prev_next, core_delta


def denoise_step(z, c, v_cache, blocks, mods, geom: Geometry, n_heads: int, act: str,
                 step: int, n_steps: int, reuse: int, sigma: float, sigma_next: float,
                 tr_first: int = -1, tr_last: int = -1):
    """One sampler step. Returns (z_next float32, v_cache float32 values of the act type).

    z [Nv+Na, d] float32; c [Nt, d] text rows (values of the act type); v_cache as returned by
    the previous step (ignored on fresh steps).
    """
    z_next, v, _, _ = denoise_step_full(z, c, v_cache, blocks, mods, geom, n_heads, act, step,
                                        n_steps, reuse, sigma, sigma_next, tr_first, tr_last)
    return z_next, v
