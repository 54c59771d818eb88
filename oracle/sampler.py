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
             tr_first: int = -1, tr_last: int = -1) -> np.ndarray:
    """Run the block stack on x0 [N, d] with optional token reduction; float64 output [N, d]."""
    x = np.asarray(x0, np.float64)
    g = geom
    n_blocks = len(blocks)
    for b in range(n_blocks):
        if b == tr_first:
            x = tokred.merge(x, g, act)
            g = g.as_merged()
        if b == tr_last + 1 and g.merged:
            x = tokred.unmerge(x, g.as_unmerged())
            g = g.as_unmerged()
        x = dit.block_forward(x, blocks[b], mods[b], g, n_heads)
    if g.merged:
        x = tokred.unmerge(x, g.as_unmerged())
    return x


def denoise_step(z, c, v_cache, blocks, mods, geom: Geometry, n_heads: int, act: str,
                 step: int, n_steps: int, reuse: int, sigma: float, sigma_next: float,
                 tr_first: int = -1, tr_last: int = -1):
    """One sampler step. Returns (z_next float32, v_cache float32 values of the act type).

    z [Nv+Na, d] float32; c [Nt, d] text rows (values of the act type); v_cache as returned by
    the previous step (ignored on fresh steps).
    """
    n_state = geom.n_video + geom.n_audio
    if is_fresh(step, n_steps, reuse):
        x0 = np.concatenate([round_storage(z, act).astype(np.float64),
                             np.asarray(c, np.float64)], axis=0)
        out = dit_eval(x0, blocks, mods, geom, n_heads, act, tr_first, tr_last)
        v = round_storage(out[:n_state], act)
    else:
        v = np.asarray(v_cache, np.float32)
    return euler_update(z, sigma_delta(sigma, sigma_next), v), v
