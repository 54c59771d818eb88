"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark.

This module holds shapes, seeds and random draws only: none of the method's arithmetic.
Every tensor comes from its own NumPy PCG64 stream, seeded as ``base * 1000003 + id``, so
any single tensor can be regenerated on its own:

* block ``b`` weights: ids ``5b + 0..4`` for W_qkv, W_o, W_gate, W_up, W_down;
* modulation for (step ``s``, block ``b``) of an ``L``-block stack: id ``10**6 + s*L + b``;
* initial latent state z0: id ``2*10**6``; text conditioning rows: id ``2*10**6 + 1``.

Draws are float32 ``N(mean, std**2)``. Configurations that store bfloat16 round the draws to
bfloat16 (round to nearest even) with torch's own conversion; the rounded values are what both
the GPU path and the oracle receive.

The workloads take their geometry from the pages' 512x512, 22-frame renders (jdon.com,
section "330亿参数是什么概念"; siami.tw, "速度與品質的可調旋鈕" control table) at synthetic
model widths; the pages publish no model dimensions.
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

SEED_STRIDE = 1000003
MOD_ID = 10**6
STATE_ID = 2 * 10**6


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes and schedule of one synthetic workload (all token counts unmerged)."""

    name: str
    d_model: int
    n_heads: int
    head_dim: int
    ffn_inner: int
    frames: int
    grid_h: int
    grid_w: int
    n_audio: int
    n_text: int
    n_blocks: int
    act: str  # "f32" or "bf16": storage type of activations (and of master weights)
    weight: str  # "f32", "bf16", "i8" (int8 weights) or "i8a8" (int8 weights and activations)
    n_steps: int = 1
    reuse: int = 1
    tr_first: int = -1
    tr_last: int = -1
    w_std: float = 0.02
    qkv_std: float = 0.02
    seed_base: int = 0

    @property
    def n_video(self) -> int:
        return self.frames * self.grid_h * self.grid_w

    @property
    def n_state(self) -> int:
        """Rows the sampler updates: video then audio."""
        return self.n_video + self.n_audio

    @property
    def n_tokens(self) -> int:
        return self.n_video + self.n_audio + self.n_text

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Tiny two-block fp32 stack: one 8x8 latent frame, 16 audio and 32 text tokens.
TINY = Workload("tiny_f32_2blk", 256, 4, 64, 1024, 1, 8, 8, 16, 32, 2, "f32", "f32",
                n_steps=20, reuse=1, seed_base=0)
# Same, with larger Q/K weights so that attention is far from uniform.
TINY_SHARP = TINY.replace(name="tiny_f32_sharp", qkv_std=0.2)
# One bf16 block at the 512x512x22-frame class latent grid (6 x 32 x 32) + 256 audio + 512 text.
BLOCK = Workload("block_bf16_6912tok", 6144, 48, 128, 24576, 6, 32, 32, 256, 512, 1, "bf16",
                 "bf16", seed_base=1)
# 45 active blocks, 20 linear-sigma Euler steps, whole-velocity reuse 2.
DENOISE45 = BLOCK.replace(name="denoise_45blk_20step_reuse2", n_blocks=45, n_steps=20, reuse=2,
                          seed_base=2)
# As above with horizontal token-pair reduction in blocks 10..34 (0-based, inclusive).
DENOISE45_TR = DENOISE45.replace(name="denoise_45blk_20step_reuse2_tr10_34", tr_first=10,
                                 tr_last=34)
# 50 blocks, int8 per-output-channel weights, 480x864-class grid 6 x 30 x 54, 4 steps.
INT8_50 = BLOCK.replace(name="int8w_50blk_4step_6x30x54", grid_h=30, grid_w=54, n_blocks=50,
                        weight="i8", n_steps=4, reuse=1, seed_base=4)

# The 45-block, 20-step, reuse-2 schedule with token reduction over blocks 10..34 at a width
# the oracle runs end to end in seconds: d 256 (2 heads x 128), F 1024, bf16, 6 x 8 x 8 video +
# 16 audio + 32 text tokens (432; 240 when merged).
TINY_LONG = BLOCK.replace(name="tiny_long_bf16_45blk_20step_reuse2_tr10_34", d_model=256, n_heads=2,
                          ffn_inner=1024, frames=6, grid_h=8, grid_w=8, n_audio=16, n_text=32,
                          n_blocks=45, n_steps=20, reuse=2, tr_first=10, tr_last=34, seed_base=31)

WORKLOADS = {w.name: w for w in (TINY, TINY_SHARP, BLOCK, DENOISE45, DENOISE45_TR, INT8_50, TINY_LONG)}


def stream(base: int, ident: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(base * SEED_STRIDE + ident))


def normal(base: int, ident: int, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """float32 draws from N(mean, std**2) on stream (base, ident)."""
    a = stream(base, ident).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return a


def to_storage(a: np.ndarray, dtype: str):
    """Return a CPU torch tensor in the storage type ('f32' or 'bf16'); bf16 rounds to nearest even."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype in ("f32", "i8"):
        return t
    raise ValueError(dtype)


def storage_values(a: np.ndarray, dtype: str) -> np.ndarray:
    """float32 array holding exactly the values of ``to_storage(a, dtype)``."""
    return to_storage(a, dtype).float().numpy()


def block_weights(w: Workload, b: int) -> dict:
    """Unpacked master weights of block b as float32 arrays (rows = output features).

    qkv [3d, d] (rows: Q | K | V, head-major), out [d, d], gate [F, d], up [F, d], down [d, F].
    """
    d, f, base = w.d_model, w.ffn_inner, w.seed_base
    return {
        "qkv": normal(base, 5 * b + 0, (3 * d, d), w.qkv_std),
        "out": normal(base, 5 * b + 1, (d, d), w.w_std),
        "gate": normal(base, 5 * b + 2, (f, d), w.w_std),
        "up": normal(base, 5 * b + 3, (f, d), w.w_std),
        "down": normal(base, 5 * b + 4, (d, f), w.w_std),
    }


def modulation(w: Workload, step: int, b: int) -> np.ndarray:
    """[6, d] float32: shift1, scale1, gate1, shift2, scale2, gate2 of block b at step ``step``.

    Shifts and scales ~ N(0, 0.1**2); gates ~ N(1, 0.1**2), so no branch is switched off.
    """
    m = normal(w.seed_base, MOD_ID + step * w.n_blocks + b, (6, w.d_model), 0.1)
    m[2] += np.float32(1.0)
    m[5] += np.float32(1.0)
    return m


def initial_state(w: Workload) -> np.ndarray:
    """z0: [n_video + n_audio, d] float32 ~ N(0, 1)."""
    return normal(w.seed_base, STATE_ID, (w.n_state, w.d_model))


def text_rows(w: Workload) -> np.ndarray:
    """Text conditioning rows c: [n_text, d] float32 ~ N(0, 1) (round to storage before use)."""
    return normal(w.seed_base, STATE_ID + 1, (w.n_text, w.d_model))


def block_input(w: Workload) -> np.ndarray:
    """A single block's input x: [n_tokens, d] float32 ~ N(0, 1) (stream of z0 then c)."""
    return np.concatenate([initial_state(w), text_rows(w)], axis=0)


def sample_rows(w: Workload, n_video: int = 40, n_audio: int = 12, n_text: int = 12,
                seed: int = 12345, merged: bool = False) -> np.ndarray:
    """Seed-fixed sorted row indices to check on large workloads.

    Always includes the first and last row of each modality and, for video, four whole
    horizontal pairs (2p, 2p+1).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    nv = w.n_video // 2 if merged else w.n_video
    na, nt = w.n_audio, w.n_text
    vid = {0, nv - 1}
    if not merged:
        for p in rng.choice(nv // 2, size=4, replace=False):
            vid.update((2 * int(p), 2 * int(p) + 1))
    while len(vid) < min(n_video, nv):
        vid.add(int(rng.integers(0, nv)))
    aud = {nv, nv + na - 1} if na else set()
    while na and len(aud) < min(n_audio, na):
        aud.add(nv + int(rng.integers(0, na)))
    txt = {nv + na, nv + na + nt - 1} if nt else set()
    while nt and len(txt) < min(n_text, nt):
        txt.add(nv + na + int(rng.integers(0, nt)))
    return np.array(sorted(vid | aud | txt), dtype=np.int64)


def sha256_prefix(t, nbytes: int = 16 << 20) -> str:
    """SHA-256 of the first ``nbytes`` of a CPU tensor or array (input provenance log)."""
    import torch

    if isinstance(t, torch.Tensor):
        raw = t.contiguous().view(torch.uint8).numpy()
    else:
        raw = np.ascontiguousarray(t).view(np.uint8)
    return hashlib.sha256(raw.reshape(-1)[:nbytes].tobytes()).hexdigest()[:16]
