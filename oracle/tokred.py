"""Token reduction: horizontal pair merge and unmerge (test infrastructure only).

Pages: jdon.com, "330亿参数是什么概念" (adjacent video tokens are paired to cut the work;
16.69 s -> 12.60 s) and siami.tw, "速度與品質的可調旋鈕" control table, row "Token 縮減"
(horizontal video tokens of the middle blocks are merged). Reading taken: a pair is merged
by its mean, rounded once to the activation storage type, and unmerged by writing the merged
row back to both members; audio and text rows pass through unchanged.
"""
from __future__ import annotations

import numpy as np

from .geometry import Geometry
from .numeric import bf16_from_f64


def _store(x64: np.ndarray, act: str) -> np.ndarray:
    if act == "bf16":
        return bf16_from_f64(x64).astype(np.float64)
    if act == "f32":
        return x64.astype(np.float32).astype(np.float64)
    raise ValueError(act)


def merge(x: np.ndarray, geom: Geometry, act: str) -> np.ndarray:
    """[N, d] unmerged rows -> [N', d] with video pairs (2p, 2p+1) -> row p (their mean)."""
    if geom.merged:
        raise ValueError("already merged")
    x = np.asarray(x, dtype=np.float64)
    nv = geom.n_video
    if nv % 2 or geom.grid_w % 2:
        raise ValueError("token pairing needs an even latent width")
    pair_sum = x[0:nv:2] + x[1:nv:2]  # two storage-type values: the float64 sum is exact
    merged_video = _store(pair_sum / 2.0, act)
    return np.concatenate([merged_video, x[nv:]], axis=0)


def unmerge(xm: np.ndarray, geom: Geometry) -> np.ndarray:
    """[N', d] merged rows (geom unmerged) -> [N, d]: row p is written to rows 2p and 2p+1."""
    xm = np.asarray(xm, dtype=np.float64)
    nvm = geom.n_video // 2
    video = np.repeat(xm[:nvm], 2, axis=0)
    return np.concatenate([video, xm[nvm:]], axis=0)
