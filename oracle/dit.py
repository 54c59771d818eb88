"""One DiT block of the dense single-stream transformer, in float64 (test infrastructure only).

The pages describe the block only in passing: a transformer forward pass (siami.tw,
"技術亮點 › 1. 完整的 Metal 原生堆疊", h3_dit.c), QKV and attention-output projections
(jdon.com, "选配还是选速"), attention heads and a normalised MLP input (siami.tw,
"3. 記憶體策略是 Apple Silicon 的殺手鐧"), an FC2 layer (jdon.com, "选配还是选速"), one
joint token stream (mobbang.com, "MiniMax H3：视频与音轨一起生成的开源模型"). The readings
taken for what they leave open:

* normalisation: RMSNorm without a learned gain, eps = 1e-6, modulated as
  ``y = x / sqrt(mean(x^2) + eps) * (1 + scale) + shift``;
* projections: ``out = in @ W.T`` with W stored [out_features, in_features]; no bias;
  QKV rows are Q | K | V and each is head-major (head h owns columns h*Dh .. h*Dh+Dh-1);
* 3D RoPE on the Q and K of video rows only; each head splits into contiguous (t | y | x)
  chunks of Dh/4, 3Dh/8, 3Dh/8 dims; within a chunk of size D, pair k = (2k, 2k+1) turns by
  ``pos * theta**(-2k/D)``, theta = 10000;
* attention: softmax(q k^T / sqrt(Dh)) v over all tokens, no mask;
* residuals: ``x1 = x + gate1 * attn_out``, ``x2 = x1 + gate2 * mlp_out``;
* MLP: SwiGLU, ``h = silu(y2 @ W_gate.T) * (y2 @ W_up.T)``, ``mlp_out = h @ W_down.T``.
"""
from __future__ import annotations

import math

import numpy as np

from .geometry import Geometry

NORM_EPS = 1e-6
ROPE_THETA = 10000.0


def rms_norm_mod(x, shift, scale, eps: float = NORM_EPS) -> np.ndarray:
    """Modulated RMSNorm over the last axis, float64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * (1.0 + np.asarray(scale, np.float64)) + np.asarray(shift, np.float64)


def rope_chunks(head_dim: int):
    """[(axis, offset, size)] of the (t, y, x) chunks of one head."""
    if head_dim % 8:
        raise ValueError("head_dim must be a multiple of 8")
    st, sy = head_dim // 4, 3 * head_dim // 8
    sx = head_dim - st - sy
    return [(0, 0, st), (1, st, sy), (2, st + sy, sx)]


def rope(z, pos, rotated, n_heads: int, theta: float = ROPE_THETA) -> np.ndarray:
    """Rotate the interleaved pairs of every head of z [n, n_heads*Dh] by 3D positions.

    pos [n, 3] holds (t, y, x); rows with rotated == False are returned unchanged.
    """
    z = np.array(z, dtype=np.float64, copy=True)
    n, d = z.shape
    dh = d // n_heads
    out = z.copy()
    for axis, off, size in rope_chunks(dh):
        for k in range(size // 2):
            omega = theta ** (-2.0 * k / size)
            phi = pos[:, axis] * omega
            c, s = np.cos(phi)[:, None], np.sin(phi)[:, None]
            for h in range(n_heads):
                i0 = h * dh + off + 2 * k
                a, b = z[:, i0:i0 + 1], z[:, i0 + 1:i0 + 2]
                out[:, i0:i0 + 1] = a * c - b * s
                out[:, i0 + 1:i0 + 2] = a * s + b * c
    return np.where(np.asarray(rotated)[:, None], out, z)


def attention(q, k, v, n_heads: int) -> np.ndarray:
    """Per-head softmax(q k^T / sqrt(Dh)) v; q [m, d], k and v [n, d] -> [m, d]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    m, d = q.shape
    dh = d // n_heads
    out = np.empty((m, d), dtype=np.float64)
    for h in range(n_heads):
        sl = slice(h * dh, (h + 1) * dh)
        s = (q[:, sl] @ k[:, sl].T) / math.sqrt(dh)
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, sl] = p @ v[:, sl]
    return out


def silu(z) -> np.ndarray:
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


def _w(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def block_forward(x, w: dict, mod, geom: Geometry, n_heads: int, rows=None, act_quant=None) -> np.ndarray:
    """Block output x2 for the rows ``rows`` (all rows if None).

    x [N, d] is the block input (all N rows are needed: every query attends to every key).
    w holds unpacked weights: qkv [3d, d], out [d, d], gate [F, d], up [F, d], down [d, F].
    mod [6, d] holds shift1, scale1, gate1, shift2, scale2, gate2.
    act_quant: None, or a function applied to each projection's input activation (the W8A8
    path passes the per-row int8 quantise-dequantise of the stored value).
    """
    aq = (lambda a: a) if act_quant is None else act_quant
    x = np.asarray(x, np.float64)
    n, d = x.shape
    if n != geom.n_tokens:
        raise ValueError(f"x has {n} rows, geometry has {geom.n_tokens}")
    rows = np.arange(n) if rows is None else np.asarray(rows)
    mod = np.asarray(mod, np.float64)
    shift1, scale1, gate1, shift2, scale2, gate2 = mod
    wqkv = _w(w["qkv"])
    wq, wk, wv = wqkv[0:d], wqkv[d:2 * d], wqkv[2 * d:3 * d]

    y = aq(rms_norm_mod(x, shift1, scale1))
    pos, rot = geom.positions()
    q = rope(y[rows] @ wq.T, pos[rows], rot[rows], n_heads)
    k = rope(y @ wk.T, pos, rot, n_heads)
    v = y @ wv.T
    o = aq(attention(q, k, v, n_heads))
    x1 = x[rows] + gate1 * (o @ _w(w["out"]).T)

    y2 = aq(rms_norm_mod(x1, shift2, scale2))
    h = aq(silu(y2 @ _w(w["gate"]).T) * (y2 @ _w(w["up"]).T))
    return x1 + gate2 * (h @ _w(w["down"]).T)


def block_flops(n_tokens: int, d: int, ffn: int) -> float:
    """Algorithmic FLOPs of one block: the four projections plus q k^T and p v."""
    proj = 2.0 * n_tokens * d * (3 * d + d + 2 * ffn + ffn)
    attn = 4.0 * n_tokens * n_tokens * d
    return proj + attn
