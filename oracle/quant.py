"""Per-output-channel symmetric int8 weights with bfloat16 scales (test infrastructure only).

Pages: 21cto.com, "M5 Max 生产环境实测数据", item 4 (int8 for MLP + QKV + attention output),
siami.tw, "2. 數據會說話" (int8 default, + QKV, + attention-output projection). The pages give
no formula; reading taken, per output row r of a bfloat16 weight W [R, C]:

* ``a = max_c |W[r, c]|``; a row with a == 0 gets scale 0 and all-zero codes;
* ``s = bf16(a / 127)`` with an IEEE float32 division rounded to nearest even, then rounded
  to bfloat16 (nearest even); if that underflows to 0 the codes are 0;
* ``q[r, c] = clamp(rint(W[r, c] / s), -127, 127)``: float32 division by the *stored* scale,
  then round half to even. -128 is never produced.

The dequantised weight is ``s * q`` (exact in float32: an 8-bit by 7-bit significand product).

W8A8 (the pages' experimental per-row int8 FC2 path, jdon.com "选配还是选速", taken further to
every projection as the ranked next step): each projection's input activation, as stored
(bfloat16), is quantised per row with a float32 scale; reading taken, per row r of X [R, C]:

* ``a = max_c |X[r, c]|``; ``inv = float32(127 / a)``, ``s = float32(a / 127)`` (IEEE float32
  divisions); a row with a == 0, or whose inv overflows, gets s = 0 and all-zero codes;
* ``q[r, c] = clamp(rint(float32(X[r, c] * inv)), -127, 127)``.

The projection is then ``out[r, c] = s_a[r] * s_w[c] * sum_k q_a[r, k] q_w[c, k]`` with an exact
integer sum.
"""
from __future__ import annotations

import numpy as np

from .numeric import bf16_rne


def pack_int8(w_bf16) -> tuple[np.ndarray, np.ndarray]:
    """(q int8 [R, C], s float32 [R] holding bfloat16 values) in the source row order."""
    w = np.asarray(w_bf16, dtype=np.float32)
    a = np.max(np.abs(w), axis=1)
    s = bf16_rne(a / np.float32(127.0))
    s = np.where(a == 0, np.float32(0.0), s).astype(np.float32)
    safe = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    quot = (w / safe[:, None]).astype(np.float32)  # float32 / float32: IEEE division
    q = np.clip(np.rint(quot), -127, 127)
    q = np.where((s == 0)[:, None], 0, q).astype(np.int8)
    return q, s


def dequant(q, s) -> np.ndarray:
    """float64 weight s[r] * q[r, c]."""
    return np.asarray(s, np.float64)[:, None] * np.asarray(q, np.float64)


def quant_act_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """(q int8 [R, C], s float32 [R]): per-row activation quantisation of float32 values."""
    x = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(x), axis=1).astype(np.float32)
    with np.errstate(divide="ignore", over="ignore"):
        inv = (np.float32(127.0) / a).astype(np.float32)
    s = (a / np.float32(127.0)).astype(np.float32)
    dead = (a == 0) | ~np.isfinite(inv)
    inv = np.where(dead, np.float32(0.0), inv).astype(np.float32)
    s = np.where(dead, np.float32(0.0), s).astype(np.float32)
    prod = (x * inv[:, None]).astype(np.float32)  # float32 product, rounded once
    q = np.clip(np.rint(prod), -127, 127).astype(np.int8)
    return q, s


def int8_matmul(qa, sa, qw, sw) -> np.ndarray:
    """float64 s_a[r] * s_w[c] * sum_k qa[r, k] qw[c, k], the integer sum exact (int64)."""
    acc = np.asarray(qa, np.int64) @ np.asarray(qw, np.int64).T
    return np.asarray(sa, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :] * acc.astype(np.float64)


def w8a8_act(act: str = "bf16"):
    """The activation hook of the W8A8 block: round to the storage type, quantise per row,
    dequantise (float64)."""
    from .numeric import round_storage

    def f(a):
        q, s = quant_act_rows(round_storage(a, act))
        return dequant(q, s)
    return f
