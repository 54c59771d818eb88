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
