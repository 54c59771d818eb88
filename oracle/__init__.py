"""Plain, slow CPU oracle of the DiT denoiser hot path (float64 NumPy).

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import or run anything in this package; the GPU product path never does, and this
package imports nothing from it. The two share only the seeded input generators in
``synth``.

What is computed, and where the pages fix it (the pages are five news write-ups of the h3.c
engine for MiniMax H3; none prints a formula, so every formula below is a stated reading):

* ``dit.block_forward`` -- one transformer block of the dense single-stream omni model
  (mobbang.com, "MiniMax H3：视频与音轨一起生成的开源模型"): modulated RMSNorm, QKV projection,
  3D RoPE on video rows, full bidirectional attention over the joint video+audio+text
  sequence (mobbang.com, "效能：M5 Max 上512×512 约3.5 秒": all frames are denoised together
  and kept coherent through attention), gated out-projection residual, modulated RMSNorm
  (the "normalised MLP input" of siami.tw, "3. 記憶體策略…"), SwiGLU MLP, gated residual.
* ``tokred.merge`` / ``tokred.unmerge`` -- token reduction: horizontally adjacent video tokens
  are paired in the middle blocks (jdon.com, "330亿参数是什么概念"; siami.tw control table,
  row "Token 縮減").
* ``sampler`` -- the linear sigma grid, the whole-velocity reuse rule (siami.tw control table,
  row "整體 denoiser 復用": 20 / 11 / 8 fresh evaluations at 20 steps) and the flow-matching
  Euler update.
* ``quant.pack_int8`` -- per-output-channel symmetric int8 weights with bfloat16 scales
  (21cto.com, "M5 Max 生产环境实测数据", item 4; siami.tw, "2. 數據會說話").

Exact definitions (Euler rounding, token merge rounding, int8 packing) are computed exactly
and are compared bit for bit; everything else is float64 and compared within tolerance.
"""
from . import numeric, dit, tokred, sampler, quant  # noqa: F401
from .geometry import Geometry  # noqa: F401
