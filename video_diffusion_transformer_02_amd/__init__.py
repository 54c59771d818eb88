"""h3x: the DiT denoiser hot path (modulated RMSNorm, QKV + 3D RoPE, joint attention, gated
out-projection, SwiGLU MLP, token-pair reduction, flow-matching Euler with velocity reuse) as
hand-written HIP kernels for MI355X (gfx950) behind the C ABI in include/h3x.h.

``binding`` marshals torch tensors into that ABI; ``build`` compiles libh3x.so in-tree.
"""
from . import binding  # noqa: F401
