"""ctypes binding of libh3x (argument marshalling only).

Every function here converts torch tensors to device pointers, passes the current HIP stream
and checks the returned status; all arithmetic runs in the library's HIP kernels. Output
buffers are allocated with torch (device memory is the only thing torch provides here). If the
library is not built, ``lib()`` raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libh3x.so")
_LIB = None

F32, BF16, I8, I8A8 = 0, 1, 2, 3
W_QKV, W_OUT, W_GATE_UP, W_DOWN = 0, 1, 2, 3
DTYPES = {"f32": F32, "bf16": BF16, "i8": I8, "i8a8": I8A8}
TORCH_ACT = {F32: torch.float32, BF16: torch.bfloat16}


class H3xError(RuntimeError):
    pass


class BlockCfg(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn_inner", ctypes.c_int32),
                ("act", ctypes.c_int32), ("weight", ctypes.c_int32),
                ("norm_eps", ctypes.c_float), ("rope_theta", ctypes.c_float)]

    @classmethod
    def make(cls, d_model, n_heads, head_dim, ffn_inner, act="bf16", weight="bf16",
             norm_eps=1e-6, rope_theta=10000.0):
        return cls(d_model, n_heads, head_dim, ffn_inner, DTYPES.get(act, act), DTYPES.get(weight, weight),
                   norm_eps, rope_theta)

    @property
    def act_dtype(self) -> torch.dtype:
        return TORCH_ACT[self.act]


class Geom(ctypes.Structure):
    _fields_ = [("frames", ctypes.c_int32), ("grid_h", ctypes.c_int32),
                ("grid_w", ctypes.c_int32), ("n_audio", ctypes.c_int32),
                ("n_text", ctypes.c_int32), ("merged", ctypes.c_int32)]

    @property
    def n_video(self) -> int:
        n = self.frames * self.grid_h * self.grid_w
        return n // 2 if self.merged else n

    @property
    def n_tokens(self) -> int:
        return self.n_video + self.n_audio + self.n_text

    def as_merged(self) -> "Geom":
        return Geom(self.frames, self.grid_h, self.grid_w, self.n_audio, self.n_text, 1)


class BlockWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("qkv", "out", "gate_up", "down", "s_qkv", "s_out", "s_gate_up", "s_down")]


class Step(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int32), ("n_steps", ctypes.c_int32), ("reuse", ctypes.c_int32),
                ("sigma", ctypes.c_float), ("sigma_next", ctypes.c_float),
                ("n_blocks", ctypes.c_int32), ("blocks", ctypes.POINTER(BlockWeights)),
                ("mod", ctypes.c_void_p), ("tr_first", ctypes.c_int32),
                ("tr_last", ctypes.c_int32),
                ("cond_first", ctypes.c_int32), ("cond_last", ctypes.c_int32),
                ("v_prev", ctypes.c_void_p), ("extrap", ctypes.c_float),
                ("core_reuse", ctypes.c_int32), ("core_first", ctypes.c_int32),
                ("core_last", ctypes.c_int32), ("core_delta", ctypes.c_void_p)]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int32),
                ("total_ms", ctypes.c_double)]


_P = ctypes.c_void_p
_I32, _I64, _SZ, _F = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
_CFG, _GEOM = ctypes.POINTER(BlockCfg), ctypes.POINTER(Geom)

SIGNATURES = {
    "h3x_abi_version": (_I32, []),
    "h3x_status_string": (ctypes.c_char_p, [_I32]),
    "h3x_last_error": (ctypes.c_char_p, []),
    "h3x_geom_tokens": (_I64, [_GEOM]),
    "h3x_packed_weight_bytes": (_SZ, [_CFG, _I32, _I64, _I64]),
    "h3x_packed_rows": (_I64, [_CFG, _I32]),
    "h3x_packed_scale_count": (_I64, [_CFG, _I32]),
    "h3x_pack_weights_bf16": (_I32, [_CFG, _I32, _P, _I64, _I64, _P, _P]),
    "h3x_pack_weights_f32": (_I32, [_CFG, _I32, _P, _I64, _I64, _P, _P]),
    "h3x_pack_int8_weights": (_I32, [_CFG, _I32, _P, _I64, _I64, _P, _P, _P]),
    "h3x_block_workspace_bytes": (_SZ, [_CFG, _GEOM]),
    "h3x_dit_block_forward": (_I32, [_CFG, _GEOM, ctypes.POINTER(BlockWeights), _P, _P, _P, _SZ, _P]),
    "h3x_dit_block_forward_noalloc": (_I32, [_CFG, _GEOM, ctypes.POINTER(BlockWeights), _P, _P, _P]),
    "h3x_step_is_fresh": (_I32, [_I32, _I32, _I32]),
    "h3x_sigma_schedule": (_I32, [_I32, _I32, ctypes.c_double, ctypes.POINTER(ctypes.c_float)]),
    "h3x_extrapolation_weight": (_F, [_F, _F, _F]),
    "h3x_step_workspace_bytes": (_SZ, [_CFG, _GEOM]),
    "h3x_denoise_step": (_I32, [_CFG, _GEOM, ctypes.POINTER(Step), _P, _P, _P, _P, _SZ, _P]),
    "h3x_norm_mod": (_I32, [_CFG, _I64, _P, _P, _P, _P, _P]),
    "h3x_rope_table_bytes": (_SZ, [_CFG, _GEOM]),
    "h3x_rope_table": (_I32, [_CFG, _GEOM, _P, _P]),
    "h3x_qkv_project": (_I32, [_CFG, _GEOM, _P, _P, _P, _P, _P, _P, _P, _P]),
    "h3x_attention_workspace_bytes": (_SZ, [_CFG, _I64, _I32]),
    "h3x_attention": (_I32, [_CFG, _I64, _P, _P, _P, _P, _I32, _P, _SZ, _P]),
    "h3x_linear_residual": (_I32, [_CFG, _I32, _I64, _P, _P, _P, _P, _P, _P]),
    "h3x_linear_swiglu": (_I32, [_CFG, _I64, _P, _P, _P, _P, _P]),
    "h3x_linear_f32out": (_I32, [_CFG, _I32, _I64, _P, _P, _P, _P, _P]),
    "h3x_quant_rows": (_I32, [_I64, _I64, _P, _P, _P, _P]),
    "h3x_norm_mod_quant": (_I32, [_CFG, _I64, _P, _P, _P, _P, _P, _P]),
    "h3x_linear_a8_f32out": (_I32, [_CFG, _I32, _I64, _P, _P, _P, _P, _P, _P]),
    "h3x_token_merge": (_I32, [_CFG, _GEOM, _P, _P, _P]),
    "h3x_token_unmerge": (_I32, [_CFG, _GEOM, _P, _P, _P]),
    "h3x_euler": (_I32, [_CFG, _I64, _P, _P, _F, _F, _P, _P]),
    "h3x_copy": (_I32, [_P, _P, _SZ, _P]),
    "h3x_mfma_probe": (_I32, [_I32, _I64, _P, ctypes.POINTER(ctypes.c_double), _P]),
    "h3x_profile_begin": (_I32, []),
    "h3x_profile_end": (_I32, [ctypes.POINTER(KernelTime), _I32]),
}


def lib():
    """The loaded libh3x (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise H3xError(f"{LIB_PATH} is missing: build it with "
                           "`python -m video_diffusion_transformer_02_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def _check(status: int, what: str):
    if status != 0:
        L = lib()
        raise H3xError(f"{what}: {L.h3x_status_string(status).decode()}: "
                       f"{L.h3x_last_error().decode()}")


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise H3xError("expected a device tensor")
    if not t.is_contiguous():
        raise H3xError("expected a contiguous tensor")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def status_of(name: str, *args) -> int:
    """Raw status of an entry point (for tests of the error paths)."""
    return getattr(lib(), name)(*args)


# ------------------------------------------------------------------ weights
@dataclasses.dataclass
class PackedBlock:
    """Packed device weights of one block (kept alive with the struct that points at them)."""

    qkv: torch.Tensor
    out: torch.Tensor
    gate_up: torch.Tensor
    down: torch.Tensor
    s_qkv: torch.Tensor | None = None
    s_out: torch.Tensor | None = None
    s_gate_up: torch.Tensor | None = None
    s_down: torch.Tensor | None = None

    def struct(self) -> BlockWeights:
        return BlockWeights(*(_p(getattr(self, n)) for n in
                              ("qkv", "out", "gate_up", "down", "s_qkv", "s_out", "s_gate_up", "s_down")))


def packed_rows(cfg: BlockCfg, kind: int) -> int:
    return lib().h3x_packed_rows(ctypes.byref(cfg), kind)


def _shape2(w: torch.Tensor):
    if w.dim() != 2:
        raise H3xError("expected a 2-D master weight")
    return w.shape[0], w.shape[1]


def packed_weight_bytes(cfg: BlockCfg, kind: int, rows: int, cols: int) -> int:
    return lib().h3x_packed_weight_bytes(ctypes.byref(cfg), kind, rows, cols)


def pack_weights(cfg: BlockCfg, kind: int, w: torch.Tensor) -> torch.Tensor:
    """bfloat16 (h3x_pack_weights_bf16) or float32 (h3x_pack_weights_f32) packing by cfg.weight."""
    rows, cols = _shape2(w)
    nbytes = packed_weight_bytes(cfg, kind, rows, cols)
    packed = torch.empty(max(nbytes // w.element_size(), 1), dtype=w.dtype, device=w.device)
    fn = lib().h3x_pack_weights_bf16 if cfg.weight == BF16 else lib().h3x_pack_weights_f32
    _check(fn(ctypes.byref(cfg), kind, _p(w), rows, cols, _p(packed), _stream()), "pack_weights")
    return packed.view(packed_rows(cfg, kind), -1)


def pack_int8_weights(cfg: BlockCfg, kind: int, w_bf16: torch.Tensor):
    rows, cols = _shape2(w_bf16)
    prow = packed_rows(cfg, kind)
    q = torch.empty(max(packed_weight_bytes(cfg, kind, rows, cols), 1), dtype=torch.int8, device=w_bf16.device)
    s = torch.empty(max(prow, 1), dtype=torch.bfloat16, device=w_bf16.device)
    _check(lib().h3x_pack_int8_weights(ctypes.byref(cfg), kind, _p(w_bf16), rows, cols, _p(q), _p(s), _stream()),
           "pack_int8_weights")
    return q.view(prow, -1), s


def pack_block(cfg: BlockCfg, w: dict) -> PackedBlock:
    """Pack a block's master weights (device tensors qkv, out, gate, up, down)."""
    gu = torch.cat([w["gate"], w["up"]], dim=0)
    srcs = {"qkv": (W_QKV, w["qkv"]), "out": (W_OUT, w["out"]), "gate_up": (W_GATE_UP, gu),
            "down": (W_DOWN, w["down"])}
    if cfg.weight in (I8, I8A8):
        fields = {}
        for name, (kind, t) in srcs.items():
            q, s = pack_int8_weights(cfg, kind, t.contiguous())
            fields[name], fields["s_" + name] = q, s
        return PackedBlock(**fields)
    return PackedBlock(**{name: pack_weights(cfg, kind, t.contiguous()) for name, (kind, t) in srcs.items()})


# ------------------------------------------------------------------ block and step
def block_workspace_bytes(cfg: BlockCfg, geom: Geom) -> int:
    return lib().h3x_block_workspace_bytes(ctypes.byref(cfg), ctypes.byref(geom))


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def dit_block_forward(cfg: BlockCfg, geom: Geom, blk: PackedBlock, mod: torch.Tensor,
                      x: torch.Tensor, ws: torch.Tensor):
    ws_struct = blk.struct()
    _check(lib().h3x_dit_block_forward(ctypes.byref(cfg), ctypes.byref(geom), ctypes.byref(ws_struct),
                                       _p(mod), _p(x), _p(ws), ws.numel(), _stream()),
           "dit_block_forward")


NOALLOC_SCRATCH_BYTES = 64 << 20  # H3X_NOALLOC_SCRATCH_BYTES


def dit_block_forward_noalloc(cfg: BlockCfg, geom: Geom, blk: PackedBlock, mod: torch.Tensor, x: torch.Tensor):
    """The block forward on the library's own device scratch (no workspace argument)."""
    w = blk.struct()
    _check(lib().h3x_dit_block_forward_noalloc(ctypes.byref(cfg), ctypes.byref(geom), ctypes.byref(w), _p(mod),
                                               _p(x), _stream()), "dit_block_forward_noalloc")


def step_is_fresh(step: int, n_steps: int, reuse: int) -> int:
    return lib().h3x_step_is_fresh(step, n_steps, reuse)


def step_workspace_bytes(cfg: BlockCfg, geom: Geom) -> int:
    return lib().h3x_step_workspace_bytes(ctypes.byref(cfg), ctypes.byref(geom))


def denoise_step(cfg: BlockCfg, geom: Geom, step: int, n_steps: int, reuse: int, sigma: float,
                 sigma_next: float, blocks, mod: torch.Tensor | None, z: torch.Tensor,
                 text: torch.Tensor, v_cache: torch.Tensor, ws: torch.Tensor,
                 tr_first: int = -1, tr_last: int = -1, cond_first: int = 0, cond_last: int = 0,
                 v_prev: torch.Tensor | None = None, extrap: float = 0.0, core_reuse: int = 0,
                 core_first: int = 0, core_last: int = 0, core_delta: torch.Tensor | None = None):
    """blocks: a ctypes array of BlockWeights (see block_array) or None on reused steps."""
    n_blocks = len(blocks) if blocks is not None else 0
    st = Step(step, n_steps, reuse, sigma, sigma_next, n_blocks,
              ctypes.cast(blocks, ctypes.POINTER(BlockWeights)) if blocks is not None else None,
              _p(mod), tr_first, tr_last, cond_first, cond_last, _p(v_prev), extrap, core_reuse,
              core_first, core_last, _p(core_delta))
    _check(lib().h3x_denoise_step(ctypes.byref(cfg), ctypes.byref(geom), ctypes.byref(st), _p(z),
                                  _p(text), _p(v_cache), _p(ws), ws.numel(), _stream()),
           "denoise_step")


SCHEDULES = {"linear": 0, "power": 1, "linear_terminal": 2}


def sigma_schedule(kind: str, n_steps: int, param: float = 1.0) -> list:
    out = (ctypes.c_float * (n_steps + 1))()
    _check(lib().h3x_sigma_schedule(SCHEDULES[kind], n_steps, float(param), out), "sigma_schedule")
    return list(out)


def extrapolation_weight(sigma: float, sigma_a: float, sigma_b: float) -> float:
    return lib().h3x_extrapolation_weight(sigma, sigma_a, sigma_b)


def block_array(packed_blocks) -> ctypes.Array:
    arr = (BlockWeights * len(packed_blocks))()
    for i, b in enumerate(packed_blocks):
        arr[i] = b.struct()
    return arr


# ------------------------------------------------------------------ kernel-level entry points
def pad_rows(n: int) -> int:
    return (n + 255) // 256 * 256


def norm_mod(cfg, x, shift, scale, y=None):
    y = torch.empty_like(x) if y is None else y
    _check(lib().h3x_norm_mod(ctypes.byref(cfg), x.shape[0], _p(x), _p(shift), _p(scale), _p(y), _stream()),
           "norm_mod")
    return y


def rope_table(cfg, geom):
    t = alloc_workspace(lib().h3x_rope_table_bytes(ctypes.byref(cfg), ctypes.byref(geom)))
    _check(lib().h3x_rope_table(ctypes.byref(cfg), ctypes.byref(geom), _p(t), _stream()), "rope_table")
    return t


def qkv_project(cfg, geom, y, w_qkv, s_qkv=None, table=None):
    n, d = geom.n_tokens, cfg.d_model
    npad = pad_rows(n)
    table = rope_table(cfg, geom) if table is None else table
    q = torch.empty(npad, d, dtype=cfg.act_dtype, device=y.device)
    k = torch.empty_like(q)
    vt = torch.empty(d, npad, dtype=cfg.act_dtype, device=y.device)
    _check(lib().h3x_qkv_project(ctypes.byref(cfg), ctypes.byref(geom), _p(y), _p(w_qkv), _p(s_qkv),
                                 _p(table), _p(q), _p(k), _p(vt), _stream()), "qkv_project")
    return q, k, vt


def attention(cfg, n_tokens, q, k, vt, o=None, slots=0):
    """slots: concurrently resident workgroups the work is planned for (0 = the device's)."""
    o = torch.empty(n_tokens, cfg.d_model, dtype=cfg.act_dtype, device=q.device) if o is None else o
    nbytes = lib().h3x_attention_workspace_bytes(ctypes.byref(cfg), n_tokens, slots)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib().h3x_attention(ctypes.byref(cfg), n_tokens, _p(q), _p(k), _p(vt), _p(o), slots, _p(ws), nbytes,
                               _stream()), "attention")
    return o


def linear_residual(cfg, kind, a, w, s, gate, x):
    _check(lib().h3x_linear_residual(ctypes.byref(cfg), kind, a.shape[0], _p(a), _p(w), _p(s), _p(gate),
                                     _p(x), _stream()), "linear_residual")
    return x


def linear_swiglu(cfg, y2, w, s=None, h=None):
    h = torch.empty(y2.shape[0], cfg.ffn_inner, dtype=cfg.act_dtype, device=y2.device) if h is None else h
    _check(lib().h3x_linear_swiglu(ctypes.byref(cfg), y2.shape[0], _p(y2), _p(w), _p(s), _p(h), _stream()),
           "linear_swiglu")
    return h


def linear_f32out(cfg, kind, a, w, s=None):
    out = torch.empty(a.shape[0], packed_rows(cfg, kind), dtype=torch.float32, device=a.device)
    _check(lib().h3x_linear_f32out(ctypes.byref(cfg), kind, a.shape[0], _p(a), _p(w), _p(s), _p(out), _stream()),
           "linear_f32out")
    return out


def token_merge(cfg, geom, x):
    xm = torch.empty(geom.as_merged().n_tokens, cfg.d_model, dtype=x.dtype, device=x.device)
    _check(lib().h3x_token_merge(ctypes.byref(cfg), ctypes.byref(geom), _p(x), _p(xm), _stream()), "token_merge")
    return xm


def token_unmerge(cfg, geom, xm):
    x = torch.empty(geom.n_tokens, cfg.d_model, dtype=xm.dtype, device=xm.device)
    _check(lib().h3x_token_unmerge(ctypes.byref(cfg), ctypes.byref(geom), _p(xm), _p(x), _stream()),
           "token_unmerge")
    return x


def euler(cfg, z, v, sigma, sigma_next, v_copy=None):
    _check(lib().h3x_euler(ctypes.byref(cfg), z.shape[0], _p(z), _p(v), sigma, sigma_next, _p(v_copy),
                           _stream()), "euler")
    return z


def copy(src, dst):
    _check(lib().h3x_copy(_p(src), _p(dst), src.numel() * src.element_size(), _stream()), "copy")


def mfma_probe(dtype, iters, out):
    """Launch the matrix-core throughput probe (dtype BF16 or I8); returns its operation count."""
    ops = ctypes.c_double(0.0)
    _check(lib().h3x_mfma_probe(dtype, iters, _p(out), ctypes.byref(ops), _stream()), "mfma_probe")
    return ops.value


def profile_begin():
    _check(lib().h3x_profile_begin(), "profile_begin")


def profile_end(max_entries: int = 64) -> dict:
    arr = (KernelTime * max_entries)()
    n = lib().h3x_profile_end(arr, max_entries)
    if n < 0:
        raise H3xError(lib().h3x_last_error().decode())
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n)}


def quant_rows(a, q=None, s=None):
    """Per-row int8 codes (slabs of 256 rows x 64 codes, flat int8 tensor of pad_rows(m) * cols
    bytes) and float32 scales [pad_rows(m)] of a bfloat16 [m x cols] tensor."""
    m, cols = a.shape
    q = torch.zeros(pad_rows(m) * cols, dtype=torch.int8, device=a.device) if q is None else q
    s = torch.zeros(pad_rows(m), dtype=torch.float32, device=a.device) if s is None else s
    _check(lib().h3x_quant_rows(m, cols, _p(a), _p(q), _p(s), _stream()), "quant_rows")
    return q, s


def norm_mod_quant(cfg, x, shift, scale, q=None, s=None):
    m, d = x.shape
    q = torch.zeros(pad_rows(m) * d, dtype=torch.int8, device=x.device) if q is None else q
    s = torch.zeros(pad_rows(m), dtype=torch.float32, device=x.device) if s is None else s
    _check(lib().h3x_norm_mod_quant(ctypes.byref(cfg), m, _p(x), _p(shift), _p(scale), _p(q), _p(s), _stream()),
           "norm_mod_quant")
    return q, s


def linear_a8_f32out(cfg, kind, m, qa, sa, w, sw):
    out = torch.empty(m, packed_rows(cfg, kind), dtype=torch.float32, device=qa.device)
    _check(lib().h3x_linear_a8_f32out(ctypes.byref(cfg), kind, m, _p(qa), _p(sa), _p(w), _p(sw), _p(out),
                                      _stream()), "linear_a8_f32out")
    return out
