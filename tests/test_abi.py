"""CPU checks of the C ABI: the library loads, exports what the headers declare, and rejects
invalid arguments before touching the GPU."""
import ctypes
import json
import math
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import sampler

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("h3x.h", "h3x_kernels.h")]
FAKE = 0x10000  # an aligned non-NULL address; never dereferenced by a call that fails validation


@pytest.fixture(scope="module")
def B():
    from video_diffusion_transformer_02_amd import binding
    try:
        binding.lib()
    except binding.H3xError as e:
        pytest.fail(str(e))
    return binding


def declared_functions():
    names = set()
    for h in HEADERS:
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names.update(re.findall(r"\b(h3x_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_headers_compile_as_c99():
    for h in HEADERS:
        r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-fsyntax-only", "-x", "c", h],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_library_exports_every_declared_symbol(B):
    names = declared_functions()
    assert len(names) >= 25
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(B.SIGNATURES), set(names) ^ set(B.SIGNATURES)
    assert L.h3x_abi_version() == 4


def test_step_struct_layout_matches_c(B, tmp_path):
    """The ctypes mirror of h3x_step has the C compiler's field offsets and size."""
    fields = [f for f, _ in B.Step._fields_]
    src = tmp_path / "layout.c"
    body = "\n".join(f'  printf("%s %zu\\n", "{f}", offsetof(h3x_step, {f}));' for f in fields)
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "h3x.h"\nint main(void) {\n'
                   + body + '\n  printf("size %zu\\n", sizeof(h3x_step));\n  return 0;\n}\n')
    exe = tmp_path / "layout"
    r = subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True).stdout.splitlines())
    for f in fields:
        assert int(out[f]) == getattr(B.Step, f).offset, f
    assert int(out["size"]) == ctypes.sizeof(B.Step)


def _cfg(B, **kw):
    base = dict(d_model=512, n_heads=4, head_dim=128, ffn_inner=768, act="bf16", weight="bf16")
    base.update(kw)
    return B.BlockCfg.make(**base)


def _geom(B, merged=0, w=12):
    return B.Geom(3, 8, w, 30, 45, merged)


def _last(B):
    return B.lib().h3x_last_error().decode()


def test_cfg_validation(B):
    L = B.lib()
    g = _geom(B)
    bad = [
        (dict(d_model=500), 1), (dict(head_dim=64), 1), (dict(head_dim=64, n_heads=8), 2),
        (dict(ffn_inner=700), 2),
        (dict(act="f32"), 2), (dict(act="f32", weight="f32", head_dim=32, n_heads=16), 2),
        (dict(norm_eps=0.0), 1), (dict(rope_theta=1.0), 1), (dict(weight=7), 1),
        (dict(act="f32", weight="i8a8"), 2),
        (dict(weight="i8a8", d_model=8448, n_heads=66), 2), (dict(weight="i8a8", ffn_inner=32896), 2),
        # Beyond the widths whose operand panels fit 32-bit buffer offsets.
        (dict(d_model=65536 + 256, n_heads=514), 2), (dict(ffn_inner=262144 + 128), 2),
    ]
    for kw, status in bad:
        c = _cfg(B, **kw)
        assert L.h3x_block_workspace_bytes(ctypes.byref(c), ctypes.byref(g)) == 0, kw
        st = L.h3x_norm_mod(ctypes.byref(c), 4, FAKE, FAKE, FAKE, FAKE, None)
        assert st == status, (kw, st, _last(B))
    assert L.h3x_norm_mod(None, 4, FAKE, FAKE, FAKE, FAKE, None) == 1
    c = _cfg(B, act="f32", weight="f32", head_dim=64, n_heads=8)
    assert L.h3x_block_workspace_bytes(ctypes.byref(c), ctypes.byref(g)) > 0


def test_geometry_validation(B):
    L = B.lib()
    assert L.h3x_geom_tokens(ctypes.byref(B.Geom(6, 32, 32, 256, 512, 0))) == 6912
    assert L.h3x_geom_tokens(ctypes.byref(B.Geom(6, 32, 32, 256, 512, 1))) == 3840
    assert L.h3x_geom_tokens(ctypes.byref(B.Geom(6, 30, 54, 256, 512, 0))) == 10488
    assert L.h3x_geom_tokens(ctypes.byref(B.Geom(1, 3, 5, 0, 0, 1))) == -1  # odd width merged
    assert L.h3x_geom_tokens(ctypes.byref(B.Geom(0, 0, 0, 0, 0, 0))) == -1
    assert L.h3x_geom_tokens(ctypes.byref(B.Geom(-1, 2, 2, 0, 0, 0))) == -1
    # Sizes whose product would overflow 64 bits, a grid extent above 2^20 (the RoPE table's
    # int32 indices) or more than 2^26 tokens are refused.
    big = 2 ** 31 - 1
    assert L.h3x_geom_tokens(ctypes.byref(B.Geom(big, big, big, 0, 0, 0))) == -1
    assert L.h3x_geom_tokens(ctypes.byref(B.Geom(1, 1, (1 << 20) + 2, 0, 0, 0))) == -1
    assert L.h3x_geom_tokens(ctypes.byref(B.Geom(1, 1, 1 << 20, 0, 0, 0))) == 1 << 20
    assert L.h3x_geom_tokens(ctypes.byref(B.Geom(1 << 13, 1 << 13, 2, 0, 0, 0))) == -1
    assert L.h3x_geom_tokens(ctypes.byref(B.Geom(1 << 13, 1 << 13, 1, 0, 0, 0))) == 1 << 26
    assert L.h3x_geom_tokens(ctypes.byref(B.Geom(0, 0, 0, big, big, 0))) == -1


def test_block_forward_rejects_before_launch(B):
    L = B.lib()
    c, g = _cfg(B), _geom(B)
    w = B.BlockWeights(FAKE, FAKE, FAKE, FAKE, None, None, None, None)
    need = L.h3x_block_workspace_bytes(ctypes.byref(c), ctypes.byref(g))
    f = L.h3x_dit_block_forward
    assert f(ctypes.byref(c), ctypes.byref(g), ctypes.byref(w), FAKE, FAKE, FAKE, need - 1, None) == 3
    assert "workspace" in _last(B)
    assert f(ctypes.byref(c), ctypes.byref(g), ctypes.byref(w), None, FAKE, FAKE, need, None) == 1
    assert f(ctypes.byref(c), ctypes.byref(g), ctypes.byref(w), FAKE + 8, FAKE, FAKE, need, None) == 1
    wi = B.BlockWeights(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None)
    assert f(ctypes.byref(c), ctypes.byref(g), ctypes.byref(wi), FAKE, FAKE, FAKE, need, None) == 1
    c8 = _cfg(B, weight="i8")
    assert f(ctypes.byref(c8), ctypes.byref(g), ctypes.byref(w), FAKE, FAKE, FAKE, need, None) == 1
    assert "scales" in _last(B)


def test_denoise_step_rejects_before_launch(B):
    L = B.lib()
    c, g = _cfg(B), _geom(B)
    blocks = (B.BlockWeights * 4)(*[B.BlockWeights(FAKE, FAKE, FAKE, FAKE, None, None, None, None)] * 4)
    need = L.h3x_step_workspace_bytes(ctypes.byref(c), ctypes.byref(g))
    assert need > L.h3x_block_workspace_bytes(ctypes.byref(c), ctypes.byref(g))

    def call(step=0, n=4, reuse=1, sigma=1.0, sigma_next=0.75, nb=4, trf=-1, trl=-1, geom=g, ws=need,
             cf=0, cl=0, vp=None, ex=0.0, core=0, c0=0, c1=0, cd=FAKE):
        st = B.Step(step, n, reuse, sigma, sigma_next, nb, blocks, FAKE, trf, trl, cf, cl, vp, ex, core, c0, c1, cd)
        return L.h3x_denoise_step(ctypes.byref(c), ctypes.byref(geom), ctypes.byref(st), FAKE, FAKE, FAKE,
                                  FAKE, ws, None)

    assert call(ws=need - 1) == 3
    assert call(step=4) == 1 and call(step=-1) == 1 and call(reuse=0) == 1
    assert call(sigma=math.nan) == 1 and call(sigma_next=math.inf) == 1
    assert call(nb=0) == 1
    assert call(trf=2, trl=1) == 1 and call(trf=0, trl=4) == 1 and call(trf=-1, trl=2) == 1
    assert call(trf=1, trl=2, geom=_geom(B, w=11)) == 1
    assert "even" in _last(B)
    assert call(geom=_geom(B, merged=1)) == 1
    # Variants: condition frames within the video, extrapolation only with v_prev, core reuse
    # exclusive with whole reuse and token reduction, inside the block range, with a buffer.
    assert call(cf=-1) == 1 and call(cl=2, cf=2) == 1 and call(cf=4) == 1
    assert call(step=1, reuse=2, ex=0.5) == 1 and "v_prev" in _last(B)
    assert call(ex=math.nan) == 1 and call(vp=FAKE + 8) == 1
    assert call(core=2, c0=1, c1=2, reuse=2) == 1 and "exclusive" in _last(B)
    # Core reuse with token reduction: the core wholly inside or wholly outside the reduced
    # blocks passes validation (and fails on the too-small workspace after it); straddling fails.
    for c0, c1, trf, trl, ok in ((1, 2, 1, 2, True), (2, 2, 1, 3, True), (0, 0, 1, 3, True),
                                 (3, 3, 1, 2, True), (0, 1, 1, 2, False), (1, 3, 1, 2, False),
                                 (0, 3, 1, 2, False)):
        st = call(core=2, c0=c0, c1=c1, trf=trf, trl=trl, ws=need - 1)
        assert st == (3 if ok else 1), (c0, c1, trf, trl, _last(B))
        if not ok:
            assert "straddle" in _last(B)
    assert call(core=2, c0=2, c1=1) == 1 and call(core=2, c0=1, c1=4) == 1 and call(core=-1) == 1
    assert call(core=2, c0=1, c1=2, cd=None) == 1 and call(core=2, c0=1, c1=2, cd=FAKE + 4) == 1


def test_sigma_schedules_match_oracle(B):
    for kind, p in (("linear", 1.0), ("power", 2.0), ("power", 3.0), ("power", 0.7), ("linear_terminal", 29.0)):
        for n in (1, 4, 7, 20):
            got = np.array(B.sigma_schedule(kind, n, p), np.float32)
            np.testing.assert_array_equal(got, sampler.sigma_schedule(kind, n, p))
    L = B.lib()
    out = (ctypes.c_float * 9)()
    assert L.h3x_sigma_schedule(2, 8, 4.0, out) == 1 and L.h3x_sigma_schedule(1, 8, 0.0, out) == 1
    assert L.h3x_sigma_schedule(5, 8, 1.0, out) == 1 and L.h3x_sigma_schedule(0, 0, 1.0, out) == 1
    for s_, a, b in ((0.625, 0.75, 1.0), (0.55, 0.6, 0.65), (0.3, 0.45, 0.5)):
        assert np.float32(B.extrapolation_weight(s_, a, b)) == sampler.extrapolation_weight(s_, a, b)
    assert math.isnan(B.extrapolation_weight(0.5, 0.6, 0.6))


def test_fresh_rule_matches_oracle_and_pages(B):
    L = B.lib()
    for n in (1, 2, 4, 7, 20, 50):
        for r in (1, 2, 3, 4, 6):
            for i in range(n):
                assert L.h3x_step_is_fresh(i, n, r) == int(sampler.is_fresh(i, n, r))
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "fresh_counts.json")))
    for r, count in g["fresh_by_reuse"].items():
        assert sum(L.h3x_step_is_fresh(i, g["n_steps"], int(r)) for i in range(g["n_steps"])) == count
    assert L.h3x_step_is_fresh(20, 20, 1) == -1 and L.h3x_step_is_fresh(0, 20, 0) == -1


def test_workspace_and_packing_sizes(B):
    L = B.lib()
    c = _cfg(B, d_model=6144, n_heads=48, ffn_inner=24576)
    g = B.Geom(6, 32, 32, 256, 512, 0)
    ws = L.h3x_block_workspace_bytes(ctypes.byref(c), ctypes.byref(g))
    # R2 [Npad x d] + R1 [Npad x max(4d, F)] bf16 arenas (6912 * 5 * 6144 * 2 bytes) and room
    # for 1024 attention key pieces (O [128 x 128] fp32 + max + sum per piece).
    base = 6912 * 5 * 6144 * 2 + 1024 * (128 * 128 * 4 + 2 * 128 * 4)
    assert base <= ws < base + (1 << 20)
    gm = B.Geom(6, 32, 32, 256, 512, 1)
    assert L.h3x_block_workspace_bytes(ctypes.byref(c), ctypes.byref(gm)) < ws
    assert L.h3x_packed_weight_bytes(ctypes.byref(c), 0, 3 * 6144, 6144) == 3 * 6144 * 6144 * 2
    assert L.h3x_packed_weight_bytes(ctypes.byref(c), 2, 2 * 24576, 6144) == 2 * 24576 * 6144 * 2
    assert L.h3x_packed_weight_bytes(ctypes.byref(c), 2, 24576, 6144) == 0  # not the kind's shape
    assert L.h3x_packed_weight_bytes(ctypes.byref(c), 3, 24576, 6144) == 0  # transposed
    c8 = _cfg(B, d_model=6144, n_heads=48, ffn_inner=24576, weight="i8")
    assert L.h3x_packed_weight_bytes(ctypes.byref(c8), 3, 6144, 24576) == 6144 * 24576
    assert L.h3x_packed_scale_count(ctypes.byref(c8), 2) == 2 * 24576
    assert L.h3x_packed_weight_bytes(ctypes.byref(c8), 9, 6144, 6144) == 0
    # W8A8: the same codes and scales, plus one int8 code per projection-input element and a
    # float32 scale per row ([Npad x max(d, F)] bytes + 4 Npad).
    ca = _cfg(B, d_model=6144, n_heads=48, ffn_inner=24576, weight="i8a8")
    assert L.h3x_packed_weight_bytes(ctypes.byref(ca), 3, 6144, 24576) == 6144 * 24576
    assert L.h3x_packed_scale_count(ctypes.byref(ca), 2) == 2 * 24576
    wa = L.h3x_block_workspace_bytes(ctypes.byref(ca), ctypes.byref(g))
    assert wa - ws == 6912 * 24576 + 6912 * 4
    # int8 weights (W8A16): room to widen the largest matrix (gate/up, 2F x d) to bfloat16.
    w8 = L.h3x_block_workspace_bytes(ctypes.byref(c8), ctypes.byref(g))
    assert w8 - ws == 2 * 24576 * 6144 * 2


def test_pack_calls_reject_before_launch(B):
    """The packing calls check the weight type, the caller's source shape and the pointers."""
    L = B.lib()
    c, cf, c8 = _cfg(B), _cfg(B, act="f32", weight="f32", head_dim=64, n_heads=8), _cfg(B, weight="i8")
    d, f = 512, 768
    ok_shapes = {0: (3 * d, d), 1: (d, d), 2: (2 * f, d), 3: (d, f)}
    for kind, (r, cc) in ok_shapes.items():
        assert L.h3x_packed_weight_bytes(ctypes.byref(c), kind, r, cc) == r * cc * 2
        assert L.h3x_pack_weights_bf16(ctypes.byref(c), kind, FAKE, r + 1, cc, FAKE * 2, None) == 1
        assert "needs" in _last(B)
        if r != cc:  # the transposed shape
            assert L.h3x_pack_weights_bf16(ctypes.byref(c), kind, FAKE, cc, r, FAKE * 2, None) == 1
        assert L.h3x_pack_int8_weights(ctypes.byref(c8), kind, FAKE, r, cc + 64, FAKE * 2, FAKE * 3, None) == 1
    assert L.h3x_pack_weights_bf16(ctypes.byref(cf), 1, FAKE, d, d, FAKE * 2, None) == 1  # F32 cfg
    assert L.h3x_pack_weights_f32(ctypes.byref(c), 1, FAKE, d, d, FAKE * 2, None) == 1    # BF16 cfg
    assert L.h3x_pack_weights_bf16(ctypes.byref(c8), 1, FAKE, d, d, FAKE * 2, None) == 1  # I8 cfg
    assert L.h3x_pack_int8_weights(ctypes.byref(c), 1, FAKE, d, d, FAKE * 2, FAKE * 3, None) == 1
    assert L.h3x_pack_weights_bf16(ctypes.byref(c), 1, FAKE, d, d, FAKE, None) == 1       # in place
    assert L.h3x_pack_weights_bf16(ctypes.byref(c), 1, FAKE + 8, d, d, FAKE * 2, None) == 1
    assert L.h3x_pack_int8_weights(ctypes.byref(c8), 1, FAKE, d, d, FAKE * 2, None, None) == 1
    assert L.h3x_pack_weights_bf16(ctypes.byref(c), 4, FAKE, d, d, FAKE * 2, None) == 1


# The calls the boundary's contract names (a C ABI of plain pointers and sizes), with their
# argument counts: the library must export each of them under that name.
CONTRACT = {
    "h3x_block_workspace_bytes": 2, "h3x_packed_weight_bytes": 4, "h3x_pack_weights_bf16": 7,
    "h3x_pack_int8_weights": 8, "h3x_dit_block_forward": 8, "h3x_step_is_fresh": 3,
    "h3x_step_workspace_bytes": 2, "h3x_denoise_step": 9, "h3x_status_string": 1,
    "h3x_last_error": 0,
}


def test_contract_names_and_arities(B):
    for name, nargs in CONTRACT.items():
        assert name in B.SIGNATURES, name
        assert len(B.SIGNATURES[name][1]) == nargs, name
        assert hasattr(B.lib(), name), name
    # Argument counts as the C header declares them (parsed from the prototype).
    src = re.sub(r"/\*.*?\*/", "", open(HEADERS[0]).read(), flags=re.S)
    for name, nargs in CONTRACT.items():
        m = re.search(r"\b" + name + r"\s*\(([^)]*)\)", src)
        assert m, name
        args = [a for a in m.group(1).split(",") if a.strip() and a.strip() != "void"]
        assert len(args) == nargs, (name, args)


def test_w8a8_kernel_level_contract(B):
    """I8A8 projections take quantised activations: the bfloat16-input entry points refuse."""
    L = B.lib()
    c = _cfg(B, weight="i8a8")
    assert L.h3x_linear_f32out(ctypes.byref(c), 1, 4, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert L.h3x_linear_residual(ctypes.byref(c), 1, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert L.h3x_linear_swiglu(ctypes.byref(c), 4, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert L.h3x_quant_rows(4, 100, FAKE, FAKE, FAKE, None) == 1
    assert L.h3x_quant_rows(4, 32832, FAKE, FAKE, FAKE, None) == 1
    assert L.h3x_norm_mod_quant(ctypes.byref(_cfg(B, weight="i8")), 4, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert L.h3x_linear_a8_f32out(ctypes.byref(_cfg(B)), 1, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert L.h3x_linear_a8_f32out(ctypes.byref(c), 5, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert L.h3x_linear_a8_f32out(ctypes.byref(c), 1, 4, FAKE, None, FAKE, FAKE, FAKE, None) == 1


def test_mfma_probe_rejects_before_launch(B):
    L = B.lib()
    ops = ctypes.c_double(-1.0)
    assert L.h3x_mfma_probe(0, 10, FAKE, ctypes.byref(ops), None) == 1  # float32: no such probe
    assert L.h3x_mfma_probe(3, 10, FAKE, ctypes.byref(ops), None) == 1
    assert L.h3x_mfma_probe(1, 0, FAKE, ctypes.byref(ops), None) == 1
    assert L.h3x_mfma_probe(1, 10, None, ctypes.byref(ops), None) == 1
    assert L.h3x_mfma_probe(2, 10, FAKE, None, None) == 1
    assert ops.value == -1.0


def test_status_strings(B):
    L = B.lib()
    assert L.h3x_status_string(0) == b"ok"
    assert L.h3x_status_string(3) == b"workspace too small"
    assert L.h3x_copy(FAKE, FAKE, 17, None) == 1


def test_zero_row_calls_enqueue_nothing(B):
    """Zero rows: valid, nothing enqueued, pointers not looked at (no device needed)."""
    L = B.lib()
    c = _cfg(B)
    ca = _cfg(B, weight="i8a8")
    assert L.h3x_norm_mod(ctypes.byref(c), 0, None, None, None, None, None) == 0
    assert L.h3x_linear_f32out(ctypes.byref(c), 1, 0, None, None, None, None, None) == 0
    assert L.h3x_linear_residual(ctypes.byref(c), 3, 0, None, None, None, None, None, None) == 0
    assert L.h3x_linear_swiglu(ctypes.byref(c), 0, None, None, None, None, None) == 0
    assert L.h3x_euler(ctypes.byref(c), 0, None, None, 1.0, 0.5, None, None) == 0
    assert L.h3x_quant_rows(0, 64, None, None, None, None) == 0
    assert L.h3x_norm_mod_quant(ctypes.byref(ca), 0, None, None, None, None, None, None) == 0
    assert L.h3x_linear_a8_f32out(ctypes.byref(ca), 1, 0, None, None, None, None, None, None) == 0
    # The row count is still range-checked, and the other arguments still validated.
    assert L.h3x_norm_mod(ctypes.byref(c), -1, None, None, None, None, None) == 1
    assert L.h3x_norm_mod(ctypes.byref(c), (1 << 26) + 1, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert L.h3x_euler(ctypes.byref(c), 1 << 40, FAKE, FAKE, 1.0, 0.5, None, None) == 1
    assert L.h3x_quant_rows(0, 100, None, None, None, None) == 1
    assert L.h3x_linear_f32out(ctypes.byref(c), 7, 0, None, None, None, None, None) == 1


def test_sequence_length_limit(B):
    """bf16 K and V^T matrices are addressed with 32-bit buffer offsets: Npad * d * 2 < 2^31."""
    L = B.lib()
    c = _cfg(B, d_model=6144, n_heads=48, ffn_inner=24576)
    g = B.Geom(1, 400, 500, 0, 0, 0)  # 200000 tokens
    st = L.h3x_dit_block_forward(ctypes.byref(c), ctypes.byref(g), None, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == 2, _last(B)
    assert L.h3x_attention(ctypes.byref(c), 200000, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 1 << 40, None) == 2
    # The largest sequence that fits still passes this check (and fails later for other reasons).
    n_ok = (2 ** 31 - 1) // (6144 * 2) // 256 * 256
    assert L.h3x_attention(ctypes.byref(c), n_ok, None, FAKE, FAKE, FAKE, 0, FAKE, 1 << 40, None) == 1


def test_binding_fails_loudly_without_the_library(tmp_path):
    """With libh3x.so absent, every entry of the binding raises: there is no other path."""
    code = f"""
import sys
sys.path.insert(0, {ROOT!r})
from video_diffusion_transformer_02_amd import binding as B
B.LIB_PATH = {str(tmp_path / 'libh3x.so')!r}
cfg = B.BlockCfg.make(256, 2, 128, 1024)
g = B.Geom(1, 8, 8, 16, 32, 0)
for call in (B.lib, lambda: B.block_workspace_bytes(cfg, g), lambda: B.step_is_fresh(0, 20, 2)):
    try:
        call()
    except B.H3xError as e:
        assert "missing" in str(e), e
    else:
        raise SystemExit("no error")
print("raised")
"""
    r = subprocess.run([os.environ.get("PYTHON", "python3"), "-c", code], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("raised"), r.stdout + r.stderr
