"""Per-kernel parity of the HIP path against the oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import synth
from oracle import dit, quant, sampler, tokred
from oracle.numeric import bf16_rne
from _util import (bf16_bits_to_f32, binding_cfg, binding_geom, host, oracle_geom, rel_l2, to_dev,
                   unslab)

pytestmark = pytest.mark.gpu

# bf16 shapes that span several 256-row, 256-column and 64-key tiles with ragged tails.
SMALL = synth.BLOCK.replace(name="small_bf16", d_model=512, n_heads=4, ffn_inner=768, frames=3,
                            grid_h=8, grid_w=12, n_audio=30, n_text=45, seed_base=11)
SMALL_F32 = SMALL.replace(name="small_f32", act="f32", weight="f32", seed_base=12)
SMALL_I8 = SMALL.replace(name="small_i8", weight="i8", seed_base=13)


@pytest.fixture(scope="module")
def B():
    from video_diffusion_transformer_02_amd import binding
    binding.lib()
    return binding


def _w(wl, name):
    return synth.block_weights(wl, 0)[name]


# ---------------------------------------------------------------- weight packing
def test_pack_int8_bit_exact(B):
    wl = SMALL_I8
    cfg = binding_cfg(wl)
    rng = np.random.default_rng(5)
    for kind, rows, cols in ((B.W_QKV, 3 * wl.d_model, wl.d_model), (B.W_GATE_UP, 2 * wl.ffn_inner, wl.d_model),
                             (B.W_DOWN, wl.d_model, wl.ffn_inner)):
        w = rng.standard_normal((rows, cols)).astype(np.float32) * np.float32(0.02)
        w[0] = 0.0                      # zero row
        w[1] = 1e-40                    # scale underflows to zero
        w[2] = 1e-36                    # subnormal scale
        w[3, 5] = -7.0                  # one dominant negative
        w[4] = np.linspace(-1, 1, cols)  # exact halves after division
        wb = bf16_rne(w)
        q, s = B.pack_int8_weights(cfg, kind, to_dev(wb, "bf16"))
        torch.cuda.synchronize()
        qr, sr = quant.pack_int8(wb)
        perm = np.array([_src(kind, p, rows) for p in range(rows)])
        np.testing.assert_array_equal(unslab(q, rows, cols, 1), qr[perm])
        np.testing.assert_array_equal(s.float().cpu().numpy(), sr[perm])


def _src(kind, p, rows):
    """Source row of packed row p, as stated in include/h3x.h."""
    if kind != 2:
        return p
    f = rows // 2
    j, i = divmod(p, 64)
    return 32 * j + i if i < 32 else f + 32 * j + (i - 32)


@pytest.mark.parametrize("wl", [SMALL, SMALL_F32], ids=lambda w: w.name)
def test_pack_layout_bit_exact(B, wl):
    cfg = binding_cfg(wl)
    gu = np.concatenate([_w(wl, "gate"), _w(wl, "up")], axis=0)
    src = synth.storage_values(gu, wl.act)
    packed = B.pack_weights(cfg, B.W_GATE_UP, to_dev(gu, wl.act))
    torch.cuda.synchronize()
    rows, cols = gu.shape
    perm = np.array([_src(2, p, rows) for p in range(rows)])
    if wl.act == "bf16":
        got = bf16_bits_to_f32(unslab(packed, rows, cols, 2))
    else:
        got = packed.cpu().numpy()
    np.testing.assert_array_equal(got, src[perm])


# ---------------------------------------------------------------- modulated RMSNorm
@pytest.mark.parametrize("wl,tol", [(SMALL, 5e-3), (SMALL_F32, 1e-6)], ids=["bf16", "f32"])
def test_norm_mod(B, wl, tol):
    cfg = binding_cfg(wl)
    x = synth.storage_values(synth.block_input(wl) * 3.0, wl.act)
    m = synth.modulation(wl, 0, 0)
    y = B.norm_mod(cfg, to_dev(x, wl.act), torch.from_numpy(m[0]).cuda(), torch.from_numpy(m[1]).cuda())
    ref = dit.rms_norm_mod(x, m[0], m[1])
    assert rel_l2(host(y), ref) < tol


@pytest.mark.parametrize("act,d", [("bf16", 256), ("bf16", 2304), ("bf16", 4096), ("bf16", 8192),
                                   ("bf16", 10240), ("f32", 256), ("f32", 1536), ("f32", 4096)])
def test_norm_mod_every_width(B, act, d):
    """Every register-resident width of the four-row kernel (one to four 16-byte chunks per
    thread and row) and the one-row kernel beyond it, with 13 rows (the last workgroup of four
    rows ragged): every row within the bar of the oracle's."""
    wl = SMALL.replace(d_model=d, n_heads=d // 128, act=act, weight=act)
    cfg = binding_cfg(wl)
    rng = np.random.default_rng(d)
    x = synth.storage_values(rng.standard_normal((13, d)).astype(np.float32) * 2.0, act)
    x[5] = 0.0
    m = (rng.standard_normal((2, d)) * 0.3).astype(np.float32)
    y = host(B.norm_mod(cfg, to_dev(x, act), torch.from_numpy(m[0]).cuda(), torch.from_numpy(m[1]).cuda()))
    ref = dit.rms_norm_mod(x, m[0], m[1])
    rows = np.linalg.norm(y - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert rows.max() < (5e-3 if act == "bf16" else 1e-6), (int(rows.argmax()), rows.max())


# ---------------------------------------------------------------- contraction alone
@pytest.mark.parametrize("wl", [SMALL, SMALL_I8, SMALL_F32], ids=lambda w: w.name)
@pytest.mark.parametrize("m", [1, 255, 363, 700])
def test_linear_f32out(B, wl, m):
    cfg = binding_cfg(wl)
    act = "f32" if wl.act == "f32" else "bf16"
    rng = np.random.default_rng(m)
    a = synth.storage_values(rng.standard_normal((m, wl.ffn_inner)).astype(np.float32), act)
    wd = synth.storage_values(_w(wl, "down"), act)
    if wl.weight == "i8":
        q, s = B.pack_int8_weights(cfg, B.W_DOWN, to_dev(wd, "bf16"))
        qr, sr = quant.pack_int8(wd)
        wref = quant.dequant(qr, sr)
    else:
        q, s = B.pack_weights(cfg, B.W_DOWN, to_dev(wd, act)), None
        wref = wd.astype(np.float64)
    out = B.linear_f32out(cfg, B.W_DOWN, to_dev(a, act), q, s)
    ref = a.astype(np.float64) @ wref.T
    assert rel_l2(host(out), ref) < 2e-6


# A gate/up projection with more tiles than the chip runs at once (3 x 192 = 576 tiles of
# 256 x 256 for 700 rows and 2 x 24576 columns, a ragged last row of tiles): the XCD-ordered tile
# walk over several rounds, against the plain product.
WIDE = SMALL.replace(name="wide_bf16", ffn_inner=24576, seed_base=19)


@pytest.mark.parametrize("weight", ["bf16", "i8"])
def test_linear_many_tile_rounds(B, weight):
    wl = WIDE.replace(weight=weight)
    cfg = binding_cfg(wl)
    m, d, f = 700, wl.d_model, wl.ffn_inner
    rng = np.random.default_rng(23)
    a = synth.storage_values(rng.standard_normal((m, d)).astype(np.float32), "bf16")
    gu = synth.storage_values(rng.standard_normal((2 * f, d)).astype(np.float32) * np.float32(0.02), "bf16")
    if weight == "i8":
        w, s = B.pack_int8_weights(cfg, B.W_GATE_UP, to_dev(gu, "bf16"))
        gu_r = quant.dequant(*quant.pack_int8(gu))
    else:
        w, s = B.pack_weights(cfg, B.W_GATE_UP, to_dev(gu, "bf16")), None
        gu_r = gu.astype(np.float64)
    ad = to_dev(a, "bf16")
    out = host(B.linear_f32out(cfg, B.W_GATE_UP, ad, w, s))
    perm = np.array([_src(B.W_GATE_UP, p, 2 * f) for p in range(2 * f)])
    ref = a.astype(np.float64) @ gu_r[perm].T
    assert rel_l2(out, ref) < 2e-6
    h = host(B.linear_swiglu(cfg, ad, w, s))
    a64 = a.astype(np.float64)
    href = dit.silu(a64 @ gu_r[:f].T) * (a64 @ gu_r[f:].T)
    assert rel_l2(h, href) < 5e-3
    # Every row on its own, the ragged last tile row (rows 512..699) included.
    den = np.linalg.norm(href, axis=1)
    assert (np.linalg.norm(h - href, axis=1) / den).max() < 1e-2


# ---------------------------------------------------------------- QKV + RoPE
@pytest.mark.parametrize("wl,tol", [(SMALL, 5e-3), (SMALL_F32, 1e-5), (SMALL_I8, 5e-3)],
                         ids=["bf16", "f32", "i8"])
@pytest.mark.parametrize("merged", [False, True])
def test_qkv_rope(B, wl, tol, merged):
    cfg, g = binding_cfg(wl), binding_geom(wl, merged)
    og = oracle_geom(wl, merged)
    act = wl.act
    n, d = og.n_tokens, wl.d_model
    rng = np.random.default_rng(3)
    y = synth.storage_values(rng.standard_normal((n, d)).astype(np.float32), act)
    wq = synth.storage_values(_w(wl, "qkv"), "f32" if act == "f32" else "bf16")
    if wl.weight == "i8":
        qw, sw = B.pack_int8_weights(cfg, B.W_QKV, to_dev(wq, "bf16"))
        wref = quant.dequant(*quant.pack_int8(wq))
    else:
        qw, sw = B.pack_weights(cfg, B.W_QKV, to_dev(wq, act)), None
        wref = wq.astype(np.float64)
    q, k, vt = B.qkv_project(cfg, g, to_dev(y, act), qw, sw)
    torch.cuda.synchronize()
    pos, rot = og.positions()
    y64 = y.astype(np.float64)
    qr = dit.rope(y64 @ wref[:d].T, pos, rot, wl.n_heads)
    kr = dit.rope(y64 @ wref[d:2 * d].T, pos, rot, wl.n_heads)
    vr = y64 @ wref[2 * d:].T
    qh, kh, vth = host(q), host(k), host(vt)
    assert rel_l2(qh[:n], qr) < tol
    assert rel_l2(kh[:n], kr) < tol
    assert rel_l2(vth[:, :n].T, vr) < tol
    # Pad rows are zero.
    assert not qh[n:].any() and not kh[n:].any() and not vth[:, n:].any()


# ---------------------------------------------------------------- attention
@pytest.mark.parametrize("wl,tol", [(SMALL, 5e-3), (SMALL_F32, 1e-5)], ids=["bf16", "f32"])
@pytest.mark.parametrize("n,sharp", [(363, 1.0), (363, 6.0), (64, 1.0), (1, 1.0), (1000, 3.0)])
def test_attention(B, wl, tol, n, sharp):
    cfg = binding_cfg(wl)
    d, npad = wl.d_model, B.pad_rows(n)
    rng = np.random.default_rng(n)
    qv = synth.storage_values(rng.standard_normal((n, d)).astype(np.float32) * np.float32(sharp), wl.act)
    kv = synth.storage_values(rng.standard_normal((n, d)).astype(np.float32), wl.act)
    vv = synth.storage_values(rng.standard_normal((n, d)).astype(np.float32), wl.act)
    qp, kp = np.zeros((npad, d), np.float32), np.zeros((npad, d), np.float32)
    vtp = np.zeros((d, npad), np.float32)
    qp[:n], kp[:n], vtp[:, :n] = qv, kv, vv.T
    kp[n:] = np.nan  # keys past the end are masked, whatever they hold
    o = B.attention(cfg, n, to_dev(qp, wl.act), to_dev(kp, wl.act), to_dev(vtp, wl.act))
    ref = dit.attention(qv, kv, vv, wl.n_heads)
    assert rel_l2(host(o), ref) < tol


def test_attention_longest_sequence(B, record):
    """The longest sequence whose bfloat16 K and V^T the attention kernel can address with 32-bit
    buffer offsets at d = 6144 (48 heads x 128): N = 174592 tokens, N * d * 2 bytes just under
    2^31. Checked on sampled query rows (the first and the last 32, and 64 drawn at random)
    against the oracle over all N keys; inputs drawn on the GPU from a seeded generator."""
    d, heads = 6144, 48
    n = (2 ** 31 - 1) // (d * 2) // 256 * 256
    assert n == 174592 and n * d * 2 < 2 ** 31
    cfg = B.BlockCfg.make(d, heads, 128, 4 * d, "bf16", "bf16")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(174592)
    draw = lambda scale: (torch.randn((n, d), generator=gen, device="cuda") * scale).to(torch.bfloat16)
    q, k, v = draw(2.0), draw(1.0), draw(1.0)
    vt = v.t().contiguous()
    print(f"[longest] attention over {n} tokens", flush=True)
    o = B.attention(cfg, n, q, k, vt)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(32), np.arange(n - 32, n), rng.integers(32, n - 32, 64)]))
    ridx = torch.from_numpy(rows).cuda()
    got = host(o.index_select(0, ridx))
    qs = q.index_select(0, ridx).float().cpu().numpy()
    del o, vt, q
    kh = k.float().cpu().numpy()
    del k
    vh = v.float().cpu().numpy()
    del v
    torch.cuda.empty_cache()
    ref = dit.attention(qs, kh, vh, heads)
    e = rel_l2(got, ref)
    worst = max(rel_l2(got[i], ref[i]) for i in range(len(rows)))
    record("attention_longest_sequence", e, 5e-3)
    record("attention_longest_sequence worst row", worst, 1e-2)
    print(f"[longest] rel-L2 {e:.2e}, worst row {worst:.2e}", flush=True)
    assert e < 5e-3 and worst < 1e-2


@pytest.mark.parametrize("slots", [0, 1])
def test_attention_needles_in_every_key_tile(B, record, slots):
    """Each query's own key dominates its softmax (q_i = 3 k_j(i), logits of about 34 against a
    spread of about 3): the keys j(i) run over every 64-key tile, the first and the last key of
    each and both ends of the ragged last tile (363 = 5 x 64 + 43 keys), so a skipped, masked or
    misplaced tile, or a wrong key order inside a tile, moves whole rows; every row is checked
    on its own. slots 0: the device's plan (key pieces); 1: every item whole."""
    wl = SMALL
    cfg = binding_cfg(wl)
    n, d = 363, wl.d_model
    npad = B.pad_rows(n)
    rng = np.random.default_rng(12)
    kv = synth.storage_values(rng.standard_normal((n, d)).astype(np.float32), "bf16")
    vv = synth.storage_values(rng.standard_normal((n, d)).astype(np.float32), "bf16")
    needles = sorted({j for t in range(0, n, 64) for j in (t, t + 1, min(t + 63, n - 1))} | {n - 43, n - 2, n - 1})
    j_of = np.array([needles[i % len(needles)] if i % 3 else (i * 7) % n for i in range(n)])
    qv = synth.storage_values(3.0 * kv[j_of], "bf16")
    qp, kp = np.zeros((npad, d), np.float32), np.zeros((npad, d), np.float32)
    vtp = np.zeros((d, npad), np.float32)
    qp[:n], kp[:n], vtp[:, :n] = qv, kv, vv.T
    o = host(B.attention(cfg, n, to_dev(qp, "bf16"), to_dev(kp, "bf16"), to_dev(vtp, "bf16"), slots=slots))
    ref = dit.attention(qv, kv, vv, wl.n_heads)
    # The references are dominated by the needles' values (the pin that the test is sharp).
    assert rel_l2(ref, vv[j_of]) < 0.3
    rows = np.linalg.norm(o - ref, axis=1) / np.linalg.norm(ref, axis=1)
    record(f"attention_needles[slots={slots}] worst row", rows.max(), 1e-2)
    assert rows.max() < 1e-2, int(rows.argmax())


@pytest.mark.parametrize("slots", [16, 12, 5, 100, 0])
def test_attention_work_split(B, record, slots):
    """The work plan for `slots` resident workgroups, for 1000 tokens and 4 heads (16 items of
    256 queries, 16 key tiles): 16 runs every item whole; 12 and 5 leave a last round of 4 and
    1 items cut into 3 and 4 key pieces; 100 and the device's default cut every item (6 pieces,
    or one tile each). Every plan agrees with the oracle, and with the plan for one slot (never
    split) up to the merge's rounding."""
    wl = SMALL
    cfg = binding_cfg(wl)
    n, d = 1000, wl.d_model
    npad = B.pad_rows(n)
    rng = np.random.default_rng(7)
    qv = synth.storage_values(rng.standard_normal((n, d)).astype(np.float32) * np.float32(4.0), "bf16")
    kv = synth.storage_values(rng.standard_normal((n, d)).astype(np.float32), "bf16")
    vv = synth.storage_values(rng.standard_normal((n, d)).astype(np.float32), "bf16")
    qp, kp = np.zeros((npad, d), np.float32), np.zeros((npad, d), np.float32)
    vtp = np.zeros((d, npad), np.float32)
    qp[:n], kp[:n], vtp[:, :n] = qv, kv, vv.T
    args = (to_dev(qp, "bf16"), to_dev(kp, "bf16"), to_dev(vtp, "bf16"))
    o = host(B.attention(cfg, n, *args, slots=slots))
    whole = host(B.attention(cfg, n, *args, slots=1))
    ref = dit.attention(qv, kv, vv, wl.n_heads)
    err = rel_l2(o, ref)
    record(f"attention_work_split[slots={slots}]", err, 5e-3)
    assert err < 5e-3
    np.testing.assert_allclose(o, whole, rtol=2e-2, atol=2e-2)


def test_attention_invariants(B):
    """V == 1 gives O == 1 exactly up to rounding; identical keys give the mean of V."""
    wl = SMALL
    cfg = binding_cfg(wl)
    n, d = 300, wl.d_model
    npad = B.pad_rows(n)
    rng = np.random.default_rng(1)
    q = np.zeros((npad, d), np.float32)
    q[:n] = rng.standard_normal((n, d)) * 4
    k = np.zeros((npad, d), np.float32)
    k[:n] = rng.standard_normal((n, d))
    vt = np.zeros((d, npad), np.float32)
    vt[:, :n] = 1.0
    o = host(B.attention(cfg, n, to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(vt, "bf16")))
    np.testing.assert_allclose(o, 1.0, rtol=4e-3)
    k[:n] = k[0]
    vt[:, :n] = synth.storage_values(rng.standard_normal((d, n)).astype(np.float32), "bf16")
    o = host(B.attention(cfg, n, to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(vt, "bf16")))
    np.testing.assert_allclose(o, np.tile(vt[:, :n].mean(axis=1), (n, 1)), atol=2e-2, rtol=1e-2)


# ---------------------------------------------------------------- gated residual and SwiGLU
@pytest.mark.parametrize("wl,tol", [(SMALL, 5e-3), (SMALL_F32, 1e-6), (SMALL_I8, 5e-3)],
                         ids=["bf16", "f32", "i8"])
def test_linear_residual_and_swiglu(B, wl, tol):
    cfg = binding_cfg(wl)
    act = wl.act
    master = "f32" if act == "f32" else "bf16"
    n, d, f = 363, wl.d_model, wl.ffn_inner
    rng = np.random.default_rng(8)
    x = synth.storage_values(rng.standard_normal((n, d)).astype(np.float32), act)
    o = synth.storage_values(rng.standard_normal((n, d)).astype(np.float32), act)
    gate = synth.modulation(wl, 0, 0)[2]
    wo = synth.storage_values(_w(wl, "out"), master)
    gu = synth.storage_values(np.concatenate([_w(wl, "gate"), _w(wl, "up")]), master)
    if wl.weight == "i8":
        po, so = B.pack_int8_weights(cfg, B.W_OUT, to_dev(wo, "bf16"))
        pg, sg = B.pack_int8_weights(cfg, B.W_GATE_UP, to_dev(gu, "bf16"))
        wo_r, gu_r = quant.dequant(*quant.pack_int8(wo)), quant.dequant(*quant.pack_int8(gu))
    else:
        po, so = B.pack_weights(cfg, B.W_OUT, to_dev(wo, master)), None
        pg, sg = B.pack_weights(cfg, B.W_GATE_UP, to_dev(gu, master)), None
        wo_r, gu_r = wo.astype(np.float64), gu.astype(np.float64)
    xd = to_dev(x, act)
    B.linear_residual(cfg, B.W_OUT, to_dev(o, act), po, so, torch.from_numpy(gate).cuda(), xd)
    ref = x + gate * (o.astype(np.float64) @ wo_r.T)
    assert rel_l2(host(xd) - x, ref - x) < tol * 2  # the branch alone
    assert rel_l2(host(xd), ref) < tol
    h = B.linear_swiglu(cfg, to_dev(o, act), pg, sg)
    o64 = o.astype(np.float64)
    href = dit.silu(o64 @ gu_r[:f].T) * (o64 @ gu_r[f:].T)
    assert rel_l2(host(h), href) < tol


# ---------------------------------------------------------------- token reduction
@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_token_merge_unmerge_bit_exact(B, act):
    wl = SMALL if act == "bf16" else SMALL_F32
    cfg, g = binding_cfg(wl), binding_geom(wl)
    og = oracle_geom(wl)
    rng = np.random.default_rng(4)
    x = synth.storage_values(rng.standard_normal((og.n_tokens, wl.d_model)).astype(np.float32) *
                             np.exp(rng.uniform(-30, 30, (og.n_tokens, 1))).astype(np.float32), act)
    xm = B.token_merge(cfg, g, to_dev(x, act))
    ref = tokred.merge(x, og, act)
    np.testing.assert_array_equal(host(xm), ref)
    xu = B.token_unmerge(cfg, g, xm)
    np.testing.assert_array_equal(host(xu), tokred.unmerge(ref, og))


# ---------------------------------------------------------------- Euler
@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_euler_bit_exact(B, act):
    wl = SMALL if act == "bf16" else SMALL_F32
    cfg = binding_cfg(wl)
    rng = np.random.default_rng(6)
    rows = 97
    z = rng.standard_normal((rows, wl.d_model)).astype(np.float32)
    v = synth.storage_values(rng.standard_normal((rows, wl.d_model)).astype(np.float32), act)
    for sigma, sigma_next in ((1.0, 0.95), (0.35, 0.35), (0.25, 0.0), (0.7368421, 0.68421054)):
        zd = torch.from_numpy(z.copy()).cuda()
        vcopy = torch.zeros(rows, wl.d_model, dtype=cfg.act_dtype, device="cuda")
        B.euler(cfg, zd, to_dev(v, act), sigma, sigma_next, vcopy)
        ref = sampler.euler_update(z, sampler.sigma_delta(sigma, sigma_next), v)
        np.testing.assert_array_equal(zd.cpu().numpy().view(np.uint32), ref.view(np.uint32))
        np.testing.assert_array_equal(host(vcopy), v)


# ---------------------------------------------------------------- measurement probe
@pytest.mark.parametrize("dtype", ["bf16", "i8"])
def test_mfma_probe_counts_and_runs(B, dtype):
    """The probe's operation count is 64 MFMAs x 8 waves x one workgroup per CU per iteration,
    and doubling the iterations takes about twice as long (the launch is MFMA work, not
    overhead)."""
    code = B.BF16 if dtype == "bf16" else B.I8
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.zeros(1, dtype=torch.float32, device="cuda")
    per = 2 * 32 * 32 * (16 if dtype == "bf16" else 32) * 64 * 8 * cus
    assert B.mfma_probe(code, 7, out) == per * 7
    times = []
    for iters in (500, 1000):
        B.mfma_probe(code, iters, out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        B.mfma_probe(code, iters, out)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    assert 1.6 < times[1] / times[0] < 2.4
