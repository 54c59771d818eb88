"""Benchmark of the DiT denoiser hot path on one MI355X.

Default run (one GPU):
  * step = one DiT block forward (modulated RMSNorm, QKV + 3D RoPE, joint attention, gated
    out-projection, modulated RMSNorm, SwiGLU MLP, gated residual) at d = 6144, 48 heads x 128,
    SwiGLU inner 24576, 6 x 32 x 32 video + 256 audio + 512 text tokens, bf16 weights and
    activations with float32 accumulation. `value` = algorithmic block FLOPs / time (TFLOP/s).
  * roofline of the dominant kernel (the gate/up + SwiGLU GEMM), timed with HIP events around
    its launches on the launch stream inside the timed region; also as a fraction of the
    measured MFMA rate (mfma_probe: register-only MFMAs with changing random operands) next to
    the device copy rate (hbm_copy_gbs).
  * cpu_baseline: the float64 NumPy oracle on a bounded sample of the same block (all K/V rows,
    a few query rows), on this host's cores.
  * block_w8a8: the same block with int8 weights and per-row int8 activations (int8 matrix
    cores, int32 accumulation); its GEMM rates are against the dense int8 peak.
  * denoise: ms per sampler step for the 45-block / 20-step / reuse-2 schedule, the same with
    token reduction over blocks 10..34, velocity extrapolation, core reuse, a four-step
    schedule with a fixed first frame, and the 50-block 4-step schedule at the 6 x 30 x 54 grid
    with int8 weights (W8A16) and with int8 weights and activations (W8A8); synthetic weights
    drawn on the GPU.
Inputs are synthetic and seeded (see synth/).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "DiT block TFLOP/s (% MFMA peak) + ms per denoise step, 512×512×22f"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-denoise", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=64, help="query rows in the oracle sample")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum oracle time")
    p.add_argument("--traffic", type=str, default=None,
                   help="counter summary with the dominant kernel's HBM bytes per launch "
                        "(default: the one under profiles/)")
    p.add_argument("--only-block", action="store_true", help="block timing only (for profilers)")
    p.add_argument("--block-weight", default="bf16", choices=["bf16", "i8", "i8a8"],
                   help="weight type of the block timed with --only-block")
    p.add_argument("--no-w8a8", action="store_true", help="skip the W8A8 block and schedule")
    p.add_argument("--only-probe", action="store_true",
                   help="the MFMA throughput probe alone, bf16 then int8 (for profilers)")
    p.add_argument("--only-sampler", action="store_true",
                   help="the memory-bound kernels alone at the block shape (for profilers)")
    p.add_argument("--copy-calib", action="store_true",
                   help="also run a 1 GiB device copy (byte-counter calibration)")
    return p.parse_args()


def block_flops(n, d, f):
    return 2.0 * n * d * (3 * d + d + 2 * f + f) + 4.0 * n * n * d


def gemm_flops(m, n, k):
    return 2.0 * m * n * k


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(path):
    """HBM bytes per launch of the dominant GEMM from the committed counter summary, or None when
    the GEMM source has changed since the counters were taken."""
    import hashlib

    path = path or os.path.join(ROOT, "profiles", "gemm_gate_up_swiglu_block6912_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path, encoding="utf-8"):
        if ":" in line and not line.startswith(("|", "#", " ")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    src = os.path.join(ROOT, "video_diffusion_transformer_02_amd", "csrc", "k_gemm.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("source_sha256") != sha or "traffic_bytes_per_launch" not in fields:
        return None
    return float(fields["traffic_bytes_per_launch"])


def measure_copy(B, torch, nbytes=1 << 30, reps=10):
    """Device copy rate (read + write bytes per second, GB/s): the practical HBM ceiling the
    memory-bound kernels are compared with."""
    # Both buffers written first, so that every page is backed before it is counted.
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    for _ in range(2):
        B.copy(src, dst)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        B.copy(src, dst)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2.0 * nbytes / ms / 1e6


def measure_mfma(B, torch, dtype, iters=4000, reps=3):
    """Dense MFMA rate with register operands that change every instruction (h3x_mfma_probe):
    the ceiling the GEMMs' instruction mix can reach at the clock the chip holds under matrix
    work, in TFLOP/s (TOP/s for int8)."""
    out = torch.zeros(1, dtype=torch.float32, device="cuda")
    B.mfma_probe(dtype, iters, out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    ops = 0.0
    for _ in range(reps):
        ops += B.mfma_probe(dtype, iters, out)
    e1.record()
    torch.cuda.synchronize()
    return ops / (e0.elapsed_time(e1) * 1e-3) / 1e12


def bench_block(args, B, torch, synth, weight="bf16"):
    w = synth.BLOCK
    cfg = B.BlockCfg.make(w.d_model, w.n_heads, w.head_dim, w.ffn_inner, "bf16", weight)
    g = B.Geom(w.frames, w.grid_h, w.grid_w, w.n_audio, w.n_text, 0)
    n, d, f = g.n_tokens, w.d_model, w.ffn_inner
    log(f"[bench] block workload: N={n} d={d} F={f} heads={w.n_heads}x{w.head_dim} weights={weight}")
    raw = synth.block_weights(w, 0)
    dev = {k: synth.to_storage(v, "bf16").cuda() for k, v in raw.items()}
    pb = B.pack_block(cfg, dev)
    del dev
    mod = synth.modulation(w, 0, 0)
    modd = torch.from_numpy(mod).cuda()
    x_host = synth.block_input(w)
    x = synth.to_storage(x_host, "bf16").cuda()
    ws = B.alloc_workspace(B.block_workspace_bytes(cfg, g))
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        B.dit_block_forward(cfg, g, pb, modd, x, ws)
    torch.cuda.synchronize()
    # Timed region: K steps; every launch inside is bracketed by HIP events on its own stream
    # (the per-kernel durations below), the wall clock gives the step time.
    # Events between consecutive steps on the launch stream give each step's own duration.
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    B.profile_begin()
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        B.dit_block_forward(cfg, g, pb, modd, x, ws)
        evs[i + 1].record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    prof = B.profile_end()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    flops = block_flops(n, d, f)
    log(f"[bench] block {ms:.3f} ms  {flops / ms / 1e9:.1f} TFLOP/s "
        f"(per step: min {per_step[0]:.3f}, median {per_step[len(per_step) // 2]:.3f} ms)")
    if args.copy_calib:
        # A plain copy of known size, for calibrating hardware byte counters.
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.zeros_like(src)
        for _ in range(3):
            B.copy(src, dst)
        torch.cuda.synchronize()
        del src, dst
    kern = {}
    # Projections multiply int8 by int8 in the W8A8 block: their rates are against that peak.
    gemm_peak = PEAK_INT8_TOPS if weight == "i8a8" else PEAK_BF16_TFLOPS
    kflops = {
        "gemm_qkv_rope": gemm_flops(n, 3 * d, d),
        "attention": 4.0 * n * n * d,
        "gemm_out_resid": gemm_flops(n, d, d),
        "gemm_gate_up_swiglu": gemm_flops(n, 2 * f, d),
        "gemm_down_resid": gemm_flops(n, d, f),
    }
    for name, (launches, total_ms) in prof.items():
        avg = total_ms / launches
        e = {"launches": launches, "avg_ms": round(avg, 5)}
        if name in kflops:
            peak = PEAK_BF16_TFLOPS if name == "attention" else gemm_peak
            e["tflops"] = round(kflops[name] / avg / 1e9, 1)
            e["frac_peak"] = round(kflops[name] / avg / 1e9 / peak, 4)
        if name == "norm_mod":
            e["gbs"] = round(2.0 * n * d * 2 / avg / 1e6, 1)
        if name == "norm_mod_quant":  # bf16 row in, int8 codes + a float32 scale per row out
            e["gbs"] = round((3.0 * n * d + 4 * n) / avg / 1e6, 1)
        kern[name] = e
        log(f"[bench]   {name:22s} {avg:8.4f} ms x{launches} {e.get('tflops', '')}")
    dom = "gemm_gate_up_swiglu"
    dom_ms = kern[dom]["avg_ms"]
    achieved = kflops[dom] / dom_ms / 1e9
    traffic = measured_traffic(args.traffic) if weight == "bf16" else None
    roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1), "peak": gemm_peak,
            "unit": "TFLOP/s" if weight != "i8a8" else "TOP/s", "frac": round(achieved / gemm_peak, 4),
            "traffic": traffic, "algorithmic_flops_per_launch": kflops[dom], "avg_launch_ms": dom_ms,
            "timing": "HIP events recorded around each launch on its launch stream, inside the timed region"}
    state = {"raw": raw, "mod": mod, "x": x_host, "w": w,
             "step_ms": {"min": round(per_step[0], 4), "median": round(per_step[len(per_step) // 2], 4)}}
    return ms, flops, kern, roof, state


def bench_sampler(args, B, torch, synth):
    """The memory-bound kernels of the path at the 6 x 32 x 32 + 256 + 512 token, d = 6144 shape:
    modulated RMSNorm, token merge and unmerge (blocks 10..34), the fresh Euler step with the
    velocity-cache write and the reused step; ms and GB/s of their algorithmic bytes."""
    w = synth.BLOCK
    cfg = B.BlockCfg.make(w.d_model, w.n_heads, w.head_dim, w.ffn_inner, "bf16", "bf16")
    g = B.Geom(w.frames, w.grid_h, w.grid_w, w.n_audio, w.n_text, 0)
    n, d = g.n_tokens, w.d_model
    nm = g.as_merged().n_tokens
    ns = w.n_state
    gen = torch.Generator(device="cuda").manual_seed(11)
    x = torch.randn(n, d, generator=gen, device="cuda").to(torch.bfloat16)
    z = torch.randn(ns, d, generator=gen, device="cuda")
    v = torch.randn(ns, d, generator=gen, device="cuda").to(torch.bfloat16)
    vc = torch.empty_like(v)
    mod = torch.from_numpy(synth.modulation(w, 0, 0)).cuda()
    y = torch.empty_like(x)
    xm = B.token_merge(cfg, g, x)
    xu = B.token_unmerge(cfg, g, xm)
    if args.copy_calib:
        measure_copy(B, torch, reps=3)
    runs = {
        "norm_mod": (lambda: B.norm_mod(cfg, x, mod[0], mod[1], y), 2.0 * n * d * 2),
        "token_merge": (lambda: B.token_merge(cfg, g, x), (n + nm) * d * 2.0),
        "token_unmerge": (lambda: B.token_unmerge(cfg, g, xm), (n + nm) * d * 2.0),
        "euler_fresh": (lambda: B.euler(cfg, z, v, 1.0, 0.95, vc), ns * d * (8.0 + 2 + 2)),
        "euler_reused": (lambda: B.euler(cfg, z, v, 0.95, 0.9), ns * d * (8.0 + 2)),
    }
    out = {}
    for name, (fn, nbytes) in runs.items():
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        B.profile_begin()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        prof = B.profile_end()
        launches, total = next(iter(prof.values()))
        ms = total / launches
        out[name] = {"avg_ms": round(ms, 5), "algorithmic_bytes": nbytes, "gbs": round(nbytes / ms / 1e6, 1)}
        log(f"[bench] {name:14s} {ms:.4f} ms  {nbytes / ms / 1e6:7.1f} GB/s")
    del xu
    return out


def cpu_baseline(args, state):
    """The oracle on a bounded sample of the block: K/V of all rows, 64 sampled query rows;
    repeated until about 10 s of CPU time have passed."""
    import synth
    from oracle import dit
    from oracle.geometry import Geometry

    w = state["w"]
    geom = Geometry(w.frames, w.grid_h, w.grid_w, w.n_audio, w.n_text)
    x = synth.storage_values(state["x"], "bf16")
    vals = {k: synth.storage_values(v, "bf16") for k, v in state["raw"].items()}
    rows = synth.sample_rows(w)[: args.cpu_rows]
    n, d, f = geom.n_tokens, w.d_model, w.ffn_inner
    r = len(rows)
    # K and V of all n rows; Q, attention, out-projection and MLP of the r sampled rows.
    flops = 2.0 * 2 * n * d * d + 2.0 * r * d * d + 4.0 * r * n * d + 2.0 * r * d * d + 2.0 * r * d * 3 * f
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count()
    host = host_cpu()
    reps, t0 = 0, time.perf_counter()
    while True:
        dit.block_forward(x, vals, state["mod"], geom, w.n_heads, rows=rows)
        reps += 1
        if time.perf_counter() - t0 >= args.cpu_seconds:
            break
    dt = time.perf_counter() - t0
    log(f"[bench] oracle sample: {reps} x ({r} query rows, {flops / 1e12:.3f} TFLOP) in {dt:.1f} s on {cores} threads"
        f" ({host})")
    # The schedules' work at the sample's rate (extrapolated, not timed): one block, one fresh
    # step of the 45-block schedule without and with token reduction over blocks 10..34 (3840
    # tokens when merged), one step of the 50-block schedule at 6 x 30 x 54 (10488 tokens).
    rate = reps * flops / dt
    nm = w.frames * w.grid_h * w.grid_w // 2 + w.n_audio + w.n_text
    n4 = w.frames * 30 * 54 + w.n_audio + w.n_text
    bf = block_flops(n, d, f)
    extrapolated = {
        "block_ms": round(bf / rate * 1e3, 1),
        "denoise_45blk_fresh_step_ms": round(45 * bf / rate * 1e3, 1),
        "denoise_45blk_tr10_34_fresh_step_ms": round((20 * bf + 25 * block_flops(nm, d, f)) / rate * 1e3, 1),
        "int8w_50blk_6x30x54_step_ms": round(50 * block_flops(n4, d, f) / rate * 1e3, 1),
        "how": "algorithmic FLOPs of the configuration / the sample's measured FLOP rate",
    }
    return {"value": round(rate / 1e12, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"one block at the same shape: K/V of all {n} rows plus {r} of {n} query rows "
                      f"({flops / 1e12:.3f} TFLOP per pass), {reps} passes in {dt:.1f} s",
            "threads": "cores = BLAS threads the oracle ran on", "host": host,
            "extrapolated": extrapolated}


def host_cpu():
    """The host's CPU as the oracle sees it: model name, logical CPUs, CPUs this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": usable, "logical_cpus": os.cpu_count()}


def input_hashes(synth, state):
    """SHA-256 (first 16 MiB, as stored) of the block benchmark's seeded inputs, so that a run can
    be matched with the oracle's inputs."""
    out = {"x": synth.sha256_prefix(synth.to_storage(state["x"], "bf16")),
           "mod": synth.sha256_prefix(state["mod"])}
    for k, v in state["raw"].items():
        out["w_" + k] = synth.sha256_prefix(synth.to_storage(v, "bf16"))
    return out


def bench_denoise(args, B, torch, synth):
    """ms per sampler step on the three schedules; weights drawn on the GPU (seeded)."""
    out = {}
    gen = torch.Generator(device="cuda")

    def rand_bf16(shape, std, seed):
        gen.manual_seed(seed)
        return (torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32) * std).to(torch.bfloat16)

    def run(wl, packed, label, core=None, extrap=False, sched=("linear", 1.0), cond=(0, 0)):
        """core: (k, first, last) core reuse; extrap: linear velocity extrapolation on reused
        steps; sched: sigma schedule (kind, param); cond: fixed condition frames (first, last)."""
        cfg = B.BlockCfg.make(wl.d_model, wl.n_heads, wl.head_dim, wl.ffn_inner, "bf16", wl.weight)
        g = B.Geom(wl.frames, wl.grid_h, wl.grid_w, wl.n_audio, wl.n_text, 0)
        arr = B.block_array(packed)
        ws = B.alloc_workspace(B.step_workspace_bytes(cfg, g))
        z0 = torch.from_numpy(synth.initial_state(wl)).cuda()
        text = synth.to_storage(synth.text_rows(wl), "bf16").cuda()
        mods = [torch.from_numpy(np.stack([synth.modulation(wl, i, b) for b in range(wl.n_blocks)])).cuda()
                for i in range(wl.n_steps)]
        sig = B.sigma_schedule(sched[0], wl.n_steps, sched[1])
        v_prev = torch.empty(wl.n_state, wl.d_model, dtype=torch.bfloat16, device="cuda") if extrap else None
        delta = torch.empty(wl.n_tokens, wl.d_model, dtype=torch.float32, device="cuda") if core else None
        fresh_steps = [i for i in range(wl.n_steps) if B.step_is_fresh(i, wl.n_steps, wl.reuse)]

        def schedule(times):
            z = z0.clone()
            v = torch.empty(wl.n_state, wl.d_model, dtype=torch.bfloat16, device="cuda")
            for i in range(wl.n_steps):
                w = 0.0
                past = [j for j in fresh_steps if j < i]
                if extrap and i not in fresh_steps and len(past) >= 2:
                    w = B.extrapolation_weight(sig[i], sig[past[-1]], sig[past[-2]])
                if times is not None:
                    torch.cuda.synchronize()
                    t0 = time.perf_counter()
                B.denoise_step(cfg, g, i, wl.n_steps, wl.reuse, sig[i], sig[i + 1], arr, mods[i], z, text, v, ws,
                               wl.tr_first, wl.tr_last, cond_first=cond[0], cond_last=cond[1], v_prev=v_prev,
                               extrap=w, core_reuse=core[0] if core else 0, core_first=core[1] if core else 0,
                               core_last=core[2] if core else 0, core_delta=delta)
                if times is not None:
                    torch.cuda.synchronize()
                    times.append((time.perf_counter() - t0) * 1e3)
            return z

        schedule(None)  # warm-up
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        z = schedule(None)
        torch.cuda.synchronize()
        total = (time.perf_counter() - t0) * 1e3
        times = []
        schedule(times)
        fresh = [t for i, t in enumerate(times) if B.step_is_fresh(i, wl.n_steps, wl.reuse)]
        reused = [t for i, t in enumerate(times) if not B.step_is_fresh(i, wl.n_steps, wl.reuse)]
        n_tok = wl.n_tokens
        nm = wl.n_video // 2 + wl.n_audio + wl.n_text
        bf = block_flops(n_tok, wl.d_model, wl.ffn_inner)
        bf_m = block_flops(nm, wl.d_model, wl.ffn_inner)
        per_block = [bf_m if wl.tr_first <= b <= wl.tr_last else bf for b in range(wl.n_blocks)]
        eval_flops = sum(per_block)
        fresh_ms = float(np.mean(fresh))
        res = {"ms_per_step": round(total / wl.n_steps, 3), "total_ms": round(total, 2),
               "fresh_steps": len(fresh), "ms_per_fresh_step": round(fresh_ms, 3),
               "ms_per_reused_step": round(float(np.mean(reused)), 4) if reused else None,
               "finite": bool(torch.isfinite(z).all().item())}
        if core:
            k, first, last = core
            core_fresh = [B.step_is_fresh(i, wl.n_steps, k) for i in range(wl.n_steps)]
            core_part = sum(per_block[first:last + 1])
            flops = sum(eval_flops if cf else eval_flops - core_part for cf in core_fresh)
            res["core_fresh_steps"] = sum(core_fresh)
            res["tflops"] = round(flops / total / 1e9, 1)
        else:
            res["tflops_fresh"] = round(eval_flops / fresh_ms / 1e9, 1)
        if sched[0] != "linear":
            res["sigma"] = [round(x, 4) for x in sig]
        log(f"[bench] {label}: {res}")
        return res

    # 45 blocks, bf16.
    wl = synth.DENOISE45
    cfg = B.BlockCfg.make(wl.d_model, wl.n_heads, wl.head_dim, wl.ffn_inner, "bf16", "bf16")
    d, f = wl.d_model, wl.ffn_inner
    packed = []
    for b in range(wl.n_blocks):
        wts = {"qkv": rand_bf16((3 * d, d), 0.02, 5 * b), "out": rand_bf16((d, d), 0.02, 5 * b + 1),
               "gate": rand_bf16((f, d), 0.02, 5 * b + 2), "up": rand_bf16((f, d), 0.02, 5 * b + 3),
               "down": rand_bf16((d, f), 0.02, 5 * b + 4)}
        packed.append(B.pack_block(cfg, wts))
        del wts
    torch.cuda.synchronize()
    out["denoise_45blk_20step_reuse2"] = run(wl, packed, "45 blocks, 20 steps, reuse 2")
    out["denoise_45blk_20step_reuse2_tr10_34"] = run(synth.DENOISE45_TR, packed, "same + token reduction 10..34")
    out["denoise_45blk_20step_reuse2_extrap"] = run(wl, packed, "reuse 2 with linear velocity extrapolation",
                                                    extrap=True)
    out["denoise_45blk_20step_core4_10_34"] = run(wl.replace(reuse=1), packed, "core reuse 4 over blocks 10..34",
                                                  core=(4, 10, 34))
    out["denoise_45blk_20step_core4_tr10_34"] = run(synth.DENOISE45_TR.replace(reuse=1), packed,
                                                    "core reuse 4 over blocks 10..34 with token reduction 10..34",
                                                    core=(4, 10, 34))
    out["denoise_45blk_4step_linear_terminal_cond1"] = run(
        wl.replace(n_steps=4, reuse=1), packed, "4 steps, linear base grid of 20 + terminal step, first frame fixed",
        sched=("linear_terminal", 20.0), cond=(1, 0))
    del packed
    torch.cuda.empty_cache()

    # 50 blocks, int8 weights packed from bf16 masters.
    wl = synth.INT8_50
    cfg = B.BlockCfg.make(wl.d_model, wl.n_heads, wl.head_dim, wl.ffn_inner, "bf16", "i8")
    packed = []
    for b in range(wl.n_blocks):
        wts = {"qkv": rand_bf16((3 * d, d), 0.02, 1000 + 5 * b), "out": rand_bf16((d, d), 0.02, 1001 + 5 * b),
               "gate": rand_bf16((f, d), 0.02, 1002 + 5 * b), "up": rand_bf16((f, d), 0.02, 1003 + 5 * b),
               "down": rand_bf16((d, f), 0.02, 1004 + 5 * b)}
        packed.append(B.pack_block(cfg, wts))
        del wts
    torch.cuda.synchronize()
    out["int8w_50blk_4step_6x30x54"] = run(wl, packed, "50 blocks int8, 4 steps")
    del packed
    torch.cuda.empty_cache()
    if args.no_w8a8:
        return out

    # The same 50 blocks with int8 weights and per-row int8 activations.
    wl = synth.INT8_50.replace(name="w8a8_50blk_4step_6x30x54", weight="i8a8")
    cfg = B.BlockCfg.make(wl.d_model, wl.n_heads, wl.head_dim, wl.ffn_inner, "bf16", "i8a8")
    packed = []
    for b in range(wl.n_blocks):
        wts = {"qkv": rand_bf16((3 * d, d), 0.02, 1000 + 5 * b), "out": rand_bf16((d, d), 0.02, 1001 + 5 * b),
               "gate": rand_bf16((f, d), 0.02, 1002 + 5 * b), "up": rand_bf16((f, d), 0.02, 1003 + 5 * b),
               "down": rand_bf16((d, f), 0.02, 1004 + 5 * b)}
        packed.append(B.pack_block(cfg, wts))
        del wts
    torch.cuda.synchronize()
    out["w8a8_50blk_4step_6x30x54"] = run(wl, packed, "50 blocks W8A8, 4 steps")
    del packed
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch

    import synth
    from video_diffusion_transformer_02_amd import binding as B

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    B.lib()
    if args.only_probe:
        probe = {"bf16_tflops": round(measure_mfma(B, torch, B.BF16), 1),
                 "i8_tops": round(measure_mfma(B, torch, B.I8), 1)}
        print(json.dumps({"mfma_probe": probe}))
        return
    if args.only_sampler:
        print(json.dumps({"sampler_kernels": bench_sampler(args, B, torch, synth)}))
        return
    if args.only_block:
        ms, flops, kern, roof, state = bench_block(args, B, torch, synth, args.block_weight)
        print(json.dumps({"ms_per_step": ms, "weights": args.block_weight, "kernels": kern}))
        return
    ms, flops, kern, roof, state = bench_block(args, B, torch, synth)
    copy_gbs = measure_copy(B, torch)
    log(f"[bench] device copy {copy_gbs:.0f} GB/s (read + write)")
    probe = {"bf16_tflops": round(measure_mfma(B, torch, B.BF16), 1),
             "i8_tops": round(measure_mfma(B, torch, B.I8), 1)}
    log(f"[bench] MFMA probe {probe['bf16_tflops']:.0f} TFLOP/s bf16, {probe['i8_tops']:.0f} TOP/s int8")
    roof["frac_of_probe"] = round(roof["achieved"] / probe["bf16_tflops"], 4)
    sampler = bench_sampler(args, B, torch, synth)
    for e in sampler.values():
        e["frac_copy"] = round(e["gbs"] / copy_gbs, 3)
    for name in ("norm_mod", "norm_mod_quant"):
        if name in kern and "gbs" in kern[name]:
            kern[name]["frac_copy"] = round(kern[name]["gbs"] / copy_gbs, 3)
    w8a8 = None
    if not args.no_w8a8:
        ms8, _, kern8, roof8, _ = bench_block(args, B, torch, synth, "i8a8")
        roof8["frac_of_probe"] = round(roof8["achieved"] / probe["i8_tops"], 4)
        w8a8 = {"ms_per_step": round(ms8, 4), "tops": round(flops / ms8 / 1e9, 2),
                "speedup_vs_bf16": round(ms / ms8, 3), "dominant": roof8, "kernels": kern8}
    denoise = None if args.no_denoise else bench_denoise(args, B, torch, synth)
    cpu = None if args.no_cpu_baseline else cpu_baseline(args, state)
    w = synth.BLOCK
    line = {
        "metric": METRIC,
        "value": round(flops / ms / 1e9, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, N(0,0.02^2) weights, random-init)",
        "config": {"workload": "one DiT block, 6x32x32 video + 256 audio + 512 text tokens",
                   "d_model": w.d_model, "heads": w.n_heads, "head_dim": w.head_dim,
                   "ffn_inner": w.ffn_inner, "tokens": w.n_tokens, "block_flops": flops},
        "frac_of_peak": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
        "block_step_ms": state["step_ms"],
        "roofline": roof,
        "hbm_copy_gbs": round(copy_gbs, 1),
        "mfma_probe": probe,
        "sampler_kernels": sampler,
        "cpu_baseline": cpu,
        "inputs_sha256": input_hashes(synth, state),
        "kernels": kern,
        "block_w8a8": w8a8,
        "denoise": denoise,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
