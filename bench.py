#!/usr/bin/env python3
"""Throughput of one AuraFlow transformer forward on one MI355X.

Default workload: 1024 x 1024 image (latent 4 x 128 x 128 -> 4096 image tokens,
8 register + 256 text tokens, sequence 4360), CFG batch 2 ([uncond; cond] sharing
one latent and timestep), 4 joint + 32 single blocks, d = 3072, bf16 weights
drawn from the seeded synthetic recipe. One step = one full forward through the
C-ABI (every kernel of the path), inputs already resident in HBM.

Prints one JSON line. The timed region is bracketed by synchronisation and
measured with HIP events on the forward's stream (every kernel of the forward
runs on it, in order). A separate per-kernel pass brackets each launch with HIP
events on the same stream for the roofline and per-class times.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def _cpu_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except Exception:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# BLAS threads for the CPU-baseline leg (must be set before numpy loads).
os.environ.setdefault("OPENBLAS_NUM_THREADS", str(_cpu_threads()))
os.environ.setdefault("OMP_NUM_THREADS", str(_cpu_threads()))

import numpy as np  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published
MX_CLASSES = ("gemm_qkv", "gemm_out", "gemm_ffn_up", "gemm_ffn_down")   # products on MXFP8 operands in --mxfp8 runs
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published

WORKLOADS = {
    # name: (B, latent H, latent W, text T)
    "1024": (2, 128, 128, 256),
    "1536": (2, 192, 192, 256),
}


def forward_flops(d, F, L, B, S, T, Dtxt, Nimg, patch_dim):
    """Algorithmic FLOPs of one forward: QKV, attention (QK^T and PV), out-proj and
    FFN per block, plus caption projection, patch embed and output projection."""
    per_block = 2 * S * d * 3 * d + 4 * S * S * d + 2 * S * d * d + 6 * S * d * F
    return B * L * per_block + B * (2 * T * Dtxt * d + 4 * Nimg * patch_dim * d)


def class_work(name, d, F, B, S, mod_rows=0):
    """(algorithmic FLOPs or bytes per launch, unit kind) for a kernel class.
    mod_rows: rows of the gathered modulation matrix (6 d per block and stream, 2 d final)."""
    M = B * S
    if name == "gemm_qkv":
        return 2.0 * M * d * 3 * d, "mfma"
    if name == "gemm_out":
        return 2.0 * M * d * d, "mfma"
    if name == "gemm_ffn_up":
        return 2.0 * M * d * 2 * F, "mfma"
    if name == "gemm_ffn_down":
        return 2.0 * M * F * d, "mfma"
    if name == "attention":
        return 4.0 * B * S * S * d, "mfma"
    if name == "ln_modulate":
        return float(M * d * 4 + M * d * 2), "hbm"   # fp32 residual in, bf16 out
    if name == "adaln" and mod_rows:
        # bf16 weights of the timestep MLP (256 -> d -> d) and of every modulation row,
        # each read once; the vectors in and out are a few MB
        return float(2 * (d * 256 + d * d + mod_rows * d)), "hbm"
    return None, None


# HBM traffic per launch of a kernel class, from rocprofv3 FETCH_SIZE / WRITE_SIZE
# counter runs summarised under profiles/. A summary names the kernel's source
# files and the sha256 of their concatenation; when a source has changed since,
# the figure no longer describes the kernel and is not reported.
TRAFFIC_PROFILES = {
    "gemm_ffn_up": "profiles/gemm_ffn_up_1024x1024_cfg2_hbm_traffic.md",
}


def measured_traffic(kclass):
    import hashlib
    path = TRAFFIC_PROFILES.get(kclass)
    if path is None or not os.path.exists(os.path.join(ROOT, path)):
        return None
    fields = {}
    for line in open(os.path.join(ROOT, path)):
        if ":" in line and line.startswith("- `"):
            k, v = line[3:].split("`", 1)[0], line.split(":", 1)[1].strip().strip("`")
            fields[k] = v
    srcs = fields.get("kernel_source", "").split()
    if not srcs or not all(os.path.exists(os.path.join(ROOT, f)) for f in srcs):
        return None
    h = hashlib.sha256()
    for f in srcs:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    digest = h.hexdigest()
    if digest != fields.get("source_sha256"):
        return None
    return float(fields["hbm_bytes_per_launch"])


def copy_calibration():
    """A plain device copy of 512 MiB, four times: the reference the FETCH_SIZE and
    WRITE_SIZE counters are scaled by (run under rocprofv3 --pmc)."""
    import torch
    a = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(4):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copied {a.numel() * 4} bytes, 4 times", flush=True)


def cpu_baseline(shape, threads):
    """The oracle (fp32 numpy) on a bounded sample: embedding + one joint block +
    one single block at the full workload shape; forward time extrapolated as
    embed + 4 joint + 32 single."""
    import oracle
    import seeded_inputs
    from oracle import transformer as T_

    B, H, W, T = shape
    cfg = oracle.FULL
    lat = np.concatenate([seeded_inputs.latents(1, 4, H, W)] * B)
    tau = np.full(B, 0.5, np.float32)
    text = oracle.round_bf16(seeded_inputs.text_embeddings(B, T, cfg.joint_attention_dim))
    mask = seeded_inputs.length_mask(seeded_inputs.valid_lengths(B, 16, T), T)
    names = ["t_w1", "t_b1", "t_w2", "t_b2", "pe_w", "pe_b", "pos_embed", "ctx_w", "registers"]
    blk_names = [n for n, _, _ in oracle.weight_specs(cfg) if n.startswith(("joint0.", "single0."))]
    Wseed = oracle.Weights.seeded(cfg, seed=0, bf16=True)
    t0 = time.time()
    cache = {n: Wseed[n] for n in names + blk_names}
    gen_s = time.time() - t0
    Wt = oracle.Weights.from_dict(cfg, cache)
    f32 = np.float32
    t0 = time.time()
    temb, xt, xi, kv = oracle.embed(cfg, Wt, lat, tau, text, mask, f32)
    t_embed = time.time() - t0
    blk = lambda p: {k: Wt[p + k] for k in ("ada", "wq", "wk", "wv", "wo", "ff1", "ff2", "ff3")}
    t0 = time.time()
    xt2, xi2 = oracle.joint_block(cfg, blk("joint0.img."), blk("joint0.txt."), temb, xt, xi, kv, f32)
    t_joint = time.time() - t0
    x = np.concatenate([xt2, xi2], axis=1)
    t0 = time.time()
    oracle.single_block(cfg, blk("single0."), temb, x, kv, f32)
    t_single = time.time() - t0
    t_fwd = t_embed + cfg.num_mmdit_layers * t_joint + cfg.num_single_dit_layers * t_single
    return {
        "value": 1.0 / t_fwd, "unit": "forwards/s", "cores": threads, "kind": "oracle",
        "sample": (f"numpy fp32 oracle, BLAS threads={threads}: embedding ({t_embed:.2f} s) + 1 joint block "
                   f"({t_joint:.2f} s) + 1 single block ({t_single:.2f} s) at the full {8 * W}x{8 * H}-pixel CFG-batch-2 "
                   f"shape; forward extrapolated as embed + 4 joint + 32 single = {t_fwd:.1f} s (extrapolated, not a "
                   f"timed full forward); weight generation ({gen_s:.1f} s) excluded"),
        "blas": blas_vendor(),
        "full_forwards": oracle_full_forwards(),
    }


def blas_vendor():
    """The BLAS library numpy was built against (name and version as numpy reports them)."""
    try:
        dep = np.__config__.CONFIG["Build Dependencies"]["blas"]
        return f"{dep.get('name')} {dep.get('version')}"
    except Exception:
        return "unknown"


def oracle_full_forwards():
    """Timed whole oracle forwards (fp32 numpy) of the two small workloads: the tiny
    fp32 transformer (1 joint + 1 single block, 4 heads x 8, latent 4x16x16, 8 text
    tokens, batch 1, t = 500) and the full-width block pair (1 joint + 1 single block,
    d = 3072, latent 4x64x64, 256 text tokens, CFG batch 2). Weight generation and
    bf16 rounding are excluded."""
    import oracle
    import seeded_inputs
    from dataclasses import replace
    out = {}
    cases = {
        "tiny_fp32": (replace(oracle.TINY), 1, 16, 8, False),
        "block_pair_512": (replace(oracle.FULL, num_mmdit_layers=1, num_single_dit_layers=1), 2, 64, 256, True),
    }
    for name, (cfg, B, lat_hw, T, bf16) in cases.items():
        W_ = oracle.Weights.seeded(cfg, seed=0, bf16=bf16)
        W_ = oracle.Weights.from_dict(cfg, {n: W_[n] for n, _, _ in oracle.weight_specs(cfg)})
        if B == 2:
            lat = np.concatenate([seeded_inputs.latents(1, 4, lat_hw, lat_hw)] * 2)
            t = seeded_inputs.timesteps_uniform(1) / 1000.0
            tau = np.concatenate([t, t]).astype(np.float32)
            mask = seeded_inputs.length_mask(seeded_inputs.valid_lengths(B, 16, T), T)
        else:
            lat = seeded_inputs.latents(1, 4, lat_hw, lat_hw)
            tau = np.array([0.5], np.float32)
            mask = None
        text = seeded_inputs.text_embeddings(B, T, cfg.joint_attention_dim)
        if bf16:
            text = oracle.round_bf16(text)
        t0 = time.time()
        oracle.forward(cfg, W_, lat, tau, text, mask, np.float32)
        dt = time.time() - t0
        out[name] = {"s_per_forward": dt, "value": 1.0 / dt, "unit": "forwards/s",
                     "config": f"{cfg.num_mmdit_layers} joint + {cfg.num_single_dit_layers} single blocks, "
                               f"d={cfg.inner_dim}, latent 4x{lat_hw}x{lat_hw}, {T} text tokens, batch {B}"}
    return out


def text_encoder_leg(args, af, torch, steps, warmup):
    """The pipeline's text encoder (UMT5: 24 layers, d_model 2048, 32 heads of 64, d_ff 5120,
    vocabulary 32128) on 8 prompts x 256 tokens (a CFG batch of 4 images: 4 prompts and 4
    negative prompts), random bf16 weights, ragged valid lengths. Returns the timing object."""
    import seeded_inputs
    B, T = 8, 256
    cfg = af.umt5_make_config(max_batch=B, max_tokens=T)
    d, F, L = cfg.d_model, cfg.d_ff, cfg.num_layers
    enc = af.UMT5Encoder(cfg, 0)
    enc.load_seeded_weights(threads=_cpu_threads())
    ids = torch.from_numpy(seeded_inputs.token_ids(B, T, cfg.vocab_size)).cuda()
    mask = torch.from_numpy(seeded_inputs.length_mask(seeded_inputs.valid_lengths(B, 16, T), T)).cuda()
    out = torch.empty((B, T, d), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        enc.encode(ids, mask, out=out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "non-finite text-encoder output"
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        enc.encode(ids, mask, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    M = B * T
    flops = L * (2.0 * M * d * 3 * d + 2.0 * M * d * d + 2.0 * M * d * 2 * F + 2.0 * M * F * d + 4.0 * B * T * T * d)
    enc.close()
    return {"workload": f"UMT5 text encoder, {L} layers, d_model {d}, {cfg.num_heads} heads of 64, d_ff {F}, "
                        f"vocabulary {cfg.vocab_size}; {B} prompts x {T} tokens, ragged valid lengths; seeded "
                        f"random bf16 weights",
            "ms_per_encode": ms, "value": 1000.0 / ms, "unit": "encodes/s", "flops_per_encode": flops,
            "tflops": flops / (ms * 1e-3) / 1e12, "pct_peak_bf16": 100.0 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def vae_flops(cfg, B, h, w):
    """Algorithmic FLOPs of one decode (2 per multiply-add; convolutions over their
    real input channels, attention's two products and four projections)."""
    ch = list(cfg.block_out_channels)[::-1]
    P = h * w
    conv = lambda P_, cin, cout, k: 2.0 * B * P_ * k * cin * cout

    def res(P_, cin, cout):
        return conv(P_, cin, cout, 9) + conv(P_, cout, cout, 9) + (conv(P_, cin, cout, 1) if cin != cout else 0.0)

    f = conv(P, cfg.latent_channels, cfg.latent_channels, 1) + conv(P, cfg.latent_channels, ch[0], 9)
    C = ch[0]
    f += 2 * res(P, C, C) + 4 * conv(P, C, C, 1) + 4.0 * B * P * P * C
    cin = C
    for l in range(4):
        for r in range(cfg.layers_per_block + 1):
            f += res(P, cin, ch[l])
            cin = ch[l]
        if l < 3:
            P *= 4
            f += conv(P, cin, cin, 9)
    return f + conv(P, cin, cfg.out_channels, 9)


def vae_leg(args, af, torch, steps, warmup):
    """The VAE decode (AutoencoderKL decoder, widths 512/512/256/128, three ResNet blocks
    per level, mid-block attention over the 128 x 128 latent pixels) of 4 latents
    [4, 4, 128, 128] into 4 images of 1024 x 1024, random bf16 weights. Returns the
    timing object."""
    import seeded_inputs
    B, h, w = 4, 128, 128
    cfg = af.vae_make_config(max_batch=B, max_latent_h=h, max_latent_w=w)
    dec = af.VAEDecoder(cfg, 0)
    dec.load_seeded_weights(threads=_cpu_threads())
    lat = torch.from_numpy(seeded_inputs.latents(B, cfg.latent_channels, h, w, first_index=300)).cuda()
    out = torch.empty((B, cfg.out_channels, 8 * h, 8 * w), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        dec.decode(lat, out=out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "non-finite VAE output"
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        dec.decode(lat, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = vae_flops(cfg, B, h, w)
    dec.close()
    return {"workload": f"VAE decode (AutoencoderKL decoder, widths {list(cfg.block_out_channels)[::-1]}, "
                        f"{cfg.layers_per_block + 1} ResNet blocks per level, mid-block attention over {h * w} "
                        f"pixels) of {B} latents [{B}, {cfg.latent_channels}, {h}, {w}] into {B} images of "
                        f"{8 * h}x{8 * w}; seeded random bf16 weights",
            "ms_per_decode": ms, "value": B * 1000.0 / ms, "unit": "images/s", "flops_per_decode": flops,
            "tflops": flops / (ms * 1e-3) / 1e12, "pct_peak_bf16": 100.0 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def sampling_loop_bench(args, af, torch):
    """--sampling-loop: the 25-step CFG loop for 4 images at 1024^2 (transformer batch 8)
    as its own JSON line; --steps counts loops."""
    imgs, H, W, T = 4, 128, 128, 256
    B = 2 * imgs
    cfg = af.make_config(max_batch=B, max_latent_h=H, max_latent_w=W, max_text_len=T,
                         compute_dtype=af.AF_MXFP8 if args.mxfp8 else af.AF_BF16)
    model = af.AuraFlowModel(cfg, 0)
    model.load_seeded_weights(seed=0, threads=_cpu_threads())
    leg = loop_leg(af, torch, model, cfg, args.steps, args.warmup, imgs, H, W, T)
    print(json.dumps({
        "metric": "25-step CFG sampling loop, 4 images at 1024² (transformer batch 8)",
        "value": leg["value"], "unit": "images/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": leg["ms_per_loop"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp8+bf16" if args.mxfp8 else "bf16", "data": "synthetic",
        "config": {"workload": leg["workload"] + "; a step is one whole 25-step loop",
                   "global_batch": B, "seq_len": cfg.num_register_tokens + T + (H // 2) * (W // 2),
                   "parallelism": "single GPU"},
        "tflops": leg["tflops"], "pct_peak_bf16": leg["pct_peak_bf16"],
    }))
    model.close()


def workload_tensors(torch, af_cfg, B, H, W, T):
    """The bench's seeded inputs: CFG pairs sharing one latent and timestep,
    independent text rows, seeded valid lengths with the padding masked."""
    import seeded_inputs
    lat1 = seeded_inputs.latents(B // 2, 4, H, W)
    lat = torch.from_numpy(np.concatenate([lat1, lat1])).cuda()
    t = seeded_inputs.timesteps_uniform(B // 2) / 1000.0
    tau = torch.from_numpy(np.concatenate([t, t]).astype(np.float32)).cuda()
    text = torch.from_numpy(seeded_inputs.text_embeddings(B, T, af_cfg.joint_attention_dim)).cuda()
    mask = torch.from_numpy(seeded_inputs.length_mask(seeded_inputs.valid_lengths(B, 16, T), T)).cuda()
    return lat, tau, text, mask


def forward_leg(af, torch, model, cfg, B, H, W, T, steps, warmup):
    """Forwards/s, TFLOP/s and the attention roofline of one more workload on an
    existing model (timed as the headline: HIP events on the forward's stream)."""
    d = cfg.num_attention_heads * cfg.attention_head_dim
    F = ((8 * d) // 3 + 255) // 256 * 256
    L = cfg.num_mmdit_layers + cfg.num_single_dit_layers
    Nimg = (H // 2) * (W // 2)
    S = cfg.num_register_tokens + T + Nimg
    lat, tau, text, mask = workload_tensors(torch, cfg, B, H, W, T)
    out = torch.empty((B, 4, H, W), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        model.forward(lat, tau, text, mask, out=out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), f"non-finite output at {8 * W}x{8 * H}"
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        model.forward(lat, tau, text, mask, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    af.af_profile(model, True)
    for _ in range(steps):
        model.forward(lat, tau, text, mask, out=out)
    torch.cuda.synchronize()
    prof = af.af_profile_read(model)
    af.af_profile(model, False)
    kms, n = prof["attention"]
    work, _ = class_work("attention", d, F, B, S)
    att = work / (kms / n * 1e-3) / 1e12
    flops = forward_flops(d, F, L, B, S, T, cfg.joint_attention_dim, Nimg, 16)
    return {"workload": f"AuraFlow transformer forward at {8 * W}x{8 * H} pixels (latent 4x{H}x{W}: {Nimg} image + "
                        f"8 register + {T} text tokens, sequence {S}), CFG batch {B}, same model and recipe",
            "ms_per_step": ms, "value": 1000.0 / ms, "unit": "forwards/s", "steps": steps, "warmup": warmup,
            "flops_per_forward": flops, "tflops": flops / (ms * 1e-3) / 1e12,
            "pct_peak_bf16": 100.0 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "attention": {"avg_launch_ms": kms / n, "launches_per_forward": n / steps, "work_per_launch": work,
                          "tflops": att, "peak": PEAK_BF16_TFLOPS, "frac_peak": att / PEAK_BF16_TFLOPS}}


def loop_leg(af, torch, model, cfg, loops, warmup_loops, imgs=4, H=128, W=128, T=256, steps=25):
    """The 25-step flow-matching Euler + CFG loop (shift 1.73, guidance 3.5) for `imgs`
    images at 1024^2 on an existing model: transformer batch 2 imgs per step. Wall
    time per loop from HIP events around whole loops."""
    import seeded_inputs
    B = 2 * imgs
    d = cfg.num_attention_heads * cfg.attention_head_dim
    F = ((8 * d) // 3 + 255) // 256 * 256
    L = cfg.num_mmdit_layers + cfg.num_single_dit_layers
    Nimg = (H // 2) * (W // 2)
    S = cfg.num_register_tokens + T + Nimg
    x0 = torch.from_numpy(seeded_inputs.latents(imgs, 4, H, W)).cuda()
    text = torch.from_numpy(seeded_inputs.text_embeddings(B, T, cfg.joint_attention_dim)).cuda()
    mask = torch.from_numpy(seeded_inputs.length_mask(seeded_inputs.valid_lengths(B, 16, T), T)).cuda()
    x = torch.empty_like(x0)
    stream = torch.cuda.current_stream()

    def loop():
        x.copy_(x0)
        model.sample(x, text, mask, num_steps=steps, shift=1.73, guidance=3.5)

    for _ in range(warmup_loops):
        loop()
    torch.cuda.synchronize()
    assert bool(torch.isfinite(x).all()), "non-finite latents after the warm-up loop"
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(loops):
        loop()
    e1.record(stream)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(x).all()), "non-finite latents after the timed loops"
    ms = e0.elapsed_time(e1) / loops
    flops = steps * forward_flops(d, F, L, B, S, T, cfg.joint_attention_dim, Nimg, 16)
    return {"workload": f"flow-matching Euler sampling, {steps} steps, shift 1.73, guidance 3.5, {imgs} images at "
                        f"{8 * W}x{8 * H} (latent 4x{H}x{W}), [{imgs} uncond; {imgs} cond] per forward (transformer "
                        f"batch {B}), seeded random weights and text, padded text masked",
            "ms_per_loop": ms, "value": imgs * 1000.0 / ms, "unit": "images/s", "loops": loops,
            "warmup_loops": warmup_loops, "flops_per_loop": flops, "tflops": flops / (ms * 1e-3) / 1e12,
            "pct_peak_bf16": 100.0 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20 forwards; 10 loops with --sampling-loop)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="1024")
    ap.add_argument("--latent", default=None, metavar="HxW",
                    help="any latent size (even, at most 192 x 192) instead of the workload's square one")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true")
    ap.add_argument("--mxfp8", action="store_true",
                    help="time the MXFP8 model (QKV, out-projection and FFN products on MXFP8 operands) as the main line")
    ap.add_argument("--no-mxfp8-leg", action="store_true",
                    help="skip the extra MXFP8-model timing reported beside the bf16 line")
    ap.add_argument("--sampling-loop", action="store_true",
                    help="time the 25-step flow-matching Euler + CFG sampling loop for 4 images at 1024^2 "
                         "(transformer batch 8) instead of single forwards; --steps counts loops")
    ap.add_argument("--text-encoder", action="store_true",
                    help="time only the text encoder (8 prompts x 256 tokens) and print its own line")
    ap.add_argument("--no-text-encoder-leg", action="store_true",
                    help="skip the text-encoder timing reported beside the transformer line")
    ap.add_argument("--vae", action="store_true",
                    help="time only the VAE decode (4 latents of 128 x 128 into 1024 x 1024 images) and print its own line")
    ap.add_argument("--no-vae-leg", action="store_true",
                    help="skip the VAE-decode timing reported beside the transformer line")
    ap.add_argument("--no-graph-leg", action="store_true",
                    help="skip the graph-replay timing reported beside the eager line")
    ap.add_argument("--no-extra-legs", action="store_true",
                    help="skip the 1536^2 forward and the 25-step sampling loop reported beside the headline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the plain 512 MiB device copy used to scale the HBM byte counters")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 10 if args.sampling_loop else 20
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the forward runs on a single MI355X and this build has no "
              f"multi-GPU path (--gpus {args.gpus} requested).", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return

    import torch
    import flow_matching_mmdit_amd as pkg
    if not os.path.exists(pkg.LIB_PATH):
        from flow_matching_mmdit_amd import build as _b
        _b.build()
    from flow_matching_mmdit_amd import binding as af
    import seeded_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.sampling_loop:
        sampling_loop_bench(args, af, torch)
        return
    if args.text_encoder:
        leg = text_encoder_leg(args, af, torch, args.steps, args.warmup)
        print(json.dumps({"metric": "UMT5 text-encoder encodes/s (8 prompts x 256 tokens)", "value": leg["value"],
                          "unit": "encodes/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "ms_per_step": leg["ms_per_encode"], "higher_is_better": True, "scaling": "weak",
                          "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                          "config": {"workload": leg["workload"], "global_batch": 8, "seq_len": 256,
                                     "parallelism": "single GPU"},
                          "tflops": leg["tflops"], "pct_peak_bf16": leg["pct_peak_bf16"]}))
        return
    if args.vae:
        leg = vae_leg(args, af, torch, args.steps, args.warmup)
        print(json.dumps({"metric": "VAE decode images/s (4 latents 128x128 -> 1024x1024)", "value": leg["value"],
                          "unit": "images/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "ms_per_step": leg["ms_per_decode"], "higher_is_better": True, "scaling": "weak",
                          "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                          "config": {"workload": leg["workload"], "global_batch": 4, "seq_len": 16384,
                                     "parallelism": "single GPU"},
                          "tflops": leg["tflops"], "pct_peak_bf16": leg["pct_peak_bf16"]}))
        return
    B, H, W, T = WORKLOADS[args.workload]
    if args.latent:
        H, W = (int(x) for x in args.latent.lower().split("x"))
    # the headline run also times 1536^2 and the batch-8 sampling loop on the same
    # model, so its workspace is sized for both (the size does not change the kernels)
    extra = not args.no_extra_legs and not args.mxfp8 and not args.latent and args.workload == "1024"
    cfg = af.make_config(max_batch=max(B, 8) if extra else B, max_latent_h=max(H, 192) if extra else H,
                         max_latent_w=max(W, 192) if extra else W, max_text_len=T,
                         compute_dtype=af.AF_MXFP8 if args.mxfp8 else af.AF_BF16)
    d = cfg.num_attention_heads * cfg.attention_head_dim
    F = ((8 * d) // 3 + 255) // 256 * 256
    L = cfg.num_mmdit_layers + cfg.num_single_dit_layers
    Nimg = (H // 2) * (W // 2)
    S = cfg.num_register_tokens + T + Nimg

    t0 = time.time()
    model = af.AuraFlowModel(cfg, 0)
    model.load_seeded_weights(seed=0, threads=_cpu_threads())
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    print(f"[bench] weights ready in {setup_s:.1f} s", file=sys.stderr, flush=True)

    # Workload inputs: CFG pair sharing one latent and timestep, independent text, padded text masked.
    lat, tau, text, mask = workload_tensors(torch, cfg, B, H, W, T)
    out = torch.empty((B, 4, H, W), dtype=torch.float32, device="cuda")

    def check_finite(where):
        bad = (~torch.isfinite(out)).reshape(B, -1).sum(1).tolist()
        assert sum(bad) == 0, f"non-finite output after {where}: per-sample counts {bad}"

    for _ in range(args.warmup):
        model.forward(lat, tau, text, mask, out=out)
    torch.cuda.synchronize()
    check_finite("warm-up")
    print(f"[bench] warmup done", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    per_fwd = []

    def timed(n):
        # outer events bracket the n forwards; one event between consecutive forwards
        # (no synchronisation) gives the per-forward spread
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        e0.record(stream)
        ev[0].record(stream)
        for i in range(n):
            model.forward(lat, tau, text, mask, out=out)
            ev[i + 1].record(stream)
        e1.record(stream)
        torch.cuda.synchronize()
        per_fwd[:] = [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]
        return e0.elapsed_time(e1) / n

    ms_per_step = timed(args.steps)
    pct = {f"p{q}": float(np.percentile(per_fwd, q)) for q in (10, 50, 90)}
    value = 1000.0 / ms_per_step
    flops = forward_flops(d, F, L, B, S, T, cfg.joint_attention_dim, Nimg, 16)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    check_finite("the timed forwards")
    print(f"[bench] {ms_per_step:.2f} ms/forward, {tflops:.1f} TFLOP/s", file=sys.stderr, flush=True)

    # The same forward captured once in a HIP graph (through torch's capture of the
    # current stream) and replayed: no host launch work inside the timed region.
    graph_leg = None
    if not args.no_graph_leg:
        out_g = torch.empty_like(out)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            model.forward(lat, tau, text, mask, out=out_g)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            model.forward(lat, tau, text, mask, out=out_g)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out), "graph replay differs from the eager forward"
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        msg = e0.elapsed_time(e1) / args.steps
        graph_leg = {"ms_per_step": msg, "value": 1000.0 / msg, "unit": "forwards/s",
                     "note": "the forward captured once in a HIP graph and replayed (same kernels, outputs equal)"}
        del g
        print(f"[bench] graph replay: {msg:.2f} ms/forward", file=sys.stderr, flush=True)

    kernels, roofline = {}, None
    if not args.no_profile:
        af.af_profile(model, True)
        for _ in range(args.steps):
            model.forward(lat, tau, text, mask, out=out)
        torch.cuda.synchronize()
        prof = af.af_profile_read(model)
        af.af_profile(model, False)
        best = None
        for name, (kms, n) in prof.items():
            if n == 0:
                continue
            mod_rows = (2 * cfg.num_mmdit_layers + cfg.num_single_dit_layers) * 6 * d + 2 * d
            work, kind = class_work(name, d, F, B, S, mod_rows)
            entry = {"ms_per_forward": kms / args.steps, "launches_per_forward": n / args.steps,
                     "avg_launch_ms": kms / n}
            if work is not None:
                rate = work / (kms / n * 1e-3)
                if kind == "mfma":
                    peak = PEAK_FP8_TFLOPS if args.mxfp8 and name in MX_CLASSES else PEAK_BF16_TFLOPS
                    entry["tflops"] = rate / 1e12
                    entry["frac_peak"] = rate / 1e12 / peak
                else:
                    entry["gbs"] = rate / 1e9
                    entry["frac_peak"] = rate / 1e9 / PEAK_HBM_GBS
                if best is None or kms > best[1]:
                    best = (name, kms, n, work, kind)
            kernels[name] = entry
        if best is not None:
            name, kms, n, work, kind = best
            avg = kms / n * 1e-3
            if kind == "mfma":
                peak = PEAK_FP8_TFLOPS if args.mxfp8 and name in MX_CLASSES else PEAK_BF16_TFLOPS
                roofline = {"bound": "mfma", "kernel": name, "achieved": work / avg / 1e12,
                            "peak": peak, "unit": "TFLOP/s", "frac": work / avg / 1e12 / peak,
                            "traffic": None if args.mxfp8 else measured_traffic(name),
                            "avg_launch_ms": avg * 1e3, "work_per_launch": work}
            else:
                roofline = {"bound": "hbm", "kernel": name, "achieved": work / avg / 1e9, "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "frac": work / avg / 1e9 / PEAK_HBM_GBS, "traffic": measured_traffic(name),
                            "avg_launch_ms": avg * 1e3, "work_per_launch": work}

    # Beside the headline, on the same model: 1536^2 (the attention-dominated
    # workload) and the 25-step sampling loop for 4 images (transformer batch 8).
    d_leg = loop = None
    if extra:
        d_leg = forward_leg(af, torch, model, cfg, 2, 192, 192, T, min(args.steps, 10), 2)
        print(f"[bench] 1536^2: {d_leg['ms_per_step']:.2f} ms/forward, attention "
              f"{d_leg['attention']['avg_launch_ms']:.3f} ms/launch", file=sys.stderr, flush=True)
        loop = loop_leg(af, torch, model, cfg, 1, 1)
        print(f"[bench] sampling loop: {loop['ms_per_loop'] / 1000:.2f} s per 25-step loop of 4 images",
              file=sys.stderr, flush=True)

    # Beside the bf16 line: the same workload on the MXFP8 model (QKV, out-projection
    # and FFN products on MXFP8 operands), timed the same way; reported as its own
    # object, never as `value`.
    mx_leg = None
    if not args.mxfp8 and not args.no_mxfp8_leg:
        model.close()
        del model
        torch.cuda.synchronize()
        cfg8 = af.make_config(max_batch=B, max_latent_h=H, max_latent_w=W, max_text_len=T, compute_dtype=af.AF_MXFP8)
        model = af.AuraFlowModel(cfg8, 0)
        model.load_seeded_weights(seed=0, threads=_cpu_threads())
        for _ in range(args.warmup):
            model.forward(lat, tau, text, mask, out=out)
        torch.cuda.synchronize()
        check_finite("MXFP8 warm-up")
        ms8 = timed(args.steps)
        check_finite("the MXFP8 timed forwards")
        print(f"[bench] MXFP8 model: {ms8:.2f} ms/forward", file=sys.stderr, flush=True)
        mx_leg = {"ms_per_step": ms8, "value": 1000.0 / ms8, "unit": "forwards/s",
                  "tflops": flops / (ms8 * 1e-3) / 1e12,
                  "note": "same workload; QKV, out-projection and FFN products on MXFP8 operands (E4M3 values, "
                          "one power-of-two scale per 32 along K), attention on bf16 operands, the rest fp32; "
                          "TFLOP/s counts the dense model FLOPs",
                  "parity": "tests/test_gpu_mxfp8.py: every sampled block's update within 6e-2 / cosine 0.998 "
                            "of the oracle's mx mode; the 36-block output within 1.5x the oracle's own change "
                            "under a one-ulp change of the latents"}

    te = None
    if not args.no_text_encoder_leg and not args.mxfp8:
        model.close()
        del model
        torch.cuda.synchronize()
        te = text_encoder_leg(args, af, torch, args.steps, args.warmup)
        print(f"[bench] text encoder: {te['ms_per_encode']:.2f} ms/encode", file=sys.stderr, flush=True)

    vae = None
    if not args.no_vae_leg and not args.mxfp8:
        if te is None:
            model.close()
            del model
            torch.cuda.synchronize()
        vae = vae_leg(args, af, torch, args.steps, args.warmup)
        print(f"[bench] VAE decode: {vae['ms_per_decode']:.2f} ms per 4 images", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        print(f"[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline((B, H, W, T), _cpu_threads())

    res = {
        "metric": "AuraFlow transformer forwards/s at 1024² CFG batch 2; TFLOP/s as % of bf16 peak",
        "value": value,
        "unit": "forwards/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8+bf16" if args.mxfp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": f"AuraFlow transformer forward at {8 * W}x{8 * H} pixels "
                               f"(latent 4x{H}x{W}: {Nimg} image + 8 register + {T} text tokens), CFG batch {B}, "
                               f"4 joint + 32 single blocks, d=3072, 12x256 heads, FFN 8192, seeded random "
                               f"bf16 weights (6.86B params), padded text masked"
                               + (", QKV and FFN products on MXFP8 operands" if args.mxfp8 else ""),
                   "global_batch": B, "seq_len": S, "parallelism": "single GPU"},
        "tflops": tflops,
        "pct_peak_bf16": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "forward_ms_percentiles": pct,
        "flops_per_forward": flops,
        "roofline": roofline,
        "graph_replay": graph_leg,
        "config_1536": d_leg,
        "sampling_loop": loop,
        "mxfp8_model": mx_leg,
        "text_encoder": te,
        "vae_decode": vae,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "setup_s": setup_s,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
