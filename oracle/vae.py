"""VAE decoder of the pipeline (AutoencoderKL), written plainly (TEST INFRASTRUCTURE ONLY).

The pages name the decoder and how the pipeline uses it, nothing more: the
pipeline holds an AutoencoderKL that maps latents back to images ([PIPE]
AuraFlow 模型与管线概述; [DOCS] vae parameter), the latents are divided by the
VAE's scaling factor before decoding, and an fp16 VAE is upcast to fp32 for the
decode (force_upcast; [TRANS] 在 AuraFlowPipeline 中的实际调用, [PIPE] VAE 上转精度).
Reading taken for the architecture: the published latent-diffusion KL
autoencoder's decoder with the defaults of the AutoencoderKL class — latent
channels 4, block widths (128, 256, 512, 512), three ResNet blocks per
resolution level, GroupNorm with 32 groups (eps 1e-6) and SiLU, one single-head
self-attention in the middle block, nearest-neighbour 2x upsampling followed by
a 3x3 convolution between levels, a 1x1 "post-quant" convolution before the
decoder and a 3x3 convolution to 3 output channels at the end. Weights are
seeded (no trained weights are available).

Conventions: activations NCHW float32 (float64 for the self-check); a
convolution weight is [C_out, C_in, kh, kw] with y[o] = sum_i w[o, i] * x[i]
over the kh x kw window centred on the output pixel (zero padding); 1x1
convolutions and the attention projections are [C_out, C_in] matrices.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class VAEConfig:
    latent_channels: int = 4
    out_channels: int = 3
    block_out_channels: tuple = (128, 256, 512, 512)
    layers_per_block: int = 2          # the decoder runs layers_per_block + 1 ResNet blocks per level
    norm_groups: int = 32
    norm_eps: float = 1e-6
    scaling_factor: float = 0.13025

    @property
    def up_channels(self):
        """Output width of each up level, widest first."""
        return tuple(reversed(self.block_out_channels))


VAE_FULL = VAEConfig()


def vae_weight_specs(cfg: VAEConfig):
    """Canonical decoder weight list: (name, shape, kind) in blob order. kind is
    'w' (matrix or kernel), 'b' (bias), 'g' (GroupNorm scale) or 'n' (GroupNorm shift)."""
    specs = []
    C0 = cfg.up_channels[0]

    def conv(name, cout, cin, k):
        specs.append((name + ".w", (cout, cin, k, k) if k > 1 else (cout, cin), "w"))
        specs.append((name + ".b", (cout,), "b"))

    def norm(name, c):
        specs.append((name + ".g", (c,), "g"))
        specs.append((name + ".n", (c,), "n"))

    def resnet(name, cin, cout):
        norm(name + ".norm1", cin)
        conv(name + ".conv1", cout, cin, 3)
        norm(name + ".norm2", cout)
        conv(name + ".conv2", cout, cout, 3)
        if cin != cout:
            conv(name + ".shortcut", cout, cin, 1)

    conv("post_quant", cfg.latent_channels, cfg.latent_channels, 1)
    conv("conv_in", C0, cfg.latent_channels, 3)
    resnet("mid.res0", C0, C0)
    norm("mid.attn.norm", C0)
    conv("mid.attn.q", C0, C0, 1)
    conv("mid.attn.k", C0, C0, 1)
    conv("mid.attn.v", C0, C0, 1)
    conv("mid.attn.proj", C0, C0, 1)
    resnet("mid.res1", C0, C0)
    cin = C0
    for lvl, cout in enumerate(cfg.up_channels):
        for r in range(cfg.layers_per_block + 1):
            resnet(f"up{lvl}.res{r}", cin, cout)
            cin = cout
        if lvl + 1 < len(cfg.up_channels):
            conv(f"up{lvl}.upsample", cout, cout, 3)
    norm("norm_out", cin)
    conv("conv_out", cfg.out_channels, cin, 3)
    return specs


# ----------------------------------------------------------------------------- pieces

def silu(x):
    return x / (1.0 + np.exp(-x))


def conv2d(x, w, b):
    """Same-size convolution with zero padding: x [B, Ci, H, W], w [Co, Ci, k, k]
    (k odd) or [Co, Ci] (1x1), b [Co] -> [B, Co, H, W]."""
    B, Ci, H, W = x.shape
    if w.ndim == 2:
        return (w @ x.reshape(B, Ci, H * W)).reshape(B, -1, H, W) + b[None, :, None, None]
    k = w.shape[-1]
    p = k // 2
    xp = np.pad(x, ((0, 0), (0, 0), (p, p), (p, p)))
    out = np.zeros((B, w.shape[0], H * W), dtype=x.dtype)
    for dy in range(k):
        for dx in range(k):
            # tap (dy, dx) reads input pixel (y + dy - p, x + dx - p); a matrix
            # product per tap: [Co, Ci] @ [B, Ci, H W]
            shifted = np.ascontiguousarray(xp[:, :, dy:dy + H, dx:dx + W]).reshape(B, Ci, H * W)
            out += np.ascontiguousarray(w[:, :, dy, dx]) @ shifted
    return out.reshape(B, -1, H, W) + b[None, :, None, None]


def group_norm(x, groups, gamma, beta, eps):
    """GroupNorm: statistics (mean, biased variance) over each sample's group of
    C / groups channels and all pixels; per-channel affine gamma, beta."""
    B, C, H, W = x.shape
    xg = x.reshape(B, groups, C // groups, H, W)
    mean = xg.mean(axis=(2, 3, 4), keepdims=True)
    var = ((xg - mean) ** 2).mean(axis=(2, 3, 4), keepdims=True)
    y = ((xg - mean) / np.sqrt(var + eps)).reshape(B, C, H, W)
    return y * gamma[None, :, None, None] + beta[None, :, None, None]


def upsample_nearest2x(x):
    """Output pixel (y, x) takes input pixel (y // 2, x // 2)."""
    return x.repeat(2, axis=2).repeat(2, axis=3)


def resnet_block(x, W, name, cfg, dtype):
    f = lambda n: W[name + n].astype(dtype, copy=False)
    h = conv2d(silu(group_norm(x, cfg.norm_groups, f(".norm1.g"), f(".norm1.n"), dtype(cfg.norm_eps))),
               f(".conv1.w"), f(".conv1.b"))
    h = conv2d(silu(group_norm(h, cfg.norm_groups, f(".norm2.g"), f(".norm2.n"), dtype(cfg.norm_eps))),
               f(".conv2.w"), f(".conv2.b"))
    skip = conv2d(x, f(".shortcut.w"), f(".shortcut.b")) if (name + ".shortcut.w") in W else x
    return skip + h


def attention_block(x, W, name, cfg, dtype):
    """Single-head self-attention over the H x W pixels of each sample, on the
    group-normed input, with 1x1 projections and a residual connection."""
    f = lambda n: W[name + n].astype(dtype, copy=False)
    B, C, H, Wd = x.shape
    h = group_norm(x, cfg.norm_groups, f(".norm.g"), f(".norm.n"), dtype(cfg.norm_eps))
    t = h.reshape(B, C, H * Wd).transpose(0, 2, 1)                     # [B, N, C]
    q = t @ f(".q.w").T + f(".q.b")
    k = t @ f(".k.w").T + f(".k.b")
    v = t @ f(".v.w").T + f(".v.b")
    logits = (q @ k.transpose(0, 2, 1)) / np.sqrt(dtype(C))
    logits = logits - logits.max(axis=-1, keepdims=True)
    p = np.exp(logits)
    p = p / p.sum(axis=-1, keepdims=True)
    o = (p @ v) @ f(".proj.w").T + f(".proj.b")
    return x + o.transpose(0, 2, 1).reshape(B, C, H, Wd)


def decode(cfg: VAEConfig, W, latents, dtype=np.float32, taps=None):
    """latents [B, 4, h, w] (as the sampler leaves them) -> image [B, 3, 8h, 8w].

    taps(name, x) (optional) is called with the activation after the named
    stage: 'conv_in', 'mid', 'up0'..'up3'."""
    f = lambda n: W[n].astype(dtype, copy=False)
    z = np.asarray(latents, dtype) / dtype(cfg.scaling_factor)
    z = conv2d(z, f("post_quant.w"), f("post_quant.b"))
    x = conv2d(z, f("conv_in.w"), f("conv_in.b"))
    if taps:
        taps("conv_in", x)
    x = resnet_block(x, W, "mid.res0", cfg, dtype)
    x = attention_block(x, W, "mid.attn", cfg, dtype)
    x = resnet_block(x, W, "mid.res1", cfg, dtype)
    if taps:
        taps("mid", x)
    for lvl in range(len(cfg.up_channels)):
        for r in range(cfg.layers_per_block + 1):
            x = resnet_block(x, W, f"up{lvl}.res{r}", cfg, dtype)
        if lvl + 1 < len(cfg.up_channels):
            x = conv2d(upsample_nearest2x(x), f(f"up{lvl}.upsample.w"), f(f"up{lvl}.upsample.b"))
        if taps:
            taps(f"up{lvl}", x)
    x = silu(group_norm(x, cfg.norm_groups, f("norm_out.g"), f("norm_out.n"), dtype(cfg.norm_eps)))
    return conv2d(x, f("conv_out.w"), f("conv_out.b"))


# ----------------------------------------------------------------------------- synthetic weights

def vae_weight_recipe(kind: str):
    """Synthetic init (std, mean) by tensor kind: matrices and kernels N(0, 0.02^2),
    biases N(0, 0.02^2), GroupNorm scales N(1, 0.1^2), GroupNorm shifts N(0, 0.02^2)."""
    return {"w": (0.02, 0.0), "b": (0.02, 0.0), "g": (0.1, 1.0), "n": (0.02, 0.0)}[kind]


class VAEWeights(dict):
    """Name -> float32 array for the canonical decoder list, drawn from seeded
    stream (seed, index); bf16=True rounds every tensor to bfloat16 (RNE)."""

    @classmethod
    def seeded(cls, cfg: VAEConfig, seed: int, bf16: bool = False):
        import seeded_inputs
        from .numerics import round_bf16
        out = cls()
        for i, (name, shape, kind) in enumerate(vae_weight_specs(cfg)):
            std, mean = vae_weight_recipe(kind)
            a = seeded_inputs.normal(seed, i, shape, std, mean)
            out[name] = round_bf16(a) if bf16 else a
        return out
