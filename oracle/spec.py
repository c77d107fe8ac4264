"""Model configuration, derived sizes and the canonical weight list (oracle side).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Configuration fields follow the constructor parameter table of [TRANS]
(section 构造参数详解): sample_size, patch_size, in_channels, num_mmdit_layers,
num_single_dit_layers, attention_head_dim, num_attention_heads,
joint_attention_dim, caption_projection_dim, out_channels, pos_embed_max_size.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace


def find_multiple(n: int, k: int) -> int:
    """Smallest multiple of k that is >= n ([PIPE] section 深入源码 (前馈网络): rounded up to 256)."""
    if n % k == 0:
        return n
    return n + k - (n % k)


@dataclass(frozen=True)
class AuraFlowConfig:
    in_channels: int = 4
    out_channels: int = 4
    patch_size: int = 2
    num_mmdit_layers: int = 4
    num_single_dit_layers: int = 32
    num_attention_heads: int = 12
    attention_head_dim: int = 256
    joint_attention_dim: int = 2048
    caption_projection_dim: int = 3072
    pos_embed_max_size: int = 9216
    num_register_tokens: int = 8
    ln_eps: float = 1e-6
    timestep_scale: float = 1000.0
    timestep_channels: int = 256

    @property
    def inner_dim(self) -> int:
        # [TRANS] 构造参数详解: inner_dim is heads x head_dim (12 x 256 = 3072).
        return self.num_attention_heads * self.attention_head_dim

    @property
    def ffn_dim(self) -> int:
        # [TRANS] 核心子模块架构 (FeedForward): 2/3 of the 4x hidden width, then
        # find_multiple(., 256); [PIPE] 深入源码 says it is rounded up.
        return find_multiple(int(2 * (4 * self.inner_dim) / 3), 256)

    @property
    def pe_grid(self) -> int:
        g = math.isqrt(self.pos_embed_max_size)
        if g * g != self.pos_embed_max_size:
            raise ValueError("pos_embed_max_size must be a perfect square")
        return g

    @property
    def patch_dim(self) -> int:
        return self.patch_size * self.patch_size * self.in_channels

    @property
    def out_patch_dim(self) -> int:
        return self.patch_size * self.patch_size * self.out_channels

    def check(self, H: int, W: int, T: int | None = None) -> tuple[int, int]:
        """Validate a latent size; return the patch grid (h, w)."""
        if self.caption_projection_dim != self.inner_dim:
            raise ValueError("caption_projection_dim must equal heads x head_dim")
        p = self.patch_size
        if H % p or W % p:
            raise ValueError("latent height/width must be divisible by patch_size")
        h, w = H // p, W // p
        G = self.pe_grid
        if h > G or w > G:
            raise ValueError("patch grid larger than the position-embedding grid")
        return h, w


# Config A of the workloads: 4 heads x 8, 1 + 1 blocks, 8 x 8 PE grid, text dim 32.
TINY = AuraFlowConfig(num_mmdit_layers=1, num_single_dit_layers=1, num_attention_heads=4,
                      attention_head_dim=8, joint_attention_dim=32, caption_projection_dim=32,
                      pos_embed_max_size=64)
# Config B: full width, 1 joint + 1 single block.
BLOCK_PAIR = AuraFlowConfig(num_mmdit_layers=1, num_single_dit_layers=1)
# Configs C-E: the full transformer.
FULL = AuraFlowConfig()


def weight_specs(cfg: AuraFlowConfig):
    """Canonical weight list: [(name, shape, std)], in blob order.

    Linear weights are [out, in] and act as y = x @ W.T. PE std 0.1 and
    register std 0.02 follow [TRANS] 核心子模块架构 (Patch Embedding, Register
    Tokens); every other tensor is N(0, 0.02) synthetic init.
    """
    d, F = cfg.inner_dim, cfg.ffn_dim
    specs = [
        ("t_w1", (d, cfg.timestep_channels), 0.02), ("t_b1", (d,), 0.02),
        ("t_w2", (d, d), 0.02), ("t_b2", (d,), 0.02),
        ("pe_w", (d, cfg.patch_dim), 0.02), ("pe_b", (d,), 0.02),
        ("pos_embed", (cfg.pos_embed_max_size, d), 0.1),
        ("ctx_w", (d, cfg.joint_attention_dim), 0.02),
        ("registers", (cfg.num_register_tokens, d), 0.02),
    ]

    def block(prefix):
        return [(prefix + "ada", (6 * d, d), 0.02), (prefix + "wq", (d, d), 0.02),
                (prefix + "wk", (d, d), 0.02), (prefix + "wv", (d, d), 0.02),
                (prefix + "wo", (d, d), 0.02), (prefix + "ff1", (F, d), 0.02),
                (prefix + "ff2", (F, d), 0.02), (prefix + "ff3", (d, F), 0.02)]

    for j in range(cfg.num_mmdit_layers):
        specs += block(f"joint{j}.img.")
        specs += block(f"joint{j}.txt.")
    for i in range(cfg.num_single_dit_layers):
        specs += block(f"single{i}.")
    specs += [("final_ada", (2 * d, d), 0.02), ("proj_out", (cfg.out_patch_dim, d), 0.02)]
    return specs


def count_parameters(cfg: AuraFlowConfig) -> int:
    return sum(math.prod(s) for _, s, _ in weight_specs(cfg))


def with_layers(cfg: AuraFlowConfig, joint: int, single: int) -> AuraFlowConfig:
    return replace(cfg, num_mmdit_layers=joint, num_single_dit_layers=single)
