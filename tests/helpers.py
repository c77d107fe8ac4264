"""Shared helpers for the GPU parity tests: config translation, seeded inputs,
comparison metrics. No model arithmetic lives here."""
from __future__ import annotations

import numpy as np

import oracle
import seeded_inputs


def oracle_cfg(c) -> oracle.AuraFlowConfig:
    """The oracle's config with the same sizes as a library AfConfig."""
    return oracle.AuraFlowConfig(
        in_channels=c.in_channels, out_channels=c.out_channels, patch_size=c.patch_size,
        num_mmdit_layers=c.num_mmdit_layers, num_single_dit_layers=c.num_single_dit_layers,
        num_attention_heads=c.num_attention_heads, attention_head_dim=c.attention_head_dim,
        joint_attention_dim=c.joint_attention_dim, caption_projection_dim=c.caption_projection_dim,
        pos_embed_max_size=c.pos_embed_max_size, num_register_tokens=c.num_register_tokens,
        ln_eps=float(np.float32(c.ln_eps)), timestep_scale=float(c.timestep_scale))


def workload_inputs(B, C, H, W, T, Dtxt, lengths=None, cfg_pairs=True, tau=None):
    """Seeded inputs in the shape of the pages' workloads.

    cfg_pairs: the batch is [uncond; cond] halves sharing one latent per image
    (latents duplicated for CFG) and one timestep; text drawn independently per
    row. lengths: per-row valid text lengths (None = all valid).
    """
    if cfg_pairs:
        assert B % 2 == 0
        half = seeded_inputs.latents(B // 2, C, H, W)
        lat = np.concatenate([half, half])
        t = seeded_inputs.timesteps_uniform(B // 2) if tau is None else None
        taus = np.concatenate([t, t]) / 1000.0 if tau is None else np.full(B, tau)
    else:
        lat = seeded_inputs.latents(B, C, H, W)
        taus = seeded_inputs.timesteps_uniform(B) / 1000.0 if tau is None else np.full(B, tau)
    text = seeded_inputs.text_embeddings(B, T, Dtxt)
    mask = None if lengths is None else seeded_inputs.length_mask(np.asarray(lengths), T)
    return lat, taus.astype(np.float32), text, mask


def rel_max(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(a - ref).max() / np.abs(ref).max())


def cosine(a, ref):
    a = np.asarray(a, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    return float(a @ ref / (np.linalg.norm(a) * np.linalg.norm(ref)))


def to_dev(x, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


class PrefetchWeights:
    """Oracle weight getter that draws one block's tensors at a time with a thread
    pool (same seeded streams as oracle.Weights.seeded) and keeps only that block.
    Test-side plumbing so a full-size oracle forward streams 27 GB of weights."""

    def __init__(self, cfg, seed=0, bf16=True, threads=16):
        from concurrent.futures import ThreadPoolExecutor
        self.cfg = cfg
        self._base = oracle.Weights.seeded(cfg, seed=seed, bf16=bf16)
        self._specs = oracle.weight_specs(cfg)
        self._cache = {}
        self._pool = ThreadPoolExecutor(threads)

    @staticmethod
    def _group(name):
        return name.rsplit(".", 1)[0] if "." in name else "_embed"

    def __getitem__(self, name):
        # the two most recent groups stay cached (a joint block's two streams)
        grp = self._group(name)
        if grp not in self._cache:
            names = [n for n, _, _ in self._specs if self._group(n) == grp]
            if len(self._cache) >= 2:
                self._cache.pop(next(iter(self._cache)))
            self._cache[grp] = dict(zip(names, self._pool.map(lambda n: self._base[n], names)))
        return self._cache[grp][name]

    def as_weights(self):
        return oracle.Weights(self.cfg, self.__getitem__)


BLOCK_KEYS = ("ada", "wq", "wk", "wv", "wo", "ff1", "ff2", "ff3")


def block_weights(W, prefix):
    return {k: W[prefix + k] for k in BLOCK_KEYS}


def oracle_block_on(ocfg, W, temb, kv, x_prev, b, Nt, mx=False):
    """The oracle's block b (0-based over the joint, then the single blocks) applied
    to the residual x_prev [B, S, d] (rows [registers, text, image] per sample;
    the first Nt rows are the text stream)."""
    x_prev = np.asarray(x_prev, np.float32)
    if b < ocfg.num_mmdit_layers:
        xt, xi = oracle.joint_block(ocfg, block_weights(W, f"joint{b}.img."), block_weights(W, f"joint{b}.txt."),
                                    temb, x_prev[:, :Nt], x_prev[:, Nt:], kv, np.float32, mx)
        return np.concatenate([xt, xi], 1)
    return oracle.single_block(ocfg, block_weights(W, f"single{b - ocfg.num_mmdit_layers}."), temb, x_prev, kv,
                               np.float32, mx)


def update_metrics(got_prev, got, ref_next):
    """A block's own update: the GPU's (got - got_prev) against the oracle's update of
    the same input residual (ref_next - got_prev); returns (max|d|/max|ref|, cosine)."""
    dg = np.asarray(got, np.float64) - got_prev
    dr = np.asarray(ref_next, np.float64) - got_prev
    return rel_max(dg, dr), cosine(dg, dr)
