"""UMT5 text encoder (the pipeline's text encoder) as a random-weight workload.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

[DEEP] section 2.1 (文本编码器: UMT5EncoderModel) gives the configuration: d_model
2048, 32 heads, 24 layers, d_ff 5120, a 32128-token vocabulary and a relative
attention maximum distance of 128; [DOCS] (AuraFlowPipeline parameters) and
[TRANS] (在 AuraFlowPipeline 中的实际调用) name it as a frozen T5-family encoder
whose output, [batch, seq_len, 2048], is the transformer's text input. The pages
say nothing more about its arithmetic, so this module takes the published T5
encoder layer (Raffel et al., "Exploring the Limits of Transfer Learning with a
Unified Text-to-Text Transformer", section 2.1) with the UMT5 choices, and
every such reading is listed here:

  * the token embedding is looked up, not scaled;
  * each layer is pre-norm: x += SelfAttention(Norm(x)); x += FFN(Norm(x)); a
    final Norm follows the last layer;
  * Norm is the T5 layer norm: x / sqrt(mean(x^2) + eps) * weight (no mean
    subtraction, no bias), eps = 1e-6;
  * attention: heads of d_model / heads = 64 channels, projections without
    bias, logits q.k with no 1/sqrt(d) factor, plus a learned per-head bias of
    the relative position (key index - query index) in 32 bidirectional buckets
    (16 per sign: 8 exact distances, then 8 logarithmic steps up to distance
    128, larger distances share the last bucket); UMT5 gives every layer its own
    bias table; keys of padded tokens are excluded; a query whose sample has no
    valid key gets a zero output;
  * the feed-forward is gated GELU in its tanh form: wo(gelu(wi_0 x) * wi_1 x).

The logarithmic bucket is the floor of a real number; it is computed here with
exact integer comparisons (no floating-point log), which is the value of the
formula itself at every distance, including distances where it is an integer.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

import seeded_inputs
from .numerics import round_bf16


@dataclass(frozen=True)
class UMT5Config:
    d_model: int = 2048
    num_heads: int = 32
    num_layers: int = 24
    d_ff: int = 5120
    vocab_size: int = 32128
    rel_buckets: int = 32
    rel_max_distance: int = 128
    eps: float = 1e-6

    @property
    def d_kv(self) -> int:
        return self.d_model // self.num_heads


UMT5_FULL = UMT5Config()
# Two layers at the full width (a parity case that the oracle finishes in seconds).
UMT5_PAIR = replace(UMT5_FULL, num_layers=2)
# A narrow two-layer encoder: 4 heads of 64, d_ff 512, a 1000-token vocabulary.
UMT5_SMALL = UMT5Config(d_model=256, num_heads=4, num_layers=2, d_ff=512, vocab_size=1000)

LAYER_TENSORS = ("ln1", "wq", "wk", "wv", "wo", "rel_bias", "ln2", "wi0", "wi1", "wo_ff")


def umt5_weight_specs(cfg: UMT5Config):
    """Canonical weight list: (name, shape, std, mean) in blob order. Matrices are
    [out, in] (y = x W^T); norm weights are drawn around 1; the relative-position
    tables are [buckets, heads]."""
    d, F = cfg.d_model, cfg.d_ff
    specs = [("embed", (cfg.vocab_size, d), 1.0, 0.0)]
    for l in range(cfg.num_layers):
        p = f"layer{l}."
        specs += [
            (p + "ln1", (d,), 0.1, 1.0),
            (p + "wq", (d, d), 0.01, 0.0),
            (p + "wk", (d, d), 0.01, 0.0),
            (p + "wv", (d, d), 0.02, 0.0),
            (p + "wo", (d, d), 0.02, 0.0),
            (p + "rel_bias", (cfg.rel_buckets, cfg.num_heads), 0.5, 0.0),
            (p + "ln2", (d,), 0.1, 1.0),
            (p + "wi0", (F, d), 0.02, 0.0),
            (p + "wi1", (F, d), 0.02, 0.0),
            (p + "wo_ff", (d, F), 0.02, 0.0),
        ]
    specs.append(("final_ln", (d,), 0.1, 1.0))
    return specs


class UMT5Weights:
    """Name -> float32 array; seeded tensors are regenerated on demand. With
    bf16=True the embedding and the matrices are rounded to bfloat16 (norm
    weights and relative-position tables stay float32)."""

    def __init__(self, getter):
        self._get = getter

    def __getitem__(self, name):
        return self._get(name)

    @classmethod
    def seeded(cls, cfg: UMT5Config, seed: int = seeded_inputs.SEED_ENCODER_WEIGHTS, bf16: bool = False):
        specs = {n: (i, shape, std, mean) for i, (n, shape, std, mean) in enumerate(umt5_weight_specs(cfg))}

        def get(name):
            i, shape, std, mean = specs[name]
            a = seeded_inputs.normal(seed, i, shape, std, mean)
            if bf16 and len(shape) == 2 and not name.endswith("rel_bias"):
                a = round_bf16(a)
            return a

        return cls(get)


# --------------------------------------------------------------------------- pieces

def rms_norm(x, w, eps):
    """T5 layer norm: x / sqrt(mean(x^2) + eps) * w over the last axis."""
    var = (x * x).mean(axis=-1, keepdims=True)
    return x / np.sqrt(var + eps) * w


def gelu_tanh(x):
    """GELU in its tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x * x * x)))


def _log_steps(n: int, max_exact: int, max_distance: int, steps: int) -> int:
    """floor(steps * log(n / max_exact) / log(max_distance / max_exact)) for n >= max_exact,
    exactly: the largest k in [0, steps] with (n / max_exact)^steps >= (max_distance / max_exact)^k,
    i.e. n^steps * max_exact^k >= max_distance^k * max_exact^steps (Python integers)."""
    lhs = n ** steps
    best = 0
    for k in range(0, steps + 1):
        if lhs * max_exact ** k >= max_distance ** k * max_exact ** steps:
            best = k
    return best


def relative_bucket(rel, num_buckets: int = 32, max_distance: int = 128):
    """Bucket of relative position rel = key index - query index (bidirectional):
    half the buckets for each sign (positive distances offset by half); inside a
    half, distances below half/2 are exact and larger ones take logarithmic steps
    up to max_distance, clipped to the half's last bucket."""
    rel = np.asarray(rel, np.int64)
    half = num_buckets // 2
    max_exact = half // 2
    steps = half - max_exact
    n = np.abs(rel)
    out = np.where(rel > 0, half, 0).astype(np.int64)
    table = {}
    for v in np.unique(n):
        v = int(v)
        if v < max_exact:
            table[v] = v
        else:
            table[v] = min(max_exact + _log_steps(v, max_exact, max_distance, steps), half - 1)
    return out + np.vectorize(table.__getitem__, otypes=[np.int64])(n)


def position_bias(rel_bias, T: int, cfg: UMT5Config):
    """[H, T, T] additive bias: bias[h, i, j] = rel_bias[bucket(j - i), h]."""
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    b = relative_bucket(j - i, cfg.rel_buckets, cfg.rel_max_distance)
    return np.transpose(rel_bias[b], (2, 0, 1))


def self_attention(n, wq, wk, wv, wo, rel_bias, key_valid, cfg: UMT5Config):
    """Multi-head self-attention of one layer on normalised rows n [B, T, d]."""
    B, T, d = n.shape
    H, dk = cfg.num_heads, cfg.d_kv

    def heads(y):
        return y.reshape(B, T, H, dk).transpose(0, 2, 1, 3)

    q, k, v = heads(n @ wq.T), heads(n @ wk.T), heads(n @ wv.T)
    s = q @ k.transpose(0, 1, 3, 2) + position_bias(rel_bias, T, cfg)[None].astype(n.dtype)
    s = np.where(key_valid[:, None, None, :], s, -np.inf)
    any_valid = key_valid.any(axis=1)[:, None, None, None]
    m = np.where(any_valid, s.max(axis=-1, keepdims=True), 0.0)
    p = np.where(any_valid, np.exp(s - m), 0.0)
    den = p.sum(axis=-1, keepdims=True)
    o = (p @ v) / np.where(den > 0, den, 1.0)
    o = o.transpose(0, 2, 1, 3).reshape(B, T, d)
    return o @ wo.T


def feed_forward(n, wi0, wi1, wo_ff):
    return (gelu_tanh(n @ wi0.T) * (n @ wi1.T)) @ wo_ff.T


def encode(cfg: UMT5Config, W: UMT5Weights, ids, mask=None, dtype=np.float32, taps=None):
    """ids [B, T] int, mask [B, T] (nonzero = valid token) -> [B, T, d_model].

    taps(l, x) is called with the residual stream after layer l."""
    ids = np.asarray(ids)
    B, T = ids.shape
    key_valid = np.ones((B, T), bool) if mask is None else np.asarray(mask) != 0
    x = W["embed"][ids].astype(dtype)
    for l in range(cfg.num_layers):
        g = {n: W[f"layer{l}.{n}"].astype(dtype, copy=False) for n in LAYER_TENSORS}
        x = x + self_attention(rms_norm(x, g["ln1"], cfg.eps), g["wq"], g["wk"], g["wv"], g["wo"],
                               g["rel_bias"], key_valid, cfg)
        x = x + feed_forward(rms_norm(x, g["ln2"], cfg.eps), g["wi0"], g["wi1"], g["wo_ff"])
        if taps is not None:
            taps(l, x)
    return rms_norm(x, W["final_ln"].astype(dtype), cfg.eps)
