"""AuraFlow transformer forward, written as plainly as possible (TEST INFRASTRUCTURE ONLY).

Tags [PIPE], [DOCS], [TRANS], [DEEP] name the source pages (oracle/__init__.py).

Conventions:
  * Linear layers: y = x @ W.T with W stored [out, in].
  * LN(x) = (x - mean) / sqrt(biased var + eps) over the last axis, no affine.
  * Token order inside one sample: [register tokens, text tokens, image tokens].
  * Everything is computed in ``dtype`` (float32 by default, float64 for the
    self-check); weights and inputs arrive as float32 arrays and are upcast.
"""
from __future__ import annotations

import numpy as np

import seeded_inputs
from .numerics import round_bf16, mxfp8_qdq
from .spec import AuraFlowConfig, weight_specs


# --------------------------------------------------------------------------- weights

class Weights:
    """Name -> float32 array lookup for the canonical weight list.

    ``Weights.seeded`` regenerates each tensor from its own seeded stream on
    demand, so a full-size forward never holds more than one block in memory.
    """

    def __init__(self, cfg: AuraFlowConfig, getter):
        self.cfg = cfg
        self._get = getter

    def __getitem__(self, name: str) -> np.ndarray:
        return self._get(name)

    @classmethod
    def seeded(cls, cfg: AuraFlowConfig, seed: int = seeded_inputs.SEED_WEIGHTS,
               bf16: bool = False, overrides: dict | None = None):
        specs = {name: (i, shape, std) for i, (name, shape, std) in enumerate(weight_specs(cfg))}
        overrides = dict(overrides or {})

        def get(name):
            if name in overrides:
                return np.asarray(overrides[name], np.float32)
            i, shape, std = specs[name]
            a = seeded_inputs.normal(seed, i, shape, std)
            # The position table stays float32; every other tensor is stored in
            # bfloat16 by the bf16 configuration.
            if bf16 and name != "pos_embed":
                a = round_bf16(a)
            return a

        return cls(cfg, get)

    @classmethod
    def from_dict(cls, cfg: AuraFlowConfig, tensors: dict):
        return cls(cfg, lambda name: np.asarray(tensors[name], np.float32))


def _block(W: Weights, prefix: str, dtype):
    names = ("ada", "wq", "wk", "wv", "wo", "ff1", "ff2", "ff3")
    return {n: W[prefix + n].astype(dtype, copy=False) for n in names}


# --------------------------------------------------------------------------- elementwise pieces

def silu(x):
    return x / (1.0 + np.exp(-x))


def layer_norm(x, eps):
    """FP32LayerNorm without affine ([TRANS] 核心子模块架构, 调制与归一化)."""
    mean = x.mean(axis=-1, keepdims=True)
    xc = x - mean
    var = (xc * xc).mean(axis=-1, keepdims=True)
    return xc / np.sqrt(var + eps)


def modulate(n, shift, scale):
    """n * (1 + scale) + shift, with per-sample [B, d] shift/scale broadcast over tokens."""
    return n * (1.0 + scale[:, None, :]) + shift[:, None, :]


# --------------------------------------------------------------------------- embeddings

def timestep_embedding(tau, cfg: AuraFlowConfig, dtype=np.float32):
    """Sinusoidal features of u = timestep_scale * tau ([TRANS] 前向传播流程: Timesteps, 256 channels).

    The pipeline hands the transformer t/1000 ([TRANS] 在 AuraFlowPipeline 中的实际调用); the
    features use u = 1000 * tau. Frequencies f_k = 10000^(-k/half), k = 0..half-1; the
    vector is all cosines, then all sines.
    """
    half = cfg.timestep_channels // 2
    u = np.asarray(tau, dtype) * dtype(cfg.timestep_scale)
    k = np.arange(half, dtype=dtype)
    freqs = np.power(dtype(10000.0), -k / dtype(half))
    args = u[:, None] * freqs[None, :]
    return np.concatenate([np.cos(args), np.sin(args)], axis=1)


def timestep_mlp(e, w1, b1, w2, b2):
    """TimestepEmbedding: Linear -> SiLU -> Linear, both with bias."""
    return silu(e @ w1.T + b1) @ w2.T + b2


def pe_crop_indices(G: int, h: int, w: int) -> np.ndarray:
    """Centre crop of a G x G position grid to h x w, flattened row-major.

    [PIPE] 深入源码 (Patch Embed) and [TRANS] 核心子模块架构 (Patch Embedding): the table
    is viewed as a 2-D grid and the centre sub-block matching the patch grid is
    taken. Odd leftovers put the extra row/column after the crop (floor offset).
    """
    if h > G or w > G:
        raise ValueError("patch grid larger than the position grid")
    r0 = (G - h) // 2
    c0 = (G - w) // 2
    idx = np.empty(h * w, np.int64)
    for i in range(h):
        for j in range(w):
            idx[i * w + j] = (r0 + i) * G + (c0 + j)
    return idx


def patchify(latents, p: int):
    """[B, C, H, W] -> [B, (H/p)(W/p), C*p*p]; token i*w+j, feature order (c, py, px)."""
    B, C, H, W = latents.shape
    h, w = H // p, W // p
    x = latents.reshape(B, C, h, p, w, p).transpose(0, 2, 4, 1, 3, 5)
    return x.reshape(B, h * w, C * p * p)


def unpatchify(z, p: int, C: int, h: int, w: int):
    """[B, h*w, p*p*C] with feature order (py, px, c) -> [B, C, h*p, w*p].

    Same index map as the einsum nhwpqc->nchpwq of [TRANS] 前向传播流程.
    """
    B = z.shape[0]
    x = z.reshape(B, h, w, p, p, C).transpose(0, 5, 1, 3, 2, 4)
    return x.reshape(B, C, h * p, w * p)


def patch_embed(latents, cfg: AuraFlowConfig, pe_w, pe_b, pos_embed, dtype=np.float32):
    """Linear patch projection (with bias) plus the centre-cropped learned PE."""
    B, C, H, W = latents.shape
    h, w = cfg.check(H, W)
    P = patchify(latents.astype(dtype), cfg.patch_size)
    idx = pe_crop_indices(cfg.pe_grid, h, w)
    return P @ pe_w.T + pe_b + pos_embed[idx][None, :, :]


# --------------------------------------------------------------------------- attention / FFN

def _heads(x, H):
    B, N, d = x.shape
    return x.reshape(B, N, H, d // H).transpose(0, 2, 1, 3)


def _merge(o):
    B, H, N, hd = o.shape
    return o.transpose(0, 2, 1, 3).reshape(B, N, H * hd)


def attention(q, k, v, key_valid, scale):
    """softmax(q k^T * scale, keys with key_valid == 0 removed) v, per (batch, head).

    q, k, v: [B, H, S, hd]; key_valid: [B, S] (nonzero = attend). Dropout 0, not
    causal ([TRANS] 注意力处理器与 QKV 融合).
    """
    B, Hh, S, hd = q.shape
    out = np.empty_like(q)
    for b in range(B):
        valid = np.asarray(key_valid[b]) != 0
        kb, vb = k[b][:, valid, :], v[b][:, valid, :]
        for h in range(Hh):
            logits = (q[b, h] @ kb[h].T) * scale
            m = logits.max(axis=1, keepdims=True)
            e = np.exp(logits - m)
            p = e / e.sum(axis=1, keepdims=True)
            out[b, h] = p @ vb[h]
    return out


def attention_bf16_operands(q, k, v, key_valid, scale):
    """The attention of the MXFP8 model: softmax(q k^T * scale) v with the two
    products taking bfloat16 operands -- q and k (after the QK-norm) and v are
    rounded to bfloat16 (round_bf16), and so are the unnormalised probabilities
    e = exp(logit) that multiply v; the normaliser is the sum of the unrounded e,
    and the products accumulate in the working precision. Without the roundings
    this is `attention` exactly (the max shift cancels in the ratio); no shift is
    taken here because the QK-norm bounds every logit by sqrt(hd)^2 * scale
    (16 at hd = 256), so e cannot overflow, and a shift by a whole power of two
    would leave the rounding of e unchanged anyway.
    """
    B, Hh, S, hd = q.shape
    dt = q.dtype
    qb, kb_all, vb_all = round_bf16(q).astype(dt), round_bf16(k).astype(dt), round_bf16(v).astype(dt)
    out = np.empty_like(q)
    for b in range(B):
        valid = np.asarray(key_valid[b]) != 0
        kb, vb = kb_all[b][:, valid, :], vb_all[b][:, valid, :]
        for h in range(Hh):
            e = np.exp((qb[b, h] @ kb[h].T) * scale)
            out[b, h] = (round_bf16(e).astype(dt) @ vb[h]) / e.sum(axis=1, keepdims=True)
    return out


def feed_forward(n, w1, w2, w3, mx=False):
    """SiLU-gated FFN: (silu(n W1^T) * (n W2^T)) W3^T ([PIPE] 深入源码 (前馈网络)).
    mx: the hidden activations are MXFP8-quantized before W3 (operands n and the
    weights arrive already quantized)."""
    return _mxq(silu(n @ w1.T) * (n @ w2.T), mx) @ w3.T


def _mod6(temb, ada):
    """Six modulation vectors [shift1, scale1, gate1, shift2, scale2, gate2] from SiLU(temb) A^T."""
    m = silu(temb) @ ada.T
    return np.split(m, 6, axis=1)


# MXFP8 block GEMMs (mx=True): the QKV projection, the out-projection and both
# FFN products take MXFP8 operands -- the LayerNorm + modulate outputs, the
# attention output, the SiLU-gated hidden activations and the weights of those
# four products are quantized along their contraction axis (mxfp8_qdq) and the
# products accumulate in the working precision. Attention takes bfloat16
# operands (attention_bf16_operands): the E4M3 codes of its output are decided
# from the values that bf16 attention produces. Everything else is unchanged.
MX_WEIGHTS = ("wq", "wk", "wv", "wo", "ff1", "ff2", "ff3")


def mx_block(blk):
    """A block's weight dict with the MXFP8 GEMM weights quantized and dequantized."""
    return {k: (mxfp8_qdq(v) if k in MX_WEIGHTS else v) for k, v in blk.items()}


def _mxq(x, mx):
    return mxfp8_qdq(x).astype(x.dtype) if mx else x


def _qkv(n, blk, cfg, dtype):
    H = cfg.num_attention_heads
    eps = dtype(cfg.ln_eps)
    q = layer_norm(_heads(n @ blk["wq"].T, H), eps)   # QK-norm over the head dim
    k = layer_norm(_heads(n @ blk["wk"].T, H), eps)
    v = _heads(n @ blk["wv"].T, H)
    return q, k, v


def joint_block(cfg, blk_img, blk_txt, temb, x_txt, x_img, key_valid, dtype=np.float32, mx=False):
    """One MMDiT block: two streams with their own weights sharing one attention.

    [TRANS] 核心子模块架构 (联合注意力块) and 注意力处理器与 QKV 融合: per stream
    adaLN-Zero, bias-free Q/K/V with QK-norm, concatenation text-then-image, one
    SDPA, split back, gated out-projection and gated SiLU FFN.
    """
    eps = dtype(cfg.ln_eps)
    scale = dtype(1.0 / np.sqrt(cfg.attention_head_dim))
    Nt = x_txt.shape[1]
    if mx:
        blk_img, blk_txt = mx_block(blk_img), mx_block(blk_txt)
    mi = _mod6(temb, blk_img["ada"])
    mt = _mod6(temb, blk_txt["ada"])
    n_img = _mxq(modulate(layer_norm(x_img, eps), mi[0], mi[1]), mx)
    n_txt = _mxq(modulate(layer_norm(x_txt, eps), mt[0], mt[1]), mx)
    qi, ki, vi = _qkv(n_img, blk_img, cfg, dtype)
    qt, kt, vt = _qkv(n_txt, blk_txt, cfg, dtype)
    attn = attention_bf16_operands if mx else attention
    o = attn(np.concatenate([qt, qi], axis=2), np.concatenate([kt, ki], axis=2),
             np.concatenate([vt, vi], axis=2), key_valid, scale)
    o = _mxq(_merge(o), mx)
    o_txt, o_img = o[:, :Nt], o[:, Nt:]
    x_img = x_img + mi[2][:, None, :] * (o_img @ blk_img["wo"].T)
    x_txt = x_txt + mt[2][:, None, :] * (o_txt @ blk_txt["wo"].T)
    n_img = _mxq(modulate(layer_norm(x_img, eps), mi[3], mi[4]), mx)
    n_txt = _mxq(modulate(layer_norm(x_txt, eps), mt[3], mt[4]), mx)
    x_img = x_img + mi[5][:, None, :] * feed_forward(n_img, blk_img["ff1"], blk_img["ff2"], blk_img["ff3"], mx)
    x_txt = x_txt + mt[5][:, None, :] * feed_forward(n_txt, blk_txt["ff1"], blk_txt["ff2"], blk_txt["ff3"], mx)
    return x_txt, x_img


def single_block(cfg, blk, temb, x, key_valid, dtype=np.float32, mx=False):
    """One DiT block over the concatenated [registers; text; image] sequence.

    [TRANS] 核心子模块架构 (单 DiT 块): self-attention over one sequence with the
    same QK-norm, bias-free, FP32-LayerNorm adaLN-Zero structure.
    """
    eps = dtype(cfg.ln_eps)
    scale = dtype(1.0 / np.sqrt(cfg.attention_head_dim))
    if mx:
        blk = mx_block(blk)
    m = _mod6(temb, blk["ada"])
    n = _mxq(modulate(layer_norm(x, eps), m[0], m[1]), mx)
    q, k, v = _qkv(n, blk, cfg, dtype)
    attn = attention_bf16_operands if mx else attention
    o = _mxq(_merge(attn(q, k, v, key_valid, scale)), mx)
    x = x + m[2][:, None, :] * (o @ blk["wo"].T)
    n = _mxq(modulate(layer_norm(x, eps), m[3], m[4]), mx)
    return x + m[5][:, None, :] * feed_forward(n, blk["ff1"], blk["ff2"], blk["ff3"], mx)


def pre_final(temb, x_img, final_ada):
    """AuraFlowPreFinalBlock: x * (1 + scale) + shift from SiLU(temb) A_f^T, split (scale, shift).

    [TRANS] 调制与归一化 and [PIPE] 深入源码 (pre-final 块): modulation only.
    """
    m = silu(temb) @ final_ada.T
    scale, shift = np.split(m, 2, axis=1)
    return x_img * (1.0 + scale[:, None, :]) + shift[:, None, :]


# --------------------------------------------------------------------------- whole forward

def embed(cfg: AuraFlowConfig, W: Weights, latents, tau, text, text_mask, dtype=np.float32):
    """Embedding stage ([TRANS] 前向传播流程 steps 1-4).

    Returns (temb [B,d], x_txt [B, R+T, d], x_img [B, N, d], key_valid [B, R+T+N]).
    """
    B, C, H, W_ = latents.shape
    T = text.shape[1]
    h, w = cfg.check(H, W_)
    f = lambda name: W[name].astype(dtype, copy=False)
    e = timestep_embedding(tau, cfg, dtype)
    temb = timestep_mlp(e, f("t_w1"), f("t_b1"), f("t_w2"), f("t_b2"))
    x_img = patch_embed(latents, cfg, f("pe_w"), f("pe_b"), f("pos_embed"), dtype)
    ctx = text.astype(dtype) @ f("ctx_w").T                        # no bias
    R = cfg.num_register_tokens
    reg = np.broadcast_to(f("registers")[None], (B, R, cfg.inner_dim))
    x_txt = np.concatenate([reg, ctx], axis=1)
    mask = np.ones((B, T), np.uint8) if text_mask is None else np.asarray(text_mask, np.uint8)
    key_valid = np.concatenate([np.ones((B, R), np.uint8), mask,
                                np.ones((B, h * w), np.uint8)], axis=1)
    return temb, x_txt, x_img, key_valid


def forward(cfg: AuraFlowConfig, W: Weights, latents, tau, text, text_mask=None,
            dtype=np.float32, taps=None, mx=False):
    """Full transformer forward -> [B, out_channels, H, W].

    ``taps(block_index, x_txt, x_img)`` (optional) is called after every block with
    the residual stream split into its text and image rows.
    """
    B, C, H, W_ = latents.shape
    h, w = cfg.check(H, W_)
    temb, x_txt, x_img, key_valid = embed(cfg, W, latents, tau, text, text_mask, dtype)
    Nt = x_txt.shape[1]
    bi = 0
    for j in range(cfg.num_mmdit_layers):
        x_txt, x_img = joint_block(cfg, _block(W, f"joint{j}.img.", dtype),
                                   _block(W, f"joint{j}.txt.", dtype), temb, x_txt, x_img,
                                   key_valid, dtype, mx)
        if taps is not None:
            taps(bi, x_txt, x_img)
        bi += 1
    x = np.concatenate([x_txt, x_img], axis=1)
    for i in range(cfg.num_single_dit_layers):
        x = single_block(cfg, _block(W, f"single{i}.", dtype), temb, x, key_valid, dtype, mx)
        if taps is not None:
            taps(bi, x[:, :Nt], x[:, Nt:])
        bi += 1
    y = pre_final(temb, x[:, Nt:], W["final_ada"].astype(dtype, copy=False))
    z = y @ W["proj_out"].astype(dtype, copy=False).T
    return unpatchify(z, cfg.patch_size, cfg.out_channels, h, w)
