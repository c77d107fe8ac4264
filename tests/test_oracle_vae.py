"""Pins for the oracle's VAE decoder (oracle/vae.py): each piece against an
independent definition (explicit loops over the textbook formula), closed forms
and invariants, so that a dropped term, a wrong sign or index, or a transposed
operand fails one of them."""
import math
from dataclasses import replace

import numpy as np
import pytest

from oracle import vae as V

F64 = np.float64


def _conv_loops(x, w, b):
    """Zero-padded 'same' convolution written as the definition: y[n, o, i, j] =
    b[o] + sum_c sum_u sum_v w[o, c, u, v] x[n, c, i + u - p, j + v - p]."""
    B, C, H, W = x.shape
    O, _, k, _ = w.shape
    p = k // 2
    y = np.zeros((B, O, H, W))
    for n in range(B):
        for o in range(O):
            for i in range(H):
                for j in range(W):
                    s = b[o]
                    for c in range(C):
                        for u in range(k):
                            for v in range(k):
                                ii, jj = i + u - p, j + v - p
                                if 0 <= ii < H and 0 <= jj < W:
                                    s += w[o, c, u, v] * x[n, c, ii, jj]
                    y[n, o, i, j] = s
    return y


def test_conv3x3_matches_the_definition_with_zero_padding():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((2, 3, 4, 5))
    w = rng.standard_normal((2, 3, 3, 3))
    b = rng.standard_normal(2)
    np.testing.assert_allclose(V.conv2d(x, w, b), _conv_loops(x, w, b), rtol=1e-12, atol=1e-12)


def test_conv_kernel_orientation():
    """A kernel with a single 1 at (row 0, col 2) reads the up-right neighbour:
    y[i, j] = x[i - 1, j + 1] (zero outside)."""
    x = np.arange(20, dtype=F64).reshape(1, 1, 4, 5)
    w = np.zeros((1, 1, 3, 3))
    w[0, 0, 0, 2] = 1.0
    y = V.conv2d(x, w, np.zeros(1))[0, 0]
    for i in range(4):
        for j in range(5):
            want = x[0, 0, i - 1, j + 1] if (i - 1 >= 0 and j + 1 < 5) else 0.0
            assert y[i, j] == want


def test_conv1x1_is_a_channel_matrix():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 4, 3, 3))
    w = rng.standard_normal((5, 4))
    b = rng.standard_normal(5)
    y = V.conv2d(x, w, b)
    for n in range(2):
        for i in range(3):
            for j in range(3):
                np.testing.assert_allclose(y[n, :, i, j], w @ x[n, :, i, j] + b, rtol=1e-12)


def _gn_loops(x, G, g, be, eps):
    B, C, H, W = x.shape
    y = np.empty_like(x)
    cg = C // G
    for n in range(B):
        for grp in range(G):
            vals = [x[n, c, i, j] for c in range(grp * cg, (grp + 1) * cg) for i in range(H) for j in range(W)]
            m = sum(vals) / len(vals)
            var = sum((t - m) ** 2 for t in vals) / len(vals)
            for c in range(grp * cg, (grp + 1) * cg):
                y[n, c] = (x[n, c] - m) / math.sqrt(var + eps) * g[c] + be[c]
    return y


def test_group_norm_matches_loops_and_normalises_each_group():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 8, 3, 4)) * 3 + 1
    g, be = rng.standard_normal(8), rng.standard_normal(8)
    np.testing.assert_allclose(V.group_norm(x, 4, g, be, 1e-6), _gn_loops(x, 4, g, be, 1e-6), rtol=1e-10, atol=1e-12)
    y = V.group_norm(x, 4, np.ones(8), np.zeros(8), 1e-6)
    yg = y.reshape(2, 4, 2, 3, 4)
    np.testing.assert_allclose(yg.mean(axis=(2, 3, 4)), 0, atol=1e-12)
    np.testing.assert_allclose(yg.var(axis=(2, 3, 4)), 1, atol=1e-5)
    # groups are independent: changing group 3's channels leaves groups 0-2 unchanged
    x2 = x.copy()
    x2[:, 6:] *= 10
    np.testing.assert_array_equal(V.group_norm(x2, 4, g, be, 1e-6)[:, :6], V.group_norm(x, 4, g, be, 1e-6)[:, :6])


def test_upsample_index_map():
    x = np.arange(6, dtype=F64).reshape(1, 1, 2, 3)
    y = V.upsample_nearest2x(x)
    assert y.shape == (1, 1, 4, 6)
    for i in range(4):
        for j in range(6):
            assert y[0, 0, i, j] == x[0, 0, i // 2, j // 2]


def _small_cfg():
    return replace(V.VAE_FULL, block_out_channels=(8, 16), layers_per_block=1, norm_groups=4)


def test_attention_with_zero_query_key_is_the_mean_of_the_values():
    """q = k = 0 makes every logit equal: each pixel attends uniformly, so the
    block adds proj(mean over pixels of v) to every pixel."""
    cfg = _small_cfg()
    W = V.VAEWeights.seeded(cfg, seed=3)
    W = {k: v.astype(F64) for k, v in W.items()}
    C = cfg.up_channels[0]
    for n in ("mid.attn.q.w", "mid.attn.q.b", "mid.attn.k.w", "mid.attn.k.b"):
        W[n] = np.zeros_like(W[n])
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, C, 3, 5))
    y = V.attention_block(x, W, "mid.attn", cfg, F64)
    h = V.group_norm(x, cfg.norm_groups, W["mid.attn.norm.g"], W["mid.attn.norm.n"], cfg.norm_eps)
    for n in range(2):
        vbar = np.mean([W["mid.attn.v.w"] @ h[n, :, i, j] + W["mid.attn.v.b"] for i in range(3) for j in range(5)], axis=0)
        add = W["mid.attn.proj.w"] @ vbar + W["mid.attn.proj.b"]
        np.testing.assert_allclose(y[n] - x[n], np.broadcast_to(add[:, None, None], (C, 3, 5)), rtol=1e-10, atol=1e-12)


def test_attention_matches_explicit_softmax():
    cfg = _small_cfg()
    W = {k: v.astype(F64) for k, v in V.VAEWeights.seeded(cfg, seed=5).items()}
    W["mid.attn.q.w"] = W["mid.attn.q.w"] * 20          # sharpen the softmax so errors show
    C = cfg.up_channels[0]
    rng = np.random.default_rng(6)
    x = rng.standard_normal((1, C, 2, 3))
    y = V.attention_block(x, W, "mid.attn", cfg, F64)
    h = V.group_norm(x, cfg.norm_groups, W["mid.attn.norm.g"], W["mid.attn.norm.n"], cfg.norm_eps)[0]
    pix = [(i, j) for i in range(2) for j in range(3)]
    q = {p: W["mid.attn.q.w"] @ h[:, p[0], p[1]] + W["mid.attn.q.b"] for p in pix}
    k = {p: W["mid.attn.k.w"] @ h[:, p[0], p[1]] + W["mid.attn.k.b"] for p in pix}
    v = {p: W["mid.attn.v.w"] @ h[:, p[0], p[1]] + W["mid.attn.v.b"] for p in pix}
    for p in pix:
        logits = [float(q[p] @ k[r]) / math.sqrt(C) for r in pix]
        mx = max(logits)
        e = [math.exp(t - mx) for t in logits]
        o = sum(ei / sum(e) * v[r] for ei, r in zip(e, pix))
        want = x[0, :, p[0], p[1]] + W["mid.attn.proj.w"] @ o + W["mid.attn.proj.b"]
        np.testing.assert_allclose(y[0, :, p[0], p[1]], want, rtol=1e-10)


def test_resnet_block_with_zero_second_conv_is_its_skip_path():
    cfg = _small_cfg()
    W = {k: v.astype(F64) for k, v in V.VAEWeights.seeded(cfg, seed=7).items()}
    rng = np.random.default_rng(8)
    # same width: identity skip
    W["mid.res0.conv2.w"][:] = 0
    W["mid.res0.conv2.b"][:] = 0
    x = rng.standard_normal((1, 16, 4, 4))
    np.testing.assert_array_equal(V.resnet_block(x, W, "mid.res0", cfg, F64), x)
    # width change (16 -> 8 in the second level): the 1x1 shortcut
    W["up1.res0.conv2.w"][:] = 0
    W["up1.res0.conv2.b"][:] = 0
    y = V.resnet_block(x, W, "up1.res0", cfg, F64)
    np.testing.assert_allclose(y, V.conv2d(x, W["up1.res0.shortcut.w"], W["up1.res0.shortcut.b"]), rtol=1e-12)
    # and with the second conv on, the block differs from its skip path
    W2 = {k: v.astype(F64) for k, v in V.VAEWeights.seeded(cfg, seed=7).items()}
    assert np.abs(V.resnet_block(x, W2, "mid.res0", cfg, F64) - x).max() > 1e-3


def test_weight_list_structure_and_decode_shape():
    cfg = V.VAE_FULL
    specs = V.vae_weight_specs(cfg)
    names = [n for n, _, _ in specs]
    assert len(names) == len(set(names))
    # three ResNet blocks per level, upsampling between levels only, shortcuts where the width changes
    assert sum(n.endswith(".conv1.w") for n in names) == 2 + 4 * 3
    assert [n for n in names if n.endswith("upsample.w")] == ["up0.upsample.w", "up1.upsample.w", "up2.upsample.w"]
    assert [n for n in names if "shortcut.w" in n] == ["up2.res0.shortcut.w", "up3.res0.shortcut.w"]
    shapes = dict((n, s) for n, s, _ in specs)
    assert shapes["conv_in.w"] == (512, 4, 3, 3) and shapes["conv_out.w"] == (3, 128, 3, 3)
    assert shapes["up2.res0.conv1.w"] == (256, 512, 3, 3) and shapes["up3.res0.shortcut.w"] == (128, 256)
    small = _small_cfg()
    W = V.VAEWeights.seeded(small, seed=9)
    z = np.random.default_rng(10).standard_normal((2, 4, 3, 5)).astype(np.float32)
    out = V.decode(small, W, z)
    assert out.shape == (2, 3, 6, 10)                    # two levels: one 2x upsampling


def test_decode_scales_latents_by_the_scaling_factor():
    """Only z / scaling_factor enters: decoding z with factor s equals decoding z * t
    with factor s * t."""
    cfg = _small_cfg()
    W = V.VAEWeights.seeded(cfg, seed=11)
    W = {k: v.astype(F64) for k, v in W.items()}
    z = np.random.default_rng(12).standard_normal((1, 4, 4, 4))
    a = V.decode(cfg, W, z, F64)
    b = V.decode(replace(cfg, scaling_factor=cfg.scaling_factor * 4.0), W, z * 4.0, F64)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_decode_fp32_against_fp64():
    cfg = replace(V.VAE_FULL, block_out_channels=(32, 64), layers_per_block=1)
    W = V.VAEWeights.seeded(cfg, seed=13)
    z = np.random.default_rng(14).standard_normal((1, 4, 6, 6)).astype(np.float32)
    a = V.decode(cfg, W, z, np.float32)
    b = V.decode(cfg, W, z, F64)
    assert np.abs(a - b).max() / np.abs(b).max() < 1e-5


def test_upsampling_precedes_its_convolution():
    """The level's upsampling is nearest-neighbour 2x followed by the 3x3 conv. With
    the left-difference kernel y[i, j] = x[i, j] - x[i, j - 1], every odd output
    column differences two copies of one input pixel, so it is exactly the bias
    (convolving first and then upsampling would not give this)."""
    cfg = _small_cfg()
    W = {k: v.astype(F64) for k, v in V.VAEWeights.seeded(cfg, seed=15).items()}
    w = np.zeros_like(W["up0.upsample.w"])
    C = w.shape[0]
    for c in range(C):
        w[c, c, 1, 1] = 1.0
        w[c, c, 1, 0] = -1.0
    W["up0.upsample.w"] = w
    got = {}
    z = np.random.default_rng(16).standard_normal((1, 4, 3, 4))
    V.decode(cfg, W, z, F64, taps=lambda name, x: got.__setitem__(name, x))
    up = got["up0"][0]                                    # [C, 6, 8]
    assert up.shape == (C, 6, 8)
    np.testing.assert_allclose(up[:, :, 1::2], np.broadcast_to(W["up0.upsample.b"][:, None, None], up[:, :, 1::2].shape),
                               rtol=0, atol=1e-12)
    assert np.abs(up[:, :, 2::2] - W["up0.upsample.b"][:, None, None]).max() > 1e-3
