"""Pins for the CPU oracle: closed forms, invariants, brute force and printed values.

Each test checks the oracle against something other than itself, chosen so that
a dropped term, a wrong sign or index, or a transposed operand fails at least one
of them. Page tags: [PIPE], [TRANS], [DEEP] (see oracle/__init__.py).
"""
import json
import math
import os
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs
from oracle import spec, transformer as T

GOLD = os.path.join(os.path.dirname(__file__), "golden")
F64 = np.float64


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- config / sizes

def test_printed_config_and_inner_dim():
    g = _gold("auraflow_config.json")
    c = oracle.FULL
    d = g["default"]
    assert (c.patch_size, c.in_channels, c.out_channels) == (d["patch_size"], d["in_channels"], d["out_channels"])
    assert (c.num_mmdit_layers, c.num_single_dit_layers) == (d["num_mmdit_layers"], d["num_single_dit_layers"])
    assert (c.num_attention_heads, c.attention_head_dim) == (d["num_attention_heads"], d["attention_head_dim"])
    assert (c.joint_attention_dim, c.caption_projection_dim) == (d["joint_attention_dim"], d["caption_projection_dim"])
    assert c.inner_dim == g["inner_dim"] == 3072
    t = g["tiny_printed"]
    assert (oracle.TINY.num_attention_heads, oracle.TINY.attention_head_dim) == (t["num_attention_heads"], t["attention_head_dim"])
    assert oracle.FULL.ffn_dim == g["ffn_dim_full_derived"]
    assert oracle.TINY.ffn_dim == g["ffn_dim_tiny_derived"]


def test_find_multiple_brute_force():
    for k in (1, 7, 256):
        for n in range(1, 1200):
            m = next(x for x in range(k, n + 2 * k, k) if x >= n)
            assert oracle.find_multiple(n, k) == m


def test_ffn_int_forms_agree():
    # int(2/3 * 4d) and floor(8d/3) in exact integer arithmetic give the same width.
    for dmodel in range(1, 20000):
        assert int(2 * (4 * dmodel) / 3) == (8 * dmodel) // 3


def test_parameter_count_closed_form():
    g = _gold("auraflow_config.json")
    assert oracle.count_parameters(oracle.FULL) == g["parameters_full_derived"]
    # Workload description: "about 6.8B".
    assert 6.8e9 <= oracle.count_parameters(oracle.FULL) < 6.9e9


def test_config_validation_errors():
    c = oracle.FULL
    with pytest.raises(ValueError):
        c.check(127, 128)
    with pytest.raises(ValueError):
        c.check(194, 194)            # 97 x 97 patches > 96 x 96 grid
    assert c.check(192, 192) == (96, 96)
    assert c.check(64, 128) == (32, 64)
    with pytest.raises(ValueError):
        replace(c, pos_embed_max_size=1000).pe_grid


# ----------------------------------------------------------------------------- bf16 rounding

def test_round_bf16_hand_cases():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 3 * 2 ** -8), 1 + 2 ** -7 + 2 ** -9,
                  1 + 2 ** -7 + 2 ** -8 + 2 ** -10, 0.0, -0.0], np.float32)
    want = np.array([1.0, 1.0, 1 + 2 ** -6, -(1 + 2 ** -6), 1 + 2 ** -7, 1 + 2 ** -6, 0.0, -0.0], np.float32)
    np.testing.assert_array_equal(oracle.round_bf16(x), want)


def test_round_bf16_matches_library_cast():
    x = seeded_inputs.normal(99, 0, (4096,), 3.0)
    x = np.concatenate([x, x * 1e-30, x * 1e30])
    lib = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(oracle.round_bf16(x), lib)


# ----------------------------------------------------------------------------- PE centre crop

def test_pe_crop_brute_force_all_small_grids():
    for G in range(1, 9):
        grid = np.arange(G * G).reshape(G, G)
        for h in range(1, G + 1):
            for w in range(1, G + 1):
                r0, c0 = (G - h) // 2, (G - w) // 2
                np.testing.assert_array_equal(T.pe_crop_indices(G, h, w),
                                              grid[r0:r0 + h, c0:c0 + w].ravel())


def test_pe_crop_hand_cases():
    assert list(T.pe_crop_indices(4, 2, 2)) == [5, 6, 9, 10]
    assert list(T.pe_crop_indices(5, 2, 2)) == [6, 7, 11, 12]
    idx = T.pe_crop_indices(96, 64, 64)
    assert idx[0] == 16 * 96 + 16 and idx[-1] == 79 * 96 + 79
    assert list(T.pe_crop_indices(96, 96, 96)) == list(range(96 * 96))
    with pytest.raises(ValueError):
        T.pe_crop_indices(4, 5, 1)


# ----------------------------------------------------------------------------- timestep features

def test_timestep_features_closed_forms():
    c = oracle.FULL
    e = T.timestep_embedding(np.array([0.0, 0.25, 0.5]), c, F64)
    assert e.shape == (3, 256)
    np.testing.assert_array_equal(e[0, :128], 1.0)         # cos(0)
    np.testing.assert_array_equal(e[0, 128:], 0.0)         # sin(0)
    for r, tau in ((1, 0.25), (2, 0.5)):
        u = 1000.0 * tau
        assert math.isclose(e[r, 0], math.cos(u), abs_tol=1e-12)          # f_0 = 1
        assert math.isclose(e[r, 128], math.sin(u), abs_tol=1e-12)
        assert math.isclose(e[r, 64], math.cos(u * 0.01), abs_tol=1e-12)  # f_64 = 10000^-0.5
        assert math.isclose(e[r, 128 + 64], math.sin(u * 0.01), abs_tol=1e-12)
        # Unit circle per frequency.
        np.testing.assert_allclose(e[r, :128] ** 2 + e[r, 128:] ** 2, 1.0, atol=1e-12)


def test_timestep_mlp_brute_force():
    rng = np.random.default_rng(5)
    e = rng.standard_normal((2, 6))
    w1, b1 = rng.standard_normal((3, 6)), rng.standard_normal(3)
    w2, b2 = rng.standard_normal((4, 3)), rng.standard_normal(4)
    got = T.timestep_mlp(e, w1, b1, w2, b2)
    for b in range(2):
        hid = []
        for i in range(3):
            s = b1[i] + sum(w1[i, k] * e[b, k] for k in range(6))
            hid.append(s / (1 + math.exp(-s)))
        for o in range(4):
            want = b2[o] + sum(w2[o, i] * hid[i] for i in range(3))
            assert math.isclose(got[b, o], want, rel_tol=1e-12, abs_tol=1e-12)


# ----------------------------------------------------------------------------- LN / modulation

def test_layer_norm_hand_case():
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    got = T.layer_norm(x, 1e-6)
    want = (np.array([1.0, 2.0, 3.0, 4.0]) - 2.5) / math.sqrt(1.25 + 1e-6)
    np.testing.assert_allclose(got[0], want, rtol=0, atol=1e-15)


def test_layer_norm_invariants():
    x = np.random.default_rng(0).standard_normal((5, 7, 33)) * 3 + 2
    y = T.layer_norm(x, 1e-6)
    np.testing.assert_allclose(y.mean(-1), 0, atol=1e-13)
    var = x.var(-1)
    np.testing.assert_allclose((y * y).mean(-1), var / (var + 1e-6), rtol=1e-12)
    # Shift invariance and scale invariance (up to eps).
    np.testing.assert_allclose(T.layer_norm(x + 10, 1e-6), y, atol=1e-11)


def test_modulate_forms():
    n = np.random.default_rng(1).standard_normal((2, 3, 4))
    sh = np.random.default_rng(2).standard_normal((2, 4))
    minus_one = -np.ones((2, 4))
    out = T.modulate(n, sh, minus_one)                      # (1 + scale) = 0 -> shift only
    np.testing.assert_array_equal(out, np.broadcast_to(sh[:, None, :], n.shape))
    np.testing.assert_array_equal(T.modulate(n, np.zeros((2, 4)), np.zeros((2, 4))), n)
    np.testing.assert_allclose(T.modulate(n, np.zeros((2, 4)), np.ones((2, 4))), 2 * n)


# ----------------------------------------------------------------------------- attention

def test_attention_explicit_softmax_small():
    rng = np.random.default_rng(3)
    B, H, S, hd = 2, 2, 5, 3
    q, k, v = (rng.standard_normal((B, H, S, hd)) for _ in range(3))
    valid = np.array([[1, 0, 1, 1, 0], [1, 1, 1, 1, 1]], np.uint8)
    scale = 0.37
    got = T.attention(q, k, v, valid, scale)
    for b in range(B):
        for h in range(H):
            for i in range(S):
                logits = [sum(q[b, h, i, t] * k[b, h, j, t] for t in range(hd)) * scale if valid[b, j] else None
                          for j in range(S)]
                m = max(l for l in logits if l is not None)
                w = [math.exp(l - m) if l is not None else 0.0 for l in logits]
                z = sum(w)
                for t in range(hd):
                    want = sum(w[j] * v[b, h, j, t] for j in range(S)) / z
                    assert math.isclose(got[b, h, i, t], want, rel_tol=1e-12, abs_tol=1e-12)


def test_attention_uniform_and_single_key():
    rng = np.random.default_rng(4)
    q = np.zeros((1, 1, 3, 4))
    k, v = rng.standard_normal((1, 1, 6, 4)), rng.standard_normal((1, 1, 6, 4))
    valid = np.array([[1, 1, 0, 1, 0, 1]], np.uint8)
    got = T.attention(q, k, v, valid, 0.5)
    want = v[0, 0][valid[0] == 1].mean(0)
    np.testing.assert_allclose(got[0, 0], np.broadcast_to(want, (3, 4)), atol=1e-15)
    one = np.array([[0, 0, 0, 1, 0, 0]], np.uint8)
    q2 = rng.standard_normal((1, 1, 3, 4))
    np.testing.assert_array_equal(T.attention(q2, k, v, one, 0.5)[0, 0], np.broadcast_to(v[0, 0, 3], (3, 4)))


def test_attention_permutations_and_masked_values():
    rng = np.random.default_rng(6)
    q, k, v = (rng.standard_normal((1, 2, 7, 4)) for _ in range(3))
    valid = np.array([[1, 1, 1, 0, 1, 0, 1]], np.uint8)
    base = T.attention(q, k, v, valid, 0.5)
    pq = rng.permutation(7)
    np.testing.assert_allclose(T.attention(q[:, :, pq], k, v, valid, 0.5), base[:, :, pq], atol=1e-14)
    pk = rng.permutation(7)
    np.testing.assert_allclose(T.attention(q, k[:, :, pk], v[:, :, pk], valid[:, pk], 0.5), base, atol=1e-14)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, [3, 5]] = 1e3
    v2[:, :, [3, 5]] = -7e4
    np.testing.assert_array_equal(T.attention(q, k2, v2, valid, 0.5), base)


# ----------------------------------------------------------------------------- FFN

def test_ffn_silu_gate_order():
    rng = np.random.default_rng(7)
    n = rng.standard_normal((1, 3, 4))
    a = 1.7
    eye = np.eye(4)
    got = T.feed_forward(n, a * eye, eye, eye)
    want = (a * n) / (1 + np.exp(-a * n)) * n
    np.testing.assert_allclose(got, want, rtol=1e-14)
    swapped = T.feed_forward(n, eye, a * eye, eye)          # silu on the other branch differs
    assert not np.allclose(swapped, got)
    # W3 orientation: a permutation matrix moves features.
    P = np.eye(4)[[2, 0, 3, 1]]
    np.testing.assert_allclose(T.feed_forward(n, a * eye, eye, P), want[..., [2, 0, 3, 1]], rtol=1e-14)


# ----------------------------------------------------------------------------- blocks

def _tiny_cfg(d_heads=2, hd=2):
    return replace(oracle.TINY, num_attention_heads=d_heads, attention_head_dim=hd,
                   caption_projection_dim=d_heads * hd, joint_attention_dim=3)


def _rand_block(rng, d, F, gates=True):
    blk = {"ada": rng.standard_normal((6 * d, d)) * 0.5,
           "wq": rng.standard_normal((d, d)), "wk": rng.standard_normal((d, d)),
           "wv": rng.standard_normal((d, d)), "wo": rng.standard_normal((d, d)) * 0.5,
           "ff1": rng.standard_normal((F, d)) * 0.3, "ff2": rng.standard_normal((F, d)) * 0.3,
           "ff3": rng.standard_normal((d, F)) * 0.1}
    if not gates:
        blk["ada"][2 * d:3 * d] = 0
        blk["ada"][5 * d:6 * d] = 0
    return blk


def _brute_single_block(cfg, blk, temb, x, valid):
    """Element-by-element loops of the single DiT block (float64, tiny sizes)."""
    B, S, d = x.shape
    H, hd, F, eps = cfg.num_attention_heads, cfg.attention_head_dim, cfg.ffn_dim, cfg.ln_eps
    silu = lambda z: z / (1 + math.exp(-z))

    def ln(vec):
        mu = sum(vec) / len(vec)
        var = sum((t - mu) ** 2 for t in vec) / len(vec)
        return [(t - mu) / math.sqrt(var + eps) for t in vec]

    out = np.array(x, dtype=F64)
    for b in range(B):
        st = [silu(t) for t in temb[b]]
        mod = [sum(blk["ada"][r, c] * st[c] for c in range(d)) for r in range(6 * d)]
        sh1, sc1, g1 = mod[0:d], mod[d:2 * d], mod[2 * d:3 * d]
        sh2, sc2, g2 = mod[3 * d:4 * d], mod[4 * d:5 * d], mod[5 * d:6 * d]
        n = []
        for s in range(S):
            l = ln(list(x[b, s]))
            n.append([l[c] * (1 + sc1[c]) + sh1[c] for c in range(d)])
        proj = lambda Wm, row: [sum(Wm[o, c] * row[c] for c in range(Wm.shape[1])) for o in range(Wm.shape[0])]
        q = [proj(blk["wq"], n[s]) for s in range(S)]
        k = [proj(blk["wk"], n[s]) for s in range(S)]
        v = [proj(blk["wv"], n[s]) for s in range(S)]
        o = [[0.0] * d for _ in range(S)]
        for h in range(H):
            sl = slice(h * hd, (h + 1) * hd)
            qh = [ln(q[s][sl]) for s in range(S)]
            kh = [ln(k[s][sl]) for s in range(S)]
            for i in range(S):
                logits = [sum(qh[i][t] * kh[j][t] for t in range(hd)) / math.sqrt(hd) for j in range(S)]
                m = max(logits[j] for j in range(S) if valid[b, j])
                w = [math.exp(logits[j] - m) if valid[b, j] else 0.0 for j in range(S)]
                z = sum(w)
                for t in range(hd):
                    o[i][h * hd + t] = sum(w[j] * v[j][h * hd + t] for j in range(S)) / z
        x1 = []
        for s in range(S):
            a = proj(blk["wo"], o[s])
            x1.append([x[b, s, c] + g1[c] * a[c] for c in range(d)])
        for s in range(S):
            l = ln(x1[s])
            n2 = [l[c] * (1 + sc2[c]) + sh2[c] for c in range(d)]
            h1 = proj(blk["ff1"], n2)
            h2 = proj(blk["ff2"], n2)
            hh = [silu(h1[f]) * h2[f] for f in range(F)]
            y = proj(blk["ff3"], hh)
            for c in range(d):
                out[b, s, c] = x1[s][c] + g2[c] * y[c]
    return out


def test_single_block_brute_force():
    cfg = _tiny_cfg(2, 2)
    d, F = cfg.inner_dim, cfg.ffn_dim
    rng = np.random.default_rng(8)
    blk = _rand_block(rng, d, F)
    temb = rng.standard_normal((2, d))
    x = rng.standard_normal((2, 5, d))
    valid = np.array([[1, 1, 0, 1, 1], [1, 0, 0, 1, 1]], np.uint8)
    got = T.single_block(cfg, blk, temb, x, valid, F64)
    np.testing.assert_allclose(got, _brute_single_block(cfg, blk, temb, x, valid), rtol=1e-10, atol=1e-10)


def test_zero_gates_make_blocks_identity():
    cfg = _tiny_cfg(2, 4)
    d, F = cfg.inner_dim, cfg.ffn_dim
    rng = np.random.default_rng(9)
    temb = rng.standard_normal((2, d))
    x = rng.standard_normal((2, 6, d)) * 3
    valid = np.ones((2, 6), np.uint8)
    blk = _rand_block(rng, d, F, gates=False)
    np.testing.assert_array_equal(T.single_block(cfg, blk, temb, x, valid, F64), x)
    bi, bt = _rand_block(rng, d, F, gates=False), _rand_block(rng, d, F, gates=False)
    xt, xi = x[:, :2], x[:, 2:]
    ot, oi = T.joint_block(cfg, bi, bt, temb, xt, xi, valid, F64)
    np.testing.assert_array_equal(ot, xt)
    np.testing.assert_array_equal(oi, xi)
    # With gates on, the block is not the identity (the test above has teeth).
    blk_on = _rand_block(rng, d, F, gates=True)
    assert not np.allclose(T.single_block(cfg, blk_on, temb, x, valid, F64), x)


def test_joint_block_streams_use_their_own_weights():
    cfg = _tiny_cfg(2, 4)
    d, F = cfg.inner_dim, cfg.ffn_dim
    rng = np.random.default_rng(10)
    temb = rng.standard_normal((1, d))
    xt, xi = rng.standard_normal((1, 3, d)), rng.standard_normal((1, 4, d))
    valid = np.ones((1, 7), np.uint8)
    bi_off, bt_on = _rand_block(rng, d, F, gates=False), _rand_block(rng, d, F, gates=True)
    ot, oi = T.joint_block(cfg, bi_off, bt_on, temb, xt, xi, valid, F64)
    np.testing.assert_array_equal(oi, xi)                    # image gates zero -> image unchanged
    assert not np.allclose(ot, xt)
    ot2, oi2 = T.joint_block(cfg, bt_on, bi_off, temb, xt, xi, valid, F64)
    np.testing.assert_array_equal(ot2, xt)
    assert not np.allclose(oi2, xi)


def test_joint_block_with_shared_weights_equals_single_block():
    cfg = _tiny_cfg(2, 4)
    d, F = cfg.inner_dim, cfg.ffn_dim
    rng = np.random.default_rng(11)
    blk = _rand_block(rng, d, F)
    temb = rng.standard_normal((2, d))
    x = rng.standard_normal((2, 7, d))
    valid = np.array([[1, 0, 1, 1, 1, 1, 1], [1, 1, 1, 0, 1, 1, 1]], np.uint8)
    ot, oi = T.joint_block(cfg, blk, blk, temb, x[:, :3], x[:, 3:], valid, F64)
    np.testing.assert_allclose(np.concatenate([ot, oi], 1), T.single_block(cfg, blk, temb, x, valid, F64),
                               rtol=1e-12, atol=1e-12)


def test_pre_final_scale_shift_order():
    rng = np.random.default_rng(12)
    d = 4
    x = rng.standard_normal((1, 3, d))
    scale, shift = np.array([0.5, -1.0, 2.0, 0.0]), np.array([1.0, 2.0, 3.0, 4.0])
    t0 = 1.3
    temb = np.array([[t0, 0, 0, 0]])                         # SiLU(temb) = [silu(t0), 0, 0, 0]
    ada = np.zeros((2 * d, d))
    ada[:, 0] = np.concatenate([scale, shift]) / (t0 / (1 + math.exp(-t0)))
    got = T.pre_final(temb, x, ada)
    np.testing.assert_allclose(got, x * (1 + scale) + shift, rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------------------- whole model

def _identity_model_weights(cfg, rng, pe=None):
    """d = C*p*p; patch projection = I, no bias; every adaLN matrix zero; proj_out maps (c,py,px)->(py,px,c)."""
    d, p, C = cfg.inner_dim, cfg.patch_size, cfg.in_channels
    tensors = {}
    for name, shape, std in oracle.weight_specs(cfg):
        tensors[name] = (rng.standard_normal(shape) * std).astype(np.float32)
    for name in tensors:
        if name.endswith("ada"):
            tensors[name][:] = 0
    tensors["pe_w"] = np.eye(d, dtype=np.float32)
    tensors["pe_b"] = np.zeros(d, np.float32)
    tensors["pos_embed"] = np.zeros_like(tensors["pos_embed"]) if pe is None else pe
    P = np.zeros((d, d), np.float32)
    for c in range(C):
        for py in range(p):
            for px in range(p):
                P[(py * p + px) * C + c, c * p * p + py * p + px] = 1
    tensors["proj_out"] = P
    return tensors


def test_identity_model_returns_latents():
    cfg = replace(oracle.TINY, num_attention_heads=2, attention_head_dim=8, caption_projection_dim=16)
    rng = np.random.default_rng(13)
    W = oracle.Weights.from_dict(cfg, _identity_model_weights(cfg, rng))
    lat = rng.standard_normal((2, 4, 6, 10)).astype(np.float32)
    text = rng.standard_normal((2, 5, cfg.joint_attention_dim)).astype(np.float32)
    out = oracle.forward(cfg, W, lat, np.array([0.3, 0.9]), text, None, F64)
    np.testing.assert_array_equal(out, lat)


def test_identity_model_routes_the_patch_bias_to_its_pixels():
    """Patch embedding has a bias ([TRANS] 核心子模块架构, Patch Embedding: the
    projection is an nn.Linear written without bias=False). In the identity model
    a bias b on the patch features reaches the output through the (c, py, px) ->
    (py, px, c) permutation of proj_out, so pixel (c, y, x) gains
    b[c p^2 + (y mod p) p + (x mod p)]; written out element by element."""
    cfg = replace(oracle.TINY, num_attention_heads=2, attention_head_dim=8, caption_projection_dim=16)
    rng = np.random.default_rng(15)
    tensors = _identity_model_weights(cfg, rng)
    d, p = cfg.inner_dim, cfg.patch_size
    bias = (np.arange(d) * 0.25 - 1.5).astype(np.float32)     # distinct, exactly representable
    tensors["pe_b"] = bias
    W = oracle.Weights.from_dict(cfg, tensors)
    H_, W_ = 6, 10
    lat = rng.standard_normal((2, 4, H_, W_)).astype(np.float32)
    text = rng.standard_normal((2, 3, cfg.joint_attention_dim)).astype(np.float32)
    out = oracle.forward(cfg, W, lat, np.array([0.2, 0.7]), text, None, F64)
    for b in range(2):
        for c in range(4):
            for y in range(H_):
                for x in range(W_):
                    want = float(lat[b, c, y, x]) + float(bias[c * p * p + (y % p) * p + (x % p)])
                    assert out[b, c, y, x] == want, (b, c, y, x)


def test_identity_model_places_the_cropped_position_table():
    cfg = replace(oracle.TINY, num_attention_heads=2, attention_head_dim=8, caption_projection_dim=16)
    rng = np.random.default_rng(14)
    G, d = cfg.pe_grid, cfg.inner_dim
    pe = (np.arange(G * G)[:, None] * 1000 + np.arange(d)[None, :]).astype(np.float32)
    tensors = _identity_model_weights(cfg, rng, pe=pe)
    tensors["pe_w"][:] = 0
    W = oracle.Weights.from_dict(cfg, tensors)
    H_, W_ = 6, 10                                           # 3 x 5 patch grid in an 8 x 8 table
    lat = rng.standard_normal((1, 4, H_, W_)).astype(np.float32)
    out = oracle.forward(cfg, W, lat, np.array([0.5]), rng.standard_normal((1, 2, 32)).astype(np.float32),
                         None, F64)
    r0, c0 = (8 - 3) // 2, (8 - 5) // 2                      # 2, 1
    for c in range(4):
        for y in range(H_):
            for x in range(W_):
                i, py, j, px = y // 2, y % 2, x // 2, x % 2
                g = (r0 + i) * G + (c0 + j)
                assert out[0, c, y, x] == g * 1000 + (c * 4 + py * 2 + px)


def _tiny_inputs(cfg, B=1, T_=8, H=16, W_=16, lengths=None):
    lat = seeded_inputs.latents(B, cfg.in_channels, H, W_)
    text = seeded_inputs.text_embeddings(B, T_, cfg.joint_attention_dim)
    mask = None if lengths is None else seeded_inputs.length_mask(np.array(lengths), T_)
    return lat, text, mask


def test_fp32_oracle_against_fp64_self_check():
    cfg = oracle.TINY
    W = oracle.Weights.seeded(cfg)
    lat, text, mask = _tiny_inputs(cfg, B=2, lengths=[8, 5])
    tau = np.array([0.5, 0.137])
    o32 = oracle.forward(cfg, W, lat, tau, text, mask, np.float32)
    o64 = oracle.forward(cfg, W, lat, tau, text, mask, F64)
    rel = np.abs(o32 - o64).max() / np.abs(o64).max()
    assert rel < 2e-6, rel


def test_masked_text_does_not_change_output():
    cfg = oracle.TINY
    W = oracle.Weights.seeded(cfg)
    lat, text, mask = _tiny_inputs(cfg, B=2, lengths=[3, 6])
    tau = np.array([0.5, 0.5])
    base = oracle.forward(cfg, W, lat, tau, text, mask, np.float32)
    text2 = text.copy()
    text2[0, 3:] = 123.0
    text2[1, 6:] = -55.0
    np.testing.assert_array_equal(oracle.forward(cfg, W, lat, tau, text2, mask, np.float32), base)
    # All-ones mask equals no mask.
    ones = np.ones((2, 8), np.uint8)
    np.testing.assert_array_equal(oracle.forward(cfg, W, lat, tau, text, ones, np.float32),
                                  oracle.forward(cfg, W, lat, tau, text, None, np.float32))
    # And a valid token does matter (the mask test has teeth).
    text3 = text.copy()
    text3[0, 0] += 1.0
    assert not np.array_equal(oracle.forward(cfg, W, lat, tau, text3, mask, np.float32), base)


def test_batch_rows_are_independent():
    cfg = oracle.TINY
    W = oracle.Weights.seeded(cfg)
    lat, text, mask = _tiny_inputs(cfg, B=2, lengths=[8, 4])
    tau = np.array([0.25, 0.75])
    both = oracle.forward(cfg, W, lat, tau, text, mask, F64)
    one = oracle.forward(cfg, W, lat[1:], tau[1:], text[1:], mask[1:], F64)
    np.testing.assert_allclose(both[1:], one, rtol=1e-13, atol=1e-13)


def test_taps_cover_every_block_and_end_at_output():
    cfg = oracle.TINY
    W = oracle.Weights.seeded(cfg)
    lat, text, _ = _tiny_inputs(cfg)
    seen = []
    oracle.forward(cfg, W, lat, np.array([0.5]), text, None, F64,
                   taps=lambda i, xt, xi: seen.append((i, xt.shape, xi.shape)))
    assert seen == [(0, (1, 16, 32), (1, 64, 32)), (1, (1, 16, 32), (1, 64, 32))]


# ----------------------------------------------------------------------------- sampling

def test_sigma_schedule_golden_and_shape():
    g = _gold("sigma_schedule.json")
    s = g["shift"]
    sig = oracle.sigma_schedule(4, s)                       # u = 1, .75, .5, .25, 0
    assert sig[0] == g["sigma_at_u"]["1.0"] and sig[-1] == g["sigma_at_u"]["0.0"]
    assert math.isclose(sig[2], g["sigma_at_u"]["0.5"], rel_tol=1e-15)
    assert math.isclose(sig[3], g["sigma_at_u"]["0.25"], rel_tol=1e-15)
    sig25 = oracle.sigma_schedule(25, s)
    assert len(sig25) == 26 and np.all(np.diff(sig25) < 0)
    np.testing.assert_allclose(oracle.sigma_schedule(10, 1.0), 1 - np.arange(11) / 10, atol=1e-15)


def test_cfg_combine_forms():
    vu = np.full((2, 1, 2, 2), 1.0)
    vc = np.full((2, 1, 2, 2), 3.0)
    v = np.concatenate([vu, vc])
    np.testing.assert_array_equal(oracle.cfg_combine(v, 3.5), np.full((2, 1, 2, 2), 8.0))
    rng = np.random.default_rng(15)
    v = rng.standard_normal((4, 2, 3, 3))
    np.testing.assert_array_equal(oracle.cfg_combine(v, 1.0), v)          # off at s <= 1
    np.testing.assert_array_equal(oracle.cfg_combine(v, 0.0), v)
    for s in (1.5, 3.5, 7.0):
        np.testing.assert_allclose(oracle.cfg_combine(v, s), (1 - s) * v[:2] + s * v[2:], rtol=1e-12, atol=1e-12)


def test_euler_point_mass_lands_on_target():
    rng = np.random.default_rng(16)
    x0 = rng.standard_normal((1, 4, 8, 8))
    x = rng.standard_normal((1, 4, 8, 8))
    sig = oracle.sigma_schedule(25, 1.73)
    for i in range(25):
        v = (x - x0) / sig[i]
        x = oracle.euler_step(x, v, sig[i], sig[i + 1])
    np.testing.assert_allclose(x, x0, atol=1e-12)
    y = rng.standard_normal((2, 4, 3, 3))
    np.testing.assert_array_equal(oracle.euler_step(y, rng.standard_normal(y.shape), 0.4, 0.4), y)


def test_cfg_euler_step_composition():
    rng = np.random.default_rng(17)
    x = rng.standard_normal((2, 4, 4, 4))
    v = rng.standard_normal((4, 4, 4, 4))
    got = oracle.cfg_euler_step(x, v, 0.8, 0.6, 3.5)
    want = x + (0.6 - 0.8) * (v[:2] + 3.5 * (v[2:] - v[:2]))
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-14)
