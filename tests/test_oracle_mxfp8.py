"""Pins for the oracle's MXFP8 quantization (the block format of the FP8 GEMM path).

Checked against definitions written independently of oracle/numerics.py: the
E4M3 value table decoded from its bit fields, nearest-value search over that
table (ties to the even code), the block scale from math.frexp, and hand cases.
"""
import math

import numpy as np

import oracle
from oracle import transformer as T


def _e4m3_table():
    """(code, value) for every finite OCP E4M3 code, decoded from sign/exponent/mantissa bits."""
    out = []
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue                                    # NaN
        v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        out.append((c, -v if s else v))
    return out


TABLE = _e4m3_table()


def _nearest(x):
    best, bd = None, None
    for c, v in TABLE:
        d = abs(v - x)
        if bd is None or d < bd or (d == bd and c % 2 == 0 and best[0] % 2 == 1):
            best, bd = (c, v), d
    return best[1]


def test_e4m3_table_facts():
    vals = sorted(v for _, v in TABLE)
    assert max(vals) == 448.0 and min(vals) == -448.0
    pos = sorted(set(v for v in vals if v > 0))
    assert pos[0] == 2.0 ** -9                         # smallest subnormal
    assert 2.0 ** -6 in pos and 1.0 in pos and 1.125 in pos
    assert len(set(vals)) == 253                       # 254 finite codes, +0 and -0 equal


def test_round_e4m3_is_nearest_value_ties_to_even():
    rng = np.random.default_rng(0)
    pos = np.array(sorted(set(v for _, v in TABLE if v >= 0)))
    mids = (pos[1:] + pos[:-1]) / 2
    xs = np.concatenate([pos, -pos, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 500),
                         rng.uniform(-448, 448, 500), rng.uniform(-1, 1, 500), rng.uniform(-0.03, 0.03, 500)])
    xs = xs.astype(np.float32)
    got = oracle.round_e4m3(xs)
    want = np.array([_nearest(float(x)) for x in xs], np.float32)
    np.testing.assert_array_equal(np.abs(got), np.abs(want))
    np.testing.assert_array_equal(got[want != 0], want[want != 0])
    # hand cases: 1.0625 lies half way between 1.0 (even code) and 1.125 -> 1.0; 1.1875 -> 1.25
    np.testing.assert_array_equal(oracle.round_e4m3(np.array([1.0625, 1.1875, 300.0, 2 ** -10], np.float32)),
                                  np.array([1.0, 1.25, 288.0, 0.0], np.float32))


def _qdq_by_definition(block):
    amax = max(abs(float(v)) for v in block)
    if amax == 0:
        return [0.0] * len(block)
    e = math.frexp(amax)[1] - 1 - 8                   # floor(log2 amax) - 8
    e = max(-127, min(127, e))
    X = 2.0 ** e
    return [_nearest(max(-448.0, min(448.0, float(v) / X))) * X for v in block]


def test_mxfp8_qdq_matches_definition_per_block():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal((3, 64)) * s for s in (1e-3, 1.0, 37.0)]).astype(np.float32)
    x[0, :32] = 0.0                                    # an all-zero block
    x[1, 5] = 1e-8                                     # a tiny value next to large ones
    got = oracle.mxfp8_qdq(x)
    for r in range(x.shape[0]):
        for b in range(2):
            want = _qdq_by_definition(x[r, 32 * b:32 * b + 32])
            np.testing.assert_array_equal(got[r, 32 * b:32 * b + 32], np.array(want, np.float32))


def test_mxfp8_qdq_hand_cases_and_saturation():
    x = np.zeros((2, 32), np.float32)
    x[0, :3] = [1.0, 0.3, -0.5]       # amax 1 -> X = 2^-8: 0.3 * 256 = 76.8 -> 80 -> 0.3125
    x[1, :2] = [500.0, 1.0]           # amax 500 -> X = 1: 500 saturates to 448
    got = oracle.mxfp8_qdq(x)
    np.testing.assert_array_equal(got[0, :3], np.array([1.0, 0.3125, -0.5], np.float32))
    np.testing.assert_array_equal(got[1, :2], np.array([448.0, 1.0], np.float32))
    assert np.all(got[:, 3:] == 0)


def test_mxfp8_qdq_invariants():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((4, 96)) * 3).astype(np.float32)
    q = oracle.mxfp8_qdq(x)
    np.testing.assert_array_equal(oracle.mxfp8_qdq(q), q)                       # idempotent
    for k in (-5, 3, 20):                                                       # commutes with 2^k
        np.testing.assert_array_equal(oracle.mxfp8_qdq(x * np.float32(2.0 ** k)), q * np.float32(2.0 ** k))
    y = x.copy()
    y[:, 32:64] *= 100                                                          # blocks are independent
    q2 = oracle.mxfp8_qdq(y)
    np.testing.assert_array_equal(q2[:, :32], q[:, :32])
    np.testing.assert_array_equal(q2[:, 64:], q[:, 64:])
    # error bound: half a grid step at the block scale, for elements below the
    # saturation threshold; saturated ones become exactly +-448 X
    xb = x.reshape(4, 3, 32).astype(np.float64)
    amax = np.abs(xb).max(-1, keepdims=True)
    X = 2.0 ** (np.floor(np.log2(amax)) - 8)
    v = np.abs(xb) / X
    err = np.abs(q.reshape(4, 3, 32) - xb)
    step = 2.0 ** (np.floor(np.log2(np.maximum(v, 2 ** -6))) - 3) * X
    sat = v > 448
    assert np.all(err[~sat] <= step[~sat] / 2 + 1e-12)
    np.testing.assert_array_equal(np.abs(q.reshape(4, 3, 32))[sat], (448 * X * np.ones_like(xb))[sat])


def test_mx_forward_uses_quantized_operands_only_where_stated():
    """mx=True changes the block output by MXFP8-sized amounts; mx_block quantizes
    exactly the weights of the QKV, out-projection and FFN products."""
    cfg = oracle.TINY
    W = oracle.Weights.seeded(cfg, seed=0)
    rng = np.random.default_rng(3)
    B, T_, N = 1, 8, 64
    d = cfg.inner_dim
    temb = rng.standard_normal((B, d)).astype(np.float32)
    x = rng.standard_normal((B, cfg.num_register_tokens + T_ + N, d)).astype(np.float32)
    kv = np.ones((B, x.shape[1]), np.uint8)
    blk = {k: W["single0." + k] for k in ("ada", "wq", "wk", "wv", "wo", "ff1", "ff2", "ff3")}
    a = T.single_block(cfg, blk, temb, x, kv, np.float32, mx=False)
    b = T.single_block(cfg, blk, temb, x, kv, np.float32, mx=True)
    rel = np.abs(b - a).max() / np.abs(a - x).max()
    assert 1e-4 < rel < 0.1, rel                      # quantization is visible but small
    qb = oracle.mx_block(blk)
    assert np.array_equal(qb["ada"], blk["ada"])
    for k in ("wq", "wk", "wv", "wo", "ff1", "ff2", "ff3"):
        assert not np.array_equal(qb[k], blk[k])
        np.testing.assert_array_equal(qb[k], oracle.mxfp8_qdq(blk[k]))
    np.testing.assert_array_equal(oracle.mxfp8_qdq(qb["ff3"]), qb["ff3"])


def _torch_bf16(a):
    """bfloat16 rounding by torch's own cast (an implementation independent of
    oracle.round_bf16), returned as float32."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def _attention_bf16_by_hand(q, k, v, kv, scale):
    """softmax(q k^T scale) v with q, k, v and exp(logit) rounded by torch's bf16
    cast, normalised by the sum of the unrounded exponentials; keys with kv == 0
    left out."""
    out = np.empty_like(q)
    qb, kb, vb = _torch_bf16(q), _torch_bf16(k), _torch_bf16(v)
    for b in range(q.shape[0]):
        keep = kv[b] != 0
        for h in range(q.shape[1]):
            e = np.exp((qb[b, h] @ kb[b, h][keep].T) * scale)
            out[b, h] = (_torch_bf16(e) @ vb[b, h][keep]) / e.sum(axis=1, keepdims=True)
    return out


def test_bf16_operand_attention_hand_case():
    """One query, two kept keys and one excluded key, head dim 16, scale 1/4:
    q = 1 + 2^-10 rounds to 1 in bf16, so the logits are exactly 0 and 1; e^1 =
    2.71828 (float32) rounds to 2.71875 in bf16; v0 = 0.1 rounds to
    0.10009765625. The output is (1 * 0.10009765625 + 2.71875 * 3) / (1 + e^1):
    rounded probabilities in the numerator, unrounded ones in the normaliser."""
    hd = 16
    q = np.zeros((1, 1, 1, hd), np.float32)
    q[0, 0, 0, 0] = 1 + 2.0 ** -10
    k = np.zeros((1, 1, 3, hd), np.float32)
    k[0, 0, 1, 0] = 4.0
    k[0, 0, 2, 0] = 8.0                      # excluded below
    v = np.zeros((1, 1, 3, hd), np.float32)
    v[0, 0, :, 3] = [0.1, 3.0, 1000.0]
    kv = np.array([[1, 1, 0]], np.uint8)
    got = oracle.attention_bf16_operands(q, k, v, kv, np.float32(0.25))
    e1 = float(np.exp(np.float32(1.0)))
    want = (0.10009765625 + 2.71875 * 3.0) / (1.0 + e1)
    assert abs(e1 - math.e) < 4e-7          # float32 exp, within an ulp either way
    assert abs(float(got[0, 0, 0, 3]) - want) <= 2e-7 * want
    assert np.all(got[0, 0, 0, [0, 1, 2, 4, 15]] == 0)
    # the plain softmax differs visibly: the roundings are really there
    plain = oracle.attention(q, k, v, kv, np.float32(0.25))
    assert abs(float(plain[0, 0, 0, 3]) - want) > 1e-4


def test_bf16_operand_attention_against_torch_casts_and_plain_softmax():
    """Random ragged case: equal to the composition with torch's bf16 cast; within
    bf16's relative half-ulp bound (2^-9 per rounded operand) of the float64 plain
    attention; with q = 0 the output is the mean of the bf16-rounded values of
    the kept keys, exactly."""
    rng = np.random.default_rng(21)
    B, H, S, hd = 2, 3, 37, 16
    q, k, v = (rng.standard_normal((B, H, S, hd)).astype(np.float32) for _ in range(3))
    q, k = T.layer_norm(q, np.float32(1e-6)), T.layer_norm(k, np.float32(1e-6))
    kv = np.ones((B, S), np.uint8)
    kv[1, 20:30] = 0
    sc = np.float32(0.25)
    got = oracle.attention_bf16_operands(q, k, v, kv, sc)
    np.testing.assert_allclose(got, _attention_bf16_by_hand(q, k, v, kv, sc), rtol=0, atol=1e-6)
    exact = oracle.attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), kv, 0.25)
    err = np.abs(got - exact).max() / np.abs(v).max()
    # q, k roundings move a logit by <= 2 * 2^-9 * |q||k| * scale = 2^-8 * 4; e and v by 2^-9 each
    assert 1e-5 < err < 4 * 2.0 ** -8 + 2 * 2.0 ** -9, err
    z = oracle.attention_bf16_operands(np.zeros_like(q), k, v, kv, sc)
    vb = oracle.round_bf16(v).astype(np.float64)
    for b in range(B):
        keep = kv[b] != 0
        want = vb[b][:, keep].mean(axis=1)
        np.testing.assert_allclose(z[b, :, 0], want, rtol=1e-6, atol=1e-7)


def _single_block_by_hand(cfg, blk, temb, x, kv, quant_points):
    """A single DiT block with MXFP8 quantize-dequantize applied exactly at the
    named activation points (a subset of 'ln1', 'attn', 'ln2', 'ffh') and to the
    weights of the QKV, out-projection and FFN products, and ('bf16attn' in the
    subset) attention on bf16 operands; everything else in float32. Composed from
    the block's equations: adaLN-Zero with six vectors, LN + modulate, bias-free
    q/k/v with per-head LayerNorm, softmax attention, gated out-projection,
    LN + modulate, SiLU-gated FFN, gated residual."""
    f32 = np.float32
    qd = lambda a, point: oracle.mxfp8_qdq(a) if point in quant_points else a
    Wq = {k: oracle.mxfp8_qdq(blk[k]) for k in ("wq", "wk", "wv", "wo", "ff1", "ff2", "ff3")}
    d = cfg.inner_dim
    H, hd = cfg.num_attention_heads, cfg.attention_head_dim
    eps = f32(cfg.ln_eps)
    mod = T.silu(temb) @ blk["ada"].T
    sh1, sc1, g1, sh2, sc2, g2 = (mod[:, i * d:(i + 1) * d] for i in range(6))
    B, S, _ = x.shape
    n1 = qd(T.layer_norm(x, eps) * (1 + sc1[:, None, :]) + sh1[:, None, :], "ln1")
    heads = lambda y: y.reshape(B, S, H, hd).transpose(0, 2, 1, 3)
    q = T.layer_norm(heads(n1 @ Wq["wq"].T), eps)
    k = T.layer_norm(heads(n1 @ Wq["wk"].T), eps)
    v = heads(n1 @ Wq["wv"].T)
    attn = _attention_bf16_by_hand if "bf16attn" in quant_points else T.attention
    o = attn(q, k, v, kv, f32(1.0 / np.sqrt(hd)))
    o = qd(o.transpose(0, 2, 1, 3).reshape(B, S, d), "attn")
    x1 = x + g1[:, None, :] * (o @ Wq["wo"].T)
    n2 = qd(T.layer_norm(x1, eps) * (1 + sc2[:, None, :]) + sh2[:, None, :], "ln2")
    h = qd(T.silu(n2 @ Wq["ff1"].T) * (n2 @ Wq["ff2"].T), "ffh")
    return x1 + g2[:, None, :] * (h @ Wq["ff3"].T)


def test_mx_single_block_quantizes_exactly_the_four_activation_points():
    """single_block(mx=True) equals the block composed by hand with MXFP8 applied at
    the LN + modulate outputs (both), the attention output and the FFN hidden
    activations, and at no other activation, with attention on bf16 operands;
    dropping any one of the five changes the result, so each of them is pinned."""
    cfg = oracle.TINY
    W = oracle.Weights.seeded(cfg, seed=0)
    rng = np.random.default_rng(11)
    B, T_, N = 2, 8, 64
    d = cfg.inner_dim
    temb = rng.standard_normal((B, d)).astype(np.float32)
    x = rng.standard_normal((B, cfg.num_register_tokens + T_ + N, d)).astype(np.float32)
    kv = np.ones((B, x.shape[1]), np.uint8)
    kv[1, cfg.num_register_tokens + 5:cfg.num_register_tokens + T_] = 0
    blk = {k: W["single0." + k] for k in ("ada", "wq", "wk", "wv", "wo", "ff1", "ff2", "ff3")}
    # adaLN rows scaled up so the gates and modulations are O(1) and every branch
    # moves the residual visibly
    blk["ada"] = blk["ada"] * np.float32(20.0)
    points = ("ln1", "attn", "ln2", "ffh", "bf16attn")
    got = T.single_block(cfg, blk, temb, x, kv, np.float32, mx=True)
    want = _single_block_by_hand(cfg, blk, temb, x, kv, points)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-5 * np.abs(want).max())
    for drop in points:
        other = _single_block_by_hand(cfg, blk, temb, x, kv, tuple(p for p in points if p != drop))
        # quantization moves the block output by far more than the tolerance above
        assert np.abs(other - want).max() > 1e-3 * np.abs(want - x).max(), drop


def test_mx_joint_block_quantizes_the_same_points_per_stream():
    """A joint block whose two streams carry identical weights equals the single
    block over the concatenated sequence in mx mode as well (so the joint block
    quantizes the same four points in each stream)."""
    cfg = oracle.TINY
    W = oracle.Weights.seeded(cfg, seed=0)
    rng = np.random.default_rng(12)
    B, T_, N = 1, 8, 64
    d = cfg.inner_dim
    Nt = cfg.num_register_tokens + T_
    temb = rng.standard_normal((B, d)).astype(np.float32)
    x = rng.standard_normal((B, Nt + N, d)).astype(np.float32)
    kv = np.ones((B, x.shape[1]), np.uint8)
    blk = {k: W["single0." + k] for k in ("ada", "wq", "wk", "wv", "wo", "ff1", "ff2", "ff3")}
    blk["ada"] = blk["ada"] * np.float32(20.0)
    xt, xi = T.joint_block(cfg, blk, blk, temb, x[:, :Nt], x[:, Nt:], kv, np.float32, mx=True)
    want = _single_block_by_hand(cfg, blk, temb, x, kv, ("ln1", "attn", "ln2", "ffh", "bf16attn"))
    got = np.concatenate([xt, xi], 1)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-5 * np.abs(want).max())
