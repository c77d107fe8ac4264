"""Pins for the UMT5 text-encoder oracle (oracle/umt5.py), CPU only.

Each check fixes the oracle against something other than itself: hand values of
the bucket rule worked out from its definition, a closed form of the bucket for
the 32-bucket / distance-128 configuration (bit length of n^2), brute-force loops
for attention, exact identities of the norm and of the tanh GELU, and composition
invariants of the whole encoder (zeroed output projections, masked-token and
position-shift invariance).
"""
import math

import numpy as np
import pytest

import seeded_inputs
from oracle import umt5 as U


# ----------------------------------------------------------------------------- relative-position buckets

def test_bucket_hand_values():
    # 16 buckets per sign; |rel| < 8 exact; then 8 + floor(2 log2(|rel| / 8)) up to 15.
    # 2 log2(n / 8) crosses 1 at n = 8 sqrt(2) = 11.3, 2 at 16, 3 at 22.6, 4 at 32, 6 at 64, 8 at 128.
    cases = {0: 0, -1: 1, -7: 7, 1: 17, 7: 23, -8: 8, 8: 24, -11: 8, -12: 9, -16: 10, 16: 26,
             -22: 10, -23: 11, -32: 12, -63: 13, -64: 14, -127: 15, -128: 15, 128: 31, -5000: 15, 5000: 31}
    rel = np.array(list(cases))
    got = U.relative_bucket(rel, 32, 128)
    assert got.tolist() == list(cases.values())


def test_bucket_closed_form_for_32_buckets_distance_128():
    # For 16 buckets per sign, 8 exact and max distance 128 (ratio 16 = 2^4 over 8 steps):
    # floor(8 log(n/8) / log 16) = floor(log2(n^2 / 64)) = bit_length(n^2) - 1 - 6.
    n = np.arange(8, 3000)
    closed = np.minimum(8 + np.array([(int(v) * int(v)).bit_length() - 7 for v in n]), 15)
    assert U.relative_bucket(-n, 32, 128).tolist() == closed.tolist()
    assert U.relative_bucket(n, 32, 128).tolist() == (16 + closed).tolist()


def test_bucket_float_formula_agrees_away_from_integer_points():
    # The textbook float formula gives the same buckets except where the real value
    # is an integer (n = 16, 32, 64, 128), where rounding may land either side.
    n = np.arange(8, 1000)
    flt = 8 + np.floor(np.log(n / 8.0) / np.log(16.0) * 8).astype(int)
    flt = np.minimum(flt, 15)
    exact = U.relative_bucket(-n, 32, 128)
    diff = n[flt != exact]
    assert set(diff.tolist()) <= {16, 32, 64, 128}


def test_bucket_symmetry_and_monotone():
    n = np.arange(0, 600)
    neg, pos = U.relative_bucket(-n), U.relative_bucket(n)
    assert (pos[1:] == 16 + neg[1:]).all() and pos[0] == 0
    assert (np.diff(neg) >= 0).all() and neg.max() == 15


# ----------------------------------------------------------------------------- elementwise pieces

def test_rms_norm_closed_forms():
    w = np.array([1.0, 2.0, -3.0, 0.5])
    # a constant row c normalises to c / sqrt(c^2 + eps) per element
    for c in (3.0, -0.25):
        x = np.full((1, 4), c)
        np.testing.assert_allclose(U.rms_norm(x, w, 1e-6)[0], w * c / math.sqrt(c * c + 1e-6), rtol=1e-14)
    # element by element on a small row
    x = np.array([[1.0, -2.0, 3.0, 0.5]])
    ms = (1 + 4 + 9 + 0.25) / 4
    np.testing.assert_allclose(U.rms_norm(x, w, 1e-6)[0], x[0] / math.sqrt(ms + 1e-6) * w, rtol=1e-14)
    # no mean subtraction: adding a constant changes the output
    assert not np.allclose(U.rms_norm(x + 1.0, w, 1e-6), U.rms_norm(x, w, 1e-6))


def test_gelu_tanh_identities():
    x = np.linspace(-8, 8, 2001)
    g = U.gelu_tanh(x)
    np.testing.assert_allclose(g - U.gelu_tanh(-x), x, atol=1e-12)   # tanh is odd
    erf_gelu = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in x])
    assert np.abs(g - erf_gelu).max() < 1e-3                         # close to the erf form
    assert U.gelu_tanh(np.array([0.0]))[0] == 0.0


# ----------------------------------------------------------------------------- attention by loops

def _attention_loops(n, wq, wk, wv, wo, rel_bias, valid, cfg):
    B, T, d = n.shape
    H, dk = cfg.num_heads, cfg.d_kv
    out = np.zeros((B, T, d))
    for b in range(B):
        q, k, v = n[b] @ wq.T, n[b] @ wk.T, n[b] @ wv.T
        o = np.zeros((T, d))
        for h in range(H):
            sl = slice(h * dk, (h + 1) * dk)
            for i in range(T):
                logits = []
                for j in range(T):
                    if not valid[b, j]:
                        continue
                    bucket = int(U.relative_bucket(np.array([j - i]), cfg.rel_buckets, cfg.rel_max_distance)[0])
                    logits.append((j, float(q[i, sl] @ k[j, sl]) + rel_bias[bucket, h]))
                if not logits:
                    continue
                mx = max(s for _, s in logits)
                den = sum(math.exp(s - mx) for _, s in logits)
                for j, s in logits:
                    o[i, sl] += math.exp(s - mx) / den * v[j, sl]
        out[b] = o @ wo.T
    return out


def test_attention_matches_loops():
    cfg = U.UMT5Config(d_model=8, num_heads=2, num_layers=1, d_ff=12, vocab_size=11,
                       rel_buckets=8, rel_max_distance=6)
    rng = np.random.default_rng(0)
    B, T = 2, 7
    n = rng.standard_normal((B, T, 8))
    wq, wk, wv, wo = (rng.standard_normal((8, 8)) * 0.5 for _ in range(4))
    rel_bias = rng.standard_normal((8, 2))
    valid = np.array([[1, 1, 1, 1, 1, 1, 1], [1, 1, 0, 1, 0, 0, 0]], bool)
    got = U.self_attention(n, wq, wk, wv, wo, rel_bias, valid, cfg)
    ref = _attention_loops(n, wq, wk, wv, wo, rel_bias, valid, cfg)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_attention_no_valid_key_gives_zero():
    cfg = U.UMT5Config(d_model=8, num_heads=2, num_layers=1, d_ff=12, vocab_size=11)
    rng = np.random.default_rng(1)
    n = rng.standard_normal((1, 3, 8))
    w = [rng.standard_normal((8, 8)) for _ in range(4)]
    out = U.self_attention(n, *w, rng.standard_normal((32, 2)), np.zeros((1, 3), bool), cfg)
    assert np.all(out == 0.0)


# ----------------------------------------------------------------------------- whole encoder

TINY = U.UMT5Config(d_model=16, num_heads=2, num_layers=2, d_ff=24, vocab_size=37)


def _weights(cfg, overrides=None):
    base = U.UMT5Weights.seeded(cfg)
    over = dict(overrides or {})
    return U.UMT5Weights(lambda name: over[name] if name in over else base[name])


def test_zero_output_projections_reduce_to_norm_of_embedding():
    cfg = TINY
    zero = {}
    for l in range(cfg.num_layers):
        zero[f"layer{l}.wo"] = np.zeros((cfg.d_model, cfg.d_model), np.float32)
        zero[f"layer{l}.wo_ff"] = np.zeros((cfg.d_model, cfg.d_ff), np.float32)
    W = _weights(cfg, zero)
    ids = seeded_inputs.token_ids(2, 9, cfg.vocab_size)
    out = U.encode(cfg, W, ids, dtype=np.float64)
    e = W["embed"][ids].astype(np.float64)
    ref = e / np.sqrt((e * e).mean(-1, keepdims=True) + cfg.eps) * W["final_ln"]
    np.testing.assert_allclose(out, ref, rtol=1e-12)


def test_padded_tokens_do_not_reach_valid_outputs():
    cfg = TINY
    W = _weights(cfg)
    ids = seeded_inputs.token_ids(2, 10, cfg.vocab_size)
    mask = seeded_inputs.length_mask(np.array([10, 6]), 10)
    a = U.encode(cfg, W, ids, mask, dtype=np.float64)
    ids2 = ids.copy()
    ids2[1, 6:] = (ids2[1, 6:] + 5) % cfg.vocab_size
    b = U.encode(cfg, W, ids2, mask, dtype=np.float64)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_allclose(a[1, :6], b[1, :6], rtol=1e-12, atol=1e-12)
    assert not np.allclose(a[1, 6:], b[1, 6:])


def test_position_shift_invariance():
    # Only relative positions enter: the same valid tokens moved right by k places,
    # with the k places before them masked, give the same outputs.
    cfg = TINY
    W = _weights(cfg)
    ids = seeded_inputs.token_ids(1, 8, cfg.vocab_size)
    a = U.encode(cfg, W, ids, np.ones((1, 8), np.uint8), dtype=np.float64)
    k = 3
    ids2 = np.concatenate([np.zeros((1, k), np.int32), ids], axis=1)
    mask2 = np.concatenate([np.zeros((1, k), np.uint8), np.ones((1, 8), np.uint8)], axis=1)
    b = U.encode(cfg, W, ids2, mask2, dtype=np.float64)
    np.testing.assert_allclose(b[0, k:], a[0], rtol=1e-11, atol=1e-12)


def test_encoder_direction_matters():
    # The bucket of +r and -r differ: reversing the token order is not a permutation
    # of the outputs (guards against a sign-blind bias).
    cfg = TINY
    W = _weights(cfg)
    ids = seeded_inputs.token_ids(1, 8, cfg.vocab_size)
    a = U.encode(cfg, W, ids, dtype=np.float64)
    b = U.encode(cfg, W, ids[:, ::-1].copy(), dtype=np.float64)
    assert not np.allclose(a[0], b[0, ::-1], rtol=1e-6)


def test_float32_tracks_float64():
    cfg = U.UMT5_SMALL
    W = U.UMT5Weights.seeded(cfg, bf16=True)
    ids = seeded_inputs.token_ids(2, 24, cfg.vocab_size)
    mask = seeded_inputs.length_mask(np.array([24, 11]), 24)
    a = U.encode(cfg, W, ids, mask, dtype=np.float32)
    b = U.encode(cfg, W, ids, mask, dtype=np.float64)
    assert np.abs(a - b).max() / np.abs(b).max() < 1e-4


def test_weight_list_full_config():
    specs = U.umt5_weight_specs(U.UMT5_FULL)
    assert len(specs) == 1 + 24 * len(U.LAYER_TENSORS) + 1
    total = sum(int(np.prod(s)) for _, s, _, _ in specs)
    d, F, L = 2048, 5120, 24
    assert total == 32128 * d + L * (4 * d * d + 3 * d * F + 2 * d + 32 * 32) + d
    assert U.UMT5_FULL.d_kv == 64
