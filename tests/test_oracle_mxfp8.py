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
