"""GPU parity of the text encoder (UMT5, random weights): the HIP path through the
C-ABI against the oracle (oracle/umt5.py) on the same seeded weights and tokens.

Bars: the embedding tap bit-exact (a bf16 table read into fp32); every layer's
residual stream and the final output max|d|/max|ref| <= 2e-2 and cosine >= 0.999,
and each layer's update (difference of consecutive taps) <= 1e-1 and cosine >= 0.995,
against the float32 oracle fed the same bf16-rounded weights (the GPU rounds the
matrix-product inputs, q, k, v, the attention probabilities and the gated FFN
output to bf16, 8 significant bits, which bounds each product's relative error
near 2^-8 per rounding).
"""
import numpy as np
import pytest

import seeded_inputs
from helpers import cosine, rel_max
from oracle import umt5 as U

pytestmark = pytest.mark.gpu

TOL = 2e-2
COS = 0.999


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _cfg_kw(ocfg):
    return dict(d_model=ocfg.d_model, num_heads=ocfg.num_heads, num_layers=ocfg.num_layers, d_ff=ocfg.d_ff,
                vocab_size=ocfg.vocab_size, rel_buckets=ocfg.rel_buckets, rel_max_distance=ocfg.rel_max_distance,
                eps=ocfg.eps)


def _encoder(af, ocfg, max_batch, max_tokens):
    _torch()
    m = af.UMT5Encoder(af.umt5_make_config(max_batch=max_batch, max_tokens=max_tokens, **_cfg_kw(ocfg)))
    m.load_seeded_weights(threads=16)
    return m


def _reference(ocfg, ids, mask):
    W = U.UMT5Weights.seeded(ocfg, bf16=True)
    taps = {-1: W["embed"][ids].astype(np.float32)}
    out = U.encode(ocfg, W, ids, mask, np.float32, taps=lambda l, x: taps.__setitem__(l, x.copy()))
    return out, taps


def _check(m, ocfg, ids, mask, layers):
    torch = _torch()
    ref, taps = _reference(ocfg, ids, mask)
    d_ids = torch.from_numpy(ids).cuda()
    d_mask = None if mask is None else torch.from_numpy(mask).cuda()
    got = {l: m.encode_taps(d_ids, d_mask, stop_after_layer=l).cpu().numpy() for l in [-1] + layers}
    out = m.encode(d_ids, d_mask).cpu().numpy()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got[-1], taps[-1])
    for l in layers:
        assert np.isfinite(got[l]).all(), l
        e, c = rel_max(got[l], taps[l]), cosine(got[l], taps[l])
        # the layer's own contribution (its two residual updates), which the embedding
        # does not dominate
        dg, dr = got[l] - got[l - 1], taps[l] - taps[l - 1]
        de, dc = rel_max(dg, dr), cosine(dg, dr)
        print(f"layer {l}: rel {e:.3e} cos {c:.6f}; update rel {de:.3e} cos {dc:.6f}")
        assert e <= TOL and c >= COS, (l, e, c)
        assert de <= 5 * TOL and dc >= 0.995, (l, de, dc)
    e, c = rel_max(out, ref), cosine(out, ref)
    print(f"output: rel {e:.3e} cos {c:.6f}")
    assert e <= TOL and c >= COS, (e, c)
    return out


@pytest.fixture(scope="module")
def small(af):
    m = _encoder(af, U.UMT5_SMALL, max_batch=3, max_tokens=320)
    yield m
    m.close()


def test_small_ragged_batch(af, small):
    """Three samples of 40 tokens with 40, 17 and 1 valid: several 32-key tiles, a ragged
    tail and a sample whose only key is its first token."""
    ids = seeded_inputs.token_ids(3, 40, U.UMT5_SMALL.vocab_size)
    mask = seeded_inputs.length_mask(np.array([40, 17, 1]), 40)
    _check(small, U.UMT5_SMALL, ids, mask, [0, 1])


def test_small_long_sequence(af, small):
    """300 tokens (the 512-token attention variant; relative distances past 128)."""
    ids = seeded_inputs.token_ids(1, 300, U.UMT5_SMALL.vocab_size)
    _check(small, U.UMT5_SMALL, ids, None, [0, 1])


def test_small_sample_without_valid_tokens(af, small):
    """A sample whose mask is all zero: attention contributes zero for it, as the oracle says."""
    ids = seeded_inputs.token_ids(2, 9, U.UMT5_SMALL.vocab_size)
    mask = seeded_inputs.length_mask(np.array([9, 0]), 9)
    _check(small, U.UMT5_SMALL, ids, mask, [0, 1])


def test_small_deterministic_and_mask_invariant(af, small):
    torch = _torch()
    ids = seeded_inputs.token_ids(2, 33, U.UMT5_SMALL.vocab_size)
    mask = seeded_inputs.length_mask(np.array([33, 20]), 33)
    d_ids, d_mask = torch.from_numpy(ids).cuda(), torch.from_numpy(mask).cuda()
    a = small.encode(d_ids, d_mask).cpu().numpy()
    b = small.encode(d_ids, d_mask).cpu().numpy()
    np.testing.assert_array_equal(a, b)
    ids2 = ids.copy()
    ids2[1, 20:] = (ids2[1, 20:] + 7) % U.UMT5_SMALL.vocab_size      # only padded tokens change
    c = small.encode(torch.from_numpy(ids2).cuda(), d_mask).cpu().numpy()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a[0], c[0])
    np.testing.assert_array_equal(a[1, :20], c[1, :20])


def test_full_width_two_layers(af):
    """The pages' width (d_model 2048, 32 heads, d_ff 5120, vocabulary 32128), two layers,
    a CFG-style batch of 2 prompts x 256 tokens with ragged valid lengths."""
    m = _encoder(af, U.UMT5_PAIR, max_batch=2, max_tokens=256)
    try:
        ids = seeded_inputs.token_ids(2, 256, U.UMT5_PAIR.vocab_size)
        mask = seeded_inputs.length_mask(seeded_inputs.valid_lengths(2, 16, 256), 256)
        _check(m, U.UMT5_PAIR, ids, mask, [0, 1])
    finally:
        m.close()


def test_small_empty_batch_and_no_tokens(af, small):
    """B = 0 or T = 0 enqueue nothing and return an empty result."""
    torch = _torch()
    ids = torch.zeros((0, 5), dtype=torch.int32, device="cuda")
    assert tuple(small.encode(ids).shape) == (0, 5, U.UMT5_SMALL.d_model)
    ids = torch.zeros((2, 0), dtype=torch.int32, device="cuda")
    assert tuple(small.encode(ids).shape) == (2, 0, U.UMT5_SMALL.d_model)
    torch.cuda.synchronize()
