"""GPU parity: the HIP path, called through the C-ABI, against the CPU oracle on
the same seeded inputs.

Bars: fp32 path max|d|/max|ref| <= 1e-4 against the float64 oracle; bf16 path
max|d|/max|ref| <= 2e-2 and cosine >= 0.999 per block output against the
float32 oracle fed the same bf16-rounded weights and text.
"""
import numpy as np
import pytest

import oracle
import seeded_inputs
from helpers import cosine, oracle_block_on, oracle_cfg, rel_max, to_dev, update_metrics, workload_inputs

pytestmark = pytest.mark.gpu

FP32_TOL = 1e-4
BF16_TOL = 2e-2
BF16_COS = 0.999


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _taps_ref(ocfg, W, lat, tau, text, mask, dtype):
    taps = {}
    emb = oracle.embed(ocfg, W, lat, tau, text, mask, dtype)
    taps[-1] = np.concatenate([emb[1], emb[2]], axis=1)
    out = oracle.forward(ocfg, W, lat, tau, text, mask, dtype,
                         taps=lambda i, xt, xi: taps.__setitem__(i, np.concatenate([xt, xi], axis=1)))
    return out, taps


# ============================================================================ tiny fp32 (config A family)

def _tiny_cfg(af, **kw):
    base = dict(compute_dtype=af.AF_F32, num_attention_heads=4, attention_head_dim=8, caption_projection_dim=32,
                joint_attention_dim=32, pos_embed_max_size=64, num_mmdit_layers=1, num_single_dit_layers=1,
                max_batch=6, max_latent_h=16, max_latent_w=16, max_text_len=8)
    base.update(kw)
    return af.make_config(**base)


@pytest.fixture(scope="module")
def tiny(af):
    _torch()
    cfg = _tiny_cfg(af)
    m = af.AuraFlowModel(cfg)
    m.load_seeded_weights(seed=0)
    return cfg, m


@pytest.mark.parametrize("B,H,W,T,lengths,tau", [
    (1, 16, 16, 8, None, 0.5),                 # config A: 64 image tokens, text all valid, t = 500
    (2, 12, 16, 8, [8, 3], None),              # ragged: 6 x 8 patch grid, off-centre crop, padding masked
    (2, 16, 10, 5, [5, 1], None),              # non-square, short text
    (1, 4, 4, 0, None, 0.25),                  # no text tokens at all
    (6, 12, 14, 6, [6, 2, 5, 1, 3, 4], None),  # more samples than the patch embedding stages at once
])
def test_tiny_fp32_forward_matches_oracle(af, tiny, B, H, W, T, lengths, tau):
    torch = _torch()
    cfg, m = tiny
    ocfg = oracle_cfg(cfg)
    lat, taus, text, mask = workload_inputs(B, 4, H, W, T, 32, lengths=lengths, cfg_pairs=False, tau=tau)
    W_o = oracle.Weights.seeded(ocfg, seed=0, bf16=False)
    ref, taps = _taps_ref(ocfg, W_o, lat, taus, text, mask, np.float64)
    out = m.forward(to_dev(lat), to_dev(taus), to_dev(text), None if mask is None else to_dev(mask))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert got.shape == ref.shape
    assert rel_max(got, ref) <= FP32_TOL, rel_max(got, ref)
    for blk in (-1, 0, 1):
        r = m.forward_taps(to_dev(lat), to_dev(taus), to_dev(text), None if mask is None else to_dev(mask),
                           stop_after_block=blk).cpu().numpy()
        assert rel_max(r, taps[blk]) <= FP32_TOL, (blk, rel_max(r, taps[blk]))


def test_tiny_fp32_sampling_loop_matches_oracle(af, tiny):
    torch = _torch()
    cfg, m = tiny
    ocfg = oracle_cfg(cfg)
    W_o = oracle.Weights.seeded(ocfg, seed=0, bf16=False)
    x0 = seeded_inputs.latents(1, 4, 16, 16)
    text = seeded_inputs.text_embeddings(2, 8, 32)
    mask = seeded_inputs.length_mask(np.array([2, 8]), 8)
    steps, shift, gs = 3, 1.73, 3.5
    sig = oracle.sigma_schedule(steps, shift)
    x = x0.astype(np.float64)
    for i in range(steps):
        sig32 = np.float32(sig[i])
        v = oracle.forward(ocfg, W_o, np.concatenate([x, x]).astype(np.float32),
                           np.full(2, sig32, np.float32), text, mask, np.float64)
        x = oracle.cfg_euler_step(x, v, float(np.float32(sig[i])), float(np.float32(sig[i + 1])), gs)
    xg = to_dev(x0)
    m.sample(xg, to_dev(text), to_dev(mask), num_steps=steps, shift=shift, guidance=gs)
    torch.cuda.synchronize()
    assert rel_max(xg.cpu().numpy(), x) <= FP32_TOL


# ============================================================================ Euler + CFG kernel

@pytest.mark.parametrize("gs", [3.5, 1.0, 0.0])
def test_euler_cfg_step_matches_oracle(af, gs):
    torch = _torch()
    Bi = 3
    x = seeded_inputs.normal(7, 0, (Bi, 4, 20, 12))
    nv = 2 * Bi if gs > 1 else Bi
    v = seeded_inputs.normal(7, 1, (nv, 4, 20, 12))
    xd = to_dev(x)
    af.af_flow_euler_cfg_step(xd, to_dev(v), 0.8, 0.55, gs)
    torch.cuda.synchronize()
    ref = oracle.cfg_euler_step(x.astype(np.float64), v.astype(np.float64), float(np.float32(0.8)),
                                float(np.float32(0.55)), gs)
    np.testing.assert_allclose(xd.cpu().numpy(), ref, rtol=1e-6, atol=1e-6)


# ============================================================================ small bf16 (ragged tiles)

def _small_bf16_cfg(af):
    # d = 512 (2 heads x 256), F = 1536, 16 x 16 PE grid; sizes chosen so every
    # GEMM and attention tile has a ragged tail.
    return af.make_config(num_attention_heads=2, caption_projection_dim=512, joint_attention_dim=128,
                          pos_embed_max_size=256, num_mmdit_layers=1, num_single_dit_layers=2, max_batch=3,
                          max_latent_h=32, max_latent_w=32, max_text_len=16)


@pytest.fixture(scope="module")
def small_bf16(af):
    _torch()
    cfg = _small_bf16_cfg(af)
    m = af.AuraFlowModel(cfg)
    m.load_seeded_weights(seed=0)
    ocfg = oracle_cfg(cfg)
    W_o = oracle.Weights.seeded(ocfg, seed=0, bf16=True)
    B, H, Wd, T = 3, 22, 30, 13                      # 11 x 15 patches, S = 8 + 13 + 165 = 186
    lengths = seeded_inputs.valid_lengths(B, 1, T)
    lat, taus, text, mask = workload_inputs(B, 4, H, Wd, T, 128, lengths=lengths, cfg_pairs=False)
    text = oracle.round_bf16(text)
    ref, taps = _taps_ref(ocfg, W_o, lat, taus, text, mask, np.float32)
    dev = (to_dev(lat), to_dev(taus), to_dev(text), to_dev(mask))
    return cfg, m, dev, ref, taps, (lat, taus, text, mask)


def test_small_bf16_blocks_match_oracle(af, small_bf16):
    torch = _torch()
    cfg, m, dev, ref, taps, host = small_bf16
    got = {blk: m.forward_taps(*dev, stop_after_block=blk).cpu().numpy() for blk in (-1, 0, 1, 2)}
    out = m.forward(*dev).cpu().numpy()
    torch.cuda.synchronize()
    assert rel_max(got[-1], taps[-1]) <= 1e-2
    ocfg = oracle_cfg(cfg)
    W_o = oracle.Weights.seeded(ocfg, seed=0, bf16=True)
    temb, xt, _, kv = oracle.embed(ocfg, W_o, *host, np.float32)
    for blk in (0, 1, 2):
        e, c = rel_max(got[blk], taps[blk]), cosine(got[blk], taps[blk])
        assert e <= BF16_TOL and c >= BF16_COS, (blk, e, c)
        # the block's own update: the oracle's block applied to the GPU's input residual
        eu, cu = update_metrics(got[blk - 1], got[blk],
                                oracle_block_on(ocfg, W_o, temb, kv, got[blk - 1], blk, xt.shape[1]))
        print(f"block {blk}: rel {e:.3e} cos {c:.6f}; update rel {eu:.3e} cos {cu:.6f}")
        assert eu <= BF16_TOL and cu >= BF16_COS, (blk, eu, cu)
    e, c = rel_max(out, ref), cosine(out, ref)
    assert e <= BF16_TOL and c >= BF16_COS, (e, c)


def test_small_bf16_single_sample_odd_rows(af, small_bf16):
    """One sample with S = 8 + 12 + 165 = 185 rows: an odd row count, so every
    row-tiled kernel ends on a ragged last row."""
    torch = _torch()
    cfg, m, _, _, _, _ = small_bf16
    ocfg = oracle_cfg(cfg)
    W_o = oracle.Weights.seeded(ocfg, seed=0, bf16=True)
    lat, taus, text, mask = workload_inputs(1, 4, 22, 30, 12, 128, lengths=[7], cfg_pairs=False)
    text = oracle.round_bf16(text)
    ref, taps = _taps_ref(ocfg, W_o, lat, taus, text, mask, np.float32)
    dev = (to_dev(lat), to_dev(taus), to_dev(text), to_dev(mask))
    got = {blk: m.forward_taps(*dev, stop_after_block=blk).cpu().numpy() for blk in (0, 1, 2)}
    out = m.forward(*dev).cpu().numpy()
    torch.cuda.synchronize()
    for blk in (0, 1, 2):
        e, c = rel_max(got[blk], taps[blk]), cosine(got[blk], taps[blk])
        assert e <= BF16_TOL and c >= BF16_COS, (blk, e, c)
    e, c = rel_max(out, ref), cosine(out, ref)
    assert e <= BF16_TOL and c >= BF16_COS, (e, c)


def test_small_bf16_no_text(af, small_bf16):
    """No text tokens (T = 0): the caption projection is skipped and attention runs over
    the 8 registers and the image tokens only."""
    torch = _torch()
    cfg, m, _, _, _, _ = small_bf16
    ocfg = oracle_cfg(cfg)
    W_o = oracle.Weights.seeded(ocfg, seed=0, bf16=True)
    lat, taus, text, mask = workload_inputs(2, 4, 18, 26, 0, 128, lengths=None, cfg_pairs=False)
    ref = oracle.forward(ocfg, W_o, lat, taus, text, None, np.float32)
    out = m.forward(to_dev(lat), to_dev(taus), to_dev(text), None).cpu().numpy()
    torch.cuda.synchronize()
    e, c = rel_max(out, ref), cosine(out, ref)
    assert e <= BF16_TOL and c >= BF16_COS, (e, c)


def test_small_bf16_fully_padded_text_and_empty_batch(af, small_bf16):
    """A sample whose text is all padding (only registers and image tokens are keys),
    beside one with 7 valid tokens; and an empty batch, which enqueues nothing."""
    torch = _torch()
    cfg, m, _, _, _, _ = small_bf16
    ocfg = oracle_cfg(cfg)
    W_o = oracle.Weights.seeded(ocfg, seed=0, bf16=True)
    lat, taus, text, mask = workload_inputs(2, 4, 22, 30, 13, 128, lengths=[0, 7], cfg_pairs=False)
    text = oracle.round_bf16(text)
    ref = oracle.forward(ocfg, W_o, lat, taus, text, mask, np.float32)
    out = m.forward(to_dev(lat), to_dev(taus), to_dev(text), to_dev(mask)).cpu().numpy()
    e, c = rel_max(out, ref), cosine(out, ref)
    assert e <= BF16_TOL and c >= BF16_COS, (e, c)
    empty = m.forward(to_dev(lat[:0]), to_dev(taus[:0]), to_dev(text[:0]), to_dev(mask[:0]))
    torch.cuda.synchronize()
    assert tuple(empty.shape) == (0, 4, 22, 30)


def test_small_bf16_deterministic_and_mask_invariant(af, small_bf16):
    torch = _torch()
    cfg, m, dev, ref, taps, host = small_bf16
    lat, taus, text, mask = host
    a = m.forward(*dev).cpu().numpy()
    b = m.forward(*dev).cpu().numpy()
    np.testing.assert_array_equal(a, b)
    text2 = text.copy()
    text2[mask == 0] = 37.0                       # only padded positions change
    c = m.forward(dev[0], dev[1], to_dev(text2), dev[3]).cpu().numpy()
    np.testing.assert_array_equal(a, c)
    # An all-ones mask equals no mask.
    ones = np.ones_like(mask)
    d1 = m.forward(dev[0], dev[1], dev[2], to_dev(ones)).cpu().numpy()
    d2 = m.forward(dev[0], dev[1], dev[2], None).cpu().numpy()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d1, d2)


def test_small_bf16_bf16_text_input(af, small_bf16):
    torch = _torch()
    cfg, m, dev, ref, taps, host = small_bf16
    a = m.forward(*dev).cpu().numpy()
    tb = dev[2].to(torch.bfloat16)
    b = m.forward(dev[0], dev[1], tb, dev[3]).cpu().numpy()
    np.testing.assert_array_equal(a, b)           # text already bf16-valued: same numbers


def test_small_bf16_zero_gates_reduce_to_embed_and_project(af):
    """All adaLN matrices zero: every block is the identity and the pre-final block a
    pass-through, so out = unpatchify(patch_embed(x) W_out^T) exactly as the oracle says."""
    torch = _torch()
    cfg = _small_bf16_cfg(af)
    m = af.AuraFlowModel(cfg)
    zeros = {name: np.zeros((r, c), np.float32) for name, r, c, _ in m.weights if name.endswith("ada")}
    m.load_seeded_weights(seed=0, overrides=zeros)
    ocfg = oracle_cfg(cfg)
    W_o = oracle.Weights.seeded(ocfg, seed=0, bf16=True, overrides=zeros)
    lat, taus, text, mask = workload_inputs(2, 4, 32, 32, 16, 128, lengths=[16, 3], cfg_pairs=False)
    text = oracle.round_bf16(text)
    ref = oracle.forward(ocfg, W_o, lat, taus, text, mask, np.float64)
    out = m.forward(to_dev(lat), to_dev(taus), to_dev(text), to_dev(mask)).cpu().numpy()
    torch.cuda.synchronize()
    assert rel_max(out, ref) <= 1e-5, rel_max(out, ref)
    m.close()


def test_small_bf16_embedding_stable_after_masked_attention(af, small_bf16):
    """Regression: the patch embedding once read LDS columns past C p^2 that it never
    wrote (times a zero weight); the masked attention leaves -inf key biases in LDS,
    so the embedding turned NaN after enough forwards. Interleave the two and check
    that the embedding tap stays finite and bit-identical."""
    torch = _torch()
    cfg, m, dev, ref, taps, _ = small_bf16
    first = m.forward_taps(*dev, stop_after_block=-1).cpu().numpy()
    assert np.isfinite(first).all()
    for i in range(24):
        m.forward(*dev)
        again = m.forward_taps(*dev, stop_after_block=-1).cpu().numpy()
        assert np.isfinite(again).all(), i
        np.testing.assert_array_equal(again, first)
    torch.cuda.synchronize()


# ============================================================================ config B: full-width block pair

@pytest.fixture(scope="module")
def block_pair(af):
    _torch()
    cfg = af.make_config(num_mmdit_layers=1, num_single_dit_layers=1, max_batch=2, max_latent_h=64,
                         max_latent_w=64, max_text_len=256)
    m = af.AuraFlowModel(cfg)
    m.load_seeded_weights(seed=0, threads=16)
    yield cfg, m
    m.close()


def test_block_pair_bf16_matches_oracle(af, block_pair):
    torch = _torch()
    cfg, m = block_pair
    ocfg = oracle_cfg(cfg)
    names = [n for n, _, _ in oracle.weight_specs(ocfg)]
    Wseed = oracle.Weights.seeded(ocfg, seed=0, bf16=True)
    W_o = oracle.Weights.from_dict(ocfg, {n: Wseed[n] for n in names})
    lengths = seeded_inputs.valid_lengths(2, 16, 256)
    lat, taus, text, mask = workload_inputs(2, 4, 64, 64, 256, 2048, lengths=lengths, cfg_pairs=True)
    text = oracle.round_bf16(text)
    ref, taps = _taps_ref(ocfg, W_o, lat, taus, text, mask, np.float32)
    dev = (to_dev(lat), to_dev(taus), to_dev(text), to_dev(mask))
    got = {blk: m.forward_taps(*dev, stop_after_block=blk).cpu().numpy() for blk in (-1, 0, 1)}
    out = m.forward(*dev).cpu().numpy()
    torch.cuda.synchronize()
    temb, xt, _, kv = oracle.embed(ocfg, W_o, lat, taus, text, mask, np.float32)
    for blk in (0, 1):
        assert np.isfinite(taps[blk]).all()
        bad = np.argwhere(~np.isfinite(got[blk]))
        assert len(bad) == 0, (blk, len(bad), bad[:8].tolist())
        e, c = rel_max(got[blk], taps[blk]), cosine(got[blk], taps[blk])
        # the block's own update: the oracle's block on the GPU's input residual
        eu, cu = update_metrics(got[blk - 1], got[blk],
                                oracle_block_on(ocfg, W_o, temb, kv, got[blk - 1], blk, xt.shape[1]))
        print(f"block {blk}: rel {e:.3e} cos {c:.6f}; update rel {eu:.3e} cos {cu:.6f}")
        assert e <= BF16_TOL and c >= BF16_COS, (blk, e, c)
        assert eu <= BF16_TOL and cu >= BF16_COS, (blk, eu, cu)
    e, c = rel_max(out, ref), cosine(out, ref)
    print(f"output: rel {e:.3e} cos {c:.6f}")
    assert e <= BF16_TOL and c >= BF16_COS, (e, c)
