"""GPU parity of the MXFP8 model (QKV, out-projection and FFN products on MXFP8 operands) against
the oracle's mx mode, which quantizes the same operands with the same rule
(oracle/numerics.py mxfp8_qdq, pinned in test_oracle_mxfp8.py) and accumulates
in float32. Quantization happens at the same points on both sides, but the GPU
feeds it values that already differ from the fp32 oracle's by the bf16 path's
own rounding (bf16 q/k/v and attention output, summation order): an element
whose value moves by a relative delta crosses an E4M3 rounding boundary with
probability about delta / 2^-3 and then changes by one E4M3 step (2^-3
relative). At the full width this turns the bf16 path's ~1e-3 block agreement
into several 1e-3 per block, growing through the blocks, so the bar here is
max|d|/max|ref| <= 6e-2 and cosine >= 0.998 (measured: the 1 joint + 1 single
block pair at 512^2 gives 8.1e-3 and 2.5e-2 per block and 3.9e-2 at the output,
cosine >= 0.9995; the full model at 1024^2 gives 9.0e-3 / 0.99996 after the first
block and 4.2e-2 / 0.99887 after the fifth). Each comparison also checks that
the GPU result is closer to the oracle's mx mode than to its plain mode."""
import numpy as np
import pytest

import oracle
import seeded_inputs
from helpers import PrefetchWeights, cosine, oracle_cfg, rel_max, to_dev, workload_inputs

pytestmark = pytest.mark.gpu

TOL, COS = 6e-2, 0.998


def _torch():
    import torch
    assert torch.cuda.is_available()
    return torch


def _taps(ocfg, W, lat, tau, text, mask, blocks, mx):
    taps = {}
    emb = oracle.embed(ocfg, W, lat, tau, text, mask, np.float32)
    taps[-1] = np.concatenate([emb[1], emb[2]], axis=1)
    out = oracle.forward(ocfg, W, lat, tau, text, mask, np.float32, mx=mx,
                         taps=lambda i, xt, xi: taps.__setitem__(i, np.concatenate([xt, xi], 1)) if i in blocks else None)
    return out, taps


def test_small_mxfp8_blocks_match_oracle(af):
    torch = _torch()
    cfg = af.make_config(compute_dtype=af.AF_MXFP8, num_attention_heads=2, caption_projection_dim=512,
                         joint_attention_dim=128, pos_embed_max_size=256, num_mmdit_layers=1, num_single_dit_layers=2,
                         max_batch=3, max_latent_h=32, max_latent_w=32, max_text_len=16)
    m = af.AuraFlowModel(cfg)
    m.load_seeded_weights(seed=0)
    ocfg = oracle_cfg(cfg)
    W_o = oracle.Weights.seeded(ocfg, seed=0, bf16=True)
    B, H, Wd, T = 3, 22, 30, 13
    lat, taus, text, mask = workload_inputs(B, 4, H, Wd, T, 128, lengths=seeded_inputs.valid_lengths(B, 1, T),
                                            cfg_pairs=False)
    text = oracle.round_bf16(text)
    ref, taps = _taps(ocfg, W_o, lat, taus, text, mask, (0, 1, 2), mx=True)
    ref_bf16, _ = _taps(ocfg, W_o, lat, taus, text, mask, (), mx=False)
    dev = (to_dev(lat), to_dev(taus), to_dev(text), to_dev(mask))
    got = {blk: m.forward_taps(*dev, stop_after_block=blk).cpu().numpy() for blk in (0, 1, 2)}
    out = m.forward(*dev).cpu().numpy()
    out2 = m.forward(*dev).cpu().numpy()
    torch.cuda.synchronize()
    for blk in (0, 1, 2):
        e, c = rel_max(got[blk], taps[blk]), cosine(got[blk], taps[blk])
        print(f"block {blk}: rel {e:.3e} cos {c:.6f}")
        assert e <= TOL and c >= COS, (blk, e, c)
    e, c = rel_max(out, ref), cosine(out, ref)
    e16 = rel_max(out, ref_bf16)
    print(f"output: rel {e:.3e} cos {c:.6f}; against the bf16 oracle rel {e16:.3e}")
    assert e <= TOL and c >= COS, (e, c)
    assert e16 > e                       # the quantization is really applied
    np.testing.assert_array_equal(out, out2)
    m.close()


@pytest.mark.timeout(900)
def test_block_pair_mxfp8_matches_oracle(af):
    torch = _torch()
    cfg = af.make_config(compute_dtype=af.AF_MXFP8, num_mmdit_layers=1, num_single_dit_layers=1, max_batch=2,
                         max_latent_h=64, max_latent_w=64, max_text_len=256)
    m = af.AuraFlowModel(cfg)
    m.load_seeded_weights(seed=0, threads=16)
    ocfg = oracle_cfg(cfg)
    names = [n for n, _, _ in oracle.weight_specs(ocfg)]
    Wseed = oracle.Weights.seeded(ocfg, seed=0, bf16=True)
    W_o = oracle.Weights.from_dict(ocfg, {n: Wseed[n] for n in names})
    lengths = seeded_inputs.valid_lengths(2, 16, 256)
    lat, taus, text, mask = workload_inputs(2, 4, 64, 64, 256, 2048, lengths=lengths, cfg_pairs=True)
    text = oracle.round_bf16(text)
    ref, taps = _taps(ocfg, W_o, lat, taus, text, mask, (0, 1), mx=True)
    dev = (to_dev(lat), to_dev(taus), to_dev(text), to_dev(mask))
    got = {blk: m.forward_taps(*dev, stop_after_block=blk).cpu().numpy() for blk in (0, 1)}
    out = m.forward(*dev).cpu().numpy()
    torch.cuda.synchronize()
    for blk in (0, 1):
        e, c = rel_max(got[blk], taps[blk]), cosine(got[blk], taps[blk])
        print(f"block {blk}: rel {e:.3e} cos {c:.6f}")
        assert e <= TOL and c >= COS, (blk, e, c)
    e, c = rel_max(out, ref), cosine(out, ref)
    ref_plain, _ = _taps(ocfg, W_o, lat, taus, text, mask, (), mx=False)
    e_plain = rel_max(out, ref_plain)
    print(f"output: rel {e:.3e} cos {c:.6f}; against the oracle without MXFP8 rel {e_plain:.3e}")
    assert e <= TOL and c >= COS, (e, c)
    assert e_plain > e
    m.close()


@pytest.mark.timeout(1200)
def test_full_1024_mxfp8_first_joint_and_single_blocks(af):
    """The full model at 1024^2, CFG batch 2, in MXFP8 mode: the residual after the
    first joint block and after the first single block against the oracle's mx
    mode, a finite output, and two forwards bit for bit equal."""
    torch = _torch()
    cfg = af.make_config(compute_dtype=af.AF_MXFP8, max_batch=2, max_latent_h=128, max_latent_w=128,
                         max_text_len=256)
    m = af.AuraFlowModel(cfg)
    m.load_seeded_weights(seed=0, threads=16)
    ocfg = oracle_cfg(cfg)
    lengths = seeded_inputs.valid_lengths(2, 16, 256)
    lat, taus, text, mask = workload_inputs(2, 4, 128, 128, 256, 2048, lengths=lengths, cfg_pairs=True)
    text = oracle.round_bf16(text)
    dev = (to_dev(lat), to_dev(taus), to_dev(text), to_dev(mask))
    got = {b: m.forward_taps(*dev, stop_after_block=b).cpu().numpy() for b in (0, 4)}
    a = m.forward(*dev).cpu().numpy()
    b = m.forward(*dev).cpu().numpy()
    torch.cuda.synchronize()
    assert np.isfinite(a).all()
    np.testing.assert_array_equal(a, b)
    m.close()
    W = PrefetchWeights(ocfg).as_weights()
    temb, xt, xi, kv = oracle.embed(ocfg, W, lat, taus, text, mask, np.float32)
    blk = lambda p: {k: W[p + k] for k in ("ada", "wq", "wk", "wv", "wo", "ff1", "ff2", "ff3")}
    for j in range(ocfg.num_mmdit_layers):
        xt, xi = oracle.joint_block(ocfg, blk(f"joint{j}.img."), blk(f"joint{j}.txt."), temb, xt, xi, kv,
                                    np.float32, mx=True)
        if j == 0:
            ref0 = np.concatenate([xt, xi], 1)
    x = oracle.single_block(ocfg, blk("single0."), temb, np.concatenate([xt, xi], 1), kv, np.float32, mx=True)
    # the same five blocks without quantization
    temb, pt, pi, kv = oracle.embed(ocfg, W, lat, taus, text, mask, np.float32)
    for j in range(ocfg.num_mmdit_layers):
        pt, pi = oracle.joint_block(ocfg, blk(f"joint{j}.img."), blk(f"joint{j}.txt."), temb, pt, pi, kv, np.float32)
    plain4 = oracle.single_block(ocfg, blk("single0."), temb, np.concatenate([pt, pi], 1), kv, np.float32)
    for name, g_, r in (("block 0", got[0], ref0), ("block 4", got[4], x)):
        e, c = rel_max(g_, r), cosine(g_, r)
        print(f"{name}: rel {e:.3e} cos {c:.6f}")
        assert e <= TOL and c >= COS, (name, e, c)
    e_plain = rel_max(got[4], plain4)
    print(f"block 4 against the oracle without MXFP8: rel {e_plain:.3e} cos {cosine(got[4], plain4):.6f}")
    assert e_plain > rel_max(got[4], x)


def test_block_pair_mxfp8_non_square_latent(af):
    """MXFP8 at the full width with a non-square latent and odd crop margins (66 x 158:
    33 x 79 patches, S = 8 + 256 + 2607 = 2871 tokens per sample): ragged GEMM row tiles
    and MXFP8 scale rows past the last real row."""
    torch = _torch()
    cfg = af.make_config(compute_dtype=af.AF_MXFP8, num_mmdit_layers=1, num_single_dit_layers=1, max_batch=2,
                         max_latent_h=66, max_latent_w=158, max_text_len=256)
    m = af.AuraFlowModel(cfg)
    m.load_seeded_weights(seed=0, threads=16)
    ocfg = oracle_cfg(cfg)
    names = [n for n, _, _ in oracle.weight_specs(ocfg)]
    Wseed = oracle.Weights.seeded(ocfg, seed=0, bf16=True)
    W_o = oracle.Weights.from_dict(ocfg, {n: Wseed[n] for n in names})
    lengths = seeded_inputs.valid_lengths(2, 16, 256)
    lat, taus, text, mask = workload_inputs(2, 4, 66, 158, 256, 2048, lengths=lengths, cfg_pairs=True)
    text = oracle.round_bf16(text)
    dev = (to_dev(lat), to_dev(taus), to_dev(text), to_dev(mask))
    got = {b: m.forward_taps(*dev, stop_after_block=b).cpu().numpy() for b in (0, 1)}
    out = m.forward(*dev).cpu().numpy()
    torch.cuda.synchronize()
    m.close()
    assert np.isfinite(out).all()
    taps = {}
    ref = oracle.forward(ocfg, W_o, lat, taus, text, mask, np.float32, mx=True,
                         taps=lambda i, xt, xi: taps.__setitem__(i, np.concatenate([xt, xi], axis=1)))
    for b in (0, 1):
        e, c = rel_max(got[b], taps[b]), cosine(got[b], taps[b])
        print(f"block {b}: rel {e:.3e} cos {c:.6f}")
        assert e <= TOL and c >= COS, (b, e, c)
    e, c = rel_max(out, ref), cosine(out, ref)
    print(f"output: rel {e:.3e} cos {c:.6f}")
    assert e <= TOL and c >= COS, (e, c)
