"""GPU parity at the workloads' full sizes, in the launch configuration the bench
times: the full AuraFlow transformer (4 joint + 32 single blocks, d = 3072,
12 x 256 heads, FFN 8192, 96 x 96 PE table) at 1024^2 and 1536^2 with CFG
batch 2, a batch-8 forward of the 4-image sampling workload, and the 25-step
sampling loop.

Oracle comparisons use the float32 oracle with the same bf16-rounded weights and
text. Two checks per sampled block b:
  * the residual after block b (GPU chain against oracle chain), bar
    max|d|/max|ref| <= 2e-2 and cosine >= 0.999;
  * block b's own update: the GPU's x_b - x_{b-1} against the oracle's block b
    applied to the GPU's own x_{b-1}, minus x_{b-1}, element by element, at the
    same bar (the update is about a quarter of the residual's norm, so the
    residual check alone would let an update be ~9% wrong).
The chained update (x_b - x_{b-1} of each side's own chain) is printed as well.
Where the oracle's full forward takes minutes of host time (1536^2, batch 8),
its output comes from tests/golden/fullsize_oracle.npz, written by
tests/golden/make_fullsize_golden.py from the oracle alone; the per-block
updates are computed live.
"""
import importlib.util
import os

import numpy as np
import pytest

import oracle
import seeded_inputs
from helpers import (PrefetchWeights, cosine, oracle_block_on, oracle_cfg, rel_max, to_dev, update_metrics,
                     workload_inputs)

pytestmark = pytest.mark.gpu

TOL, COS = 2e-2, 0.999
HERE = os.path.dirname(os.path.abspath(__file__))


def _golden_module():
    spec = importlib.util.spec_from_file_location("make_fullsize_golden",
                                                  os.path.join(HERE, "golden", "make_fullsize_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _golden(name, inputs):
    mod = _golden_module()
    g = np.load(os.path.join(HERE, "golden", "fullsize_oracle.npz"))
    np.testing.assert_array_equal(g[name + "_checksum"], mod.checksum(*inputs))   # same input recipe
    return g[name]


@pytest.fixture(scope="module")
def full(af):
    import torch
    assert torch.cuda.is_available()
    cfg = af.make_config(max_batch=8, max_latent_h=192, max_latent_w=192, max_text_len=256)
    m = af.AuraFlowModel(cfg)
    m.load_seeded_weights(seed=0, threads=16)
    yield cfg, m
    m.close()


def _inputs(H, W):
    lengths = seeded_inputs.valid_lengths(2, 16, 256)
    lat, taus, text, mask = workload_inputs(2, 4, H, W, 256, 2048, lengths=lengths, cfg_pairs=True)
    return lat, taus, oracle.round_bf16(text), mask


def _check(name, got, ref):
    e, c = rel_max(got, ref), cosine(got, ref)
    print(f"{name}: rel {e:.3e} cos {c:.6f}", flush=True)
    assert e <= TOL and c >= COS, (name, e, c)


def _check_updates(ocfg, W, temb, kv, got, blocks, Nt, mx=False, tol=TOL, cos=COS, chain=None):
    """Each block's own update against the oracle's block on the GPU's input."""
    for b in blocks:
        ref_next = oracle_block_on(ocfg, W, temb, kv, got[b - 1], b, Nt, mx)
        e, c = update_metrics(got[b - 1], got[b], ref_next)
        msg = f"block {b} update: rel {e:.3e} cos {c:.6f}"
        if chain is not None and b in chain and b - 1 in chain:
            ec, cc = update_metrics(chain[b - 1], got[b] - got[b - 1] + chain[b - 1], chain[b])
            msg += f" (chained update: rel {ec:.3e} cos {cc:.6f})"
        print(msg, flush=True)
        assert e <= tol and c >= cos, (b, e, c)


def _taps(m, dev, blocks):
    return {b: m.forward_taps(*dev, stop_after_block=b).cpu().numpy() for b in sorted(blocks)}


@pytest.mark.timeout(1200)
def test_full_1024_every_sampled_block_and_output(af, full):
    import torch
    cfg, m = full
    ocfg = oracle_cfg(cfg)
    lat, taus, text, mask = _inputs(128, 128)
    dev = (to_dev(lat), to_dev(taus), to_dev(text), to_dev(mask))
    blocks = (0, 3, 4, 12, 24, 35)
    got = _taps(m, dev, set(blocks) | {b - 1 for b in blocks})
    out = m.forward(*dev).cpu().numpy()
    torch.cuda.synchronize()
    taps = {}
    W = PrefetchWeights(ocfg).as_weights()
    temb, xt, xi, kv = oracle.embed(ocfg, W, lat, taus, text, mask, np.float32)
    taps[-1] = np.concatenate([xt, xi], 1)
    Nt = xt.shape[1]

    def tap(i, xt_, xi_):
        if i in got:
            taps[i] = np.concatenate([xt_, xi_], 1)
        if i in blocks:
            _check(f"block {i}", got[i], taps[i])
            _check_updates(ocfg, W, temb, kv, got, [i], Nt, chain=taps)

    ref = oracle.forward(ocfg, W, lat, taus, text, mask, np.float32, taps=tap)
    _check("output", out, ref)


def test_full_1024_deterministic_and_mask_invariant(af, full):
    import torch
    cfg, m = full
    lat, taus, text, mask = _inputs(128, 128)
    dev = (to_dev(lat), to_dev(taus), to_dev(text), to_dev(mask))
    a = m.forward(*dev).cpu().numpy()
    b = m.forward(*dev).cpu().numpy()
    assert np.isfinite(a).all()
    np.testing.assert_array_equal(a, b)
    text2 = text.copy()
    text2[mask == 0] = -3.0
    c = m.forward(dev[0], dev[1], to_dev(text2), dev[3]).cpu().numpy()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a, c)


@pytest.mark.timeout(900)
def test_full_1536_whole_forward(af, full):
    """1536^2 (S = 9480, the whole PE grid): the 36-block output against the oracle's
    (stored), the residual after the first joint block against the oracle's chain,
    and the own updates of blocks 0, 4 and 35."""
    import torch
    cfg, m = full
    ocfg = oracle_cfg(cfg)
    lat, taus, text, mask = _inputs(192, 192)
    dev = (to_dev(lat), to_dev(taus), to_dev(text), to_dev(mask))
    got = _taps(m, dev, (-1, 0, 3, 4, 34, 35))
    out = m.forward(*dev).cpu().numpy()
    torch.cuda.synchronize()
    assert np.isfinite(out).all() and out.shape == (2, 4, 192, 192)
    _check("1536 output", out, _golden("d1536", (lat, taus, text, mask)))
    W = PrefetchWeights(ocfg).as_weights()
    temb, xt, xi, kv = oracle.embed(ocfg, W, lat, taus, text, mask, np.float32)
    Nt = xt.shape[1]
    _check("1536 embedding", got[-1], np.concatenate([xt, xi], 1))
    ref0 = oracle_block_on(ocfg, W, temb, kv, np.concatenate([xt, xi], 1), 0, Nt)
    _check("1536 block 0", got[0], ref0)
    _check_updates(ocfg, W, temb, kv, got, (0, 4, 35), Nt)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("H,W", [(126, 94), (66, 158), (150, 40)])
def test_full_any_resolution_first_joint_block(af, full, H, W):
    """One library instance (workspace sized for 192 x 192 latents) serving
    non-square resolutions whose patch grids leave odd margins in the 96 x 96
    position table (centre crop offsets rounded down): the embedding, the residual
    after the first joint block and that block's own update match the oracle, and
    the whole forward is finite."""
    import torch
    cfg, m = full
    ocfg = oracle_cfg(cfg)
    lat, taus, text, mask = _inputs(H, W)
    dev = (to_dev(lat), to_dev(taus), to_dev(text), to_dev(mask))
    got = _taps(m, dev, (-1, 0))
    out = m.forward(*dev).cpu().numpy()
    torch.cuda.synchronize()
    assert np.isfinite(out).all() and out.shape == (2, 4, H, W)
    W_o = PrefetchWeights(ocfg).as_weights()
    temb, xt, xi, kv = oracle.embed(ocfg, W_o, lat, taus, text, mask, np.float32)
    Nt = xt.shape[1]
    _check(f"{H}x{W} embedding", got[-1], np.concatenate([xt, xi], 1))
    _check(f"{H}x{W} block 0", got[0], oracle_block_on(ocfg, W_o, temb, kv, np.concatenate([xt, xi], 1), 0, Nt))
    _check_updates(ocfg, W_o, temb, kv, got, (0,), Nt)


@pytest.mark.timeout(900)
def test_full_batch8_forward_sampled_samples(af, full):
    """The transformer batch of the 4-image sampling workload (8 = 4 uncond + 4 cond,
    every row at tau = sigma_10): samples 1 and 6 of the batch-8 output against the
    oracle's forward of those two samples (rows are independent outside each
    sample's attention), and the own updates of blocks 0, 4 and 35 on those rows."""
    import torch
    cfg, m = full
    ocfg = oracle_cfg(cfg)
    mod = _golden_module()
    lat, taus, text, mask = mod.e_inputs()
    dev = (to_dev(lat), to_dev(taus), to_dev(text), to_dev(mask))
    got8 = _taps(m, dev, (-1, 0, 3, 4, 34, 35))
    out = m.forward(*dev).cpu().numpy()
    torch.cuda.synchronize()
    rows = list(mod.E_SAMPLES)
    _check("batch 8 output, samples 1 and 6", out[rows], _golden("e1024_b8", (lat, taus, text, mask)))
    W = PrefetchWeights(ocfg).as_weights()
    temb, xt, xi, kv = oracle.embed(ocfg, W, lat[rows], taus[rows], text[rows], mask[rows], np.float32)
    Nt = xt.shape[1]
    got = {b: v[rows] for b, v in got8.items()}
    _check("batch 8 embedding, samples 1 and 6", got[-1], np.concatenate([xt, xi], 1))
    _check_updates(ocfg, W, temb, kv, got, (0, 4, 35), Nt)


@pytest.mark.timeout(900)
def test_block_pair_1536_attention_branch_only(af):
    """Attention-isolating case: 1 joint + 1 single block at the full width and
    1536^2 (S = 9480) with the FFN gates of every adaLN matrix zeroed, so each
    block's update is its attention branch alone; about half of each sample's text
    is padding (the split query tiles of the last partial round run). Both blocks'
    own updates and the output against the oracle."""
    import torch
    cfg = af.make_config(num_mmdit_layers=1, num_single_dit_layers=1, max_batch=2, max_latent_h=192,
                         max_latent_w=192, max_text_len=256)
    m = af.AuraFlowModel(cfg)
    ocfg = oracle_cfg(cfg)
    d = ocfg.inner_dim
    Wseed = oracle.Weights.seeded(ocfg, seed=0, bf16=False)
    overrides = {}
    for name, _, _ in oracle.weight_specs(ocfg):
        if name.endswith("ada"):
            a = Wseed[name].copy()
            a[5 * d:6 * d] = 0                     # gate2: the FFN branch contributes nothing
            overrides[name] = a
    m.load_seeded_weights(seed=0, overrides=overrides, threads=16)
    W = oracle.Weights.seeded(ocfg, seed=0, bf16=True, overrides={k: oracle.round_bf16(v) for k, v in overrides.items()})
    lat, taus, text, _ = _inputs(192, 192)
    mask = seeded_inputs.length_mask(np.array([128, 97]), 256)
    dev = (to_dev(lat), to_dev(taus), to_dev(text), to_dev(mask))
    got = _taps(m, dev, (-1, 0, 1))
    out = m.forward(*dev).cpu().numpy()
    torch.cuda.synchronize()
    m.close()
    temb, xt, xi, kv = oracle.embed(ocfg, W, lat, taus, text, mask, np.float32)
    Nt = xt.shape[1]
    _check_updates(ocfg, W, temb, kv, got, (0, 1), Nt)
    ref = oracle.forward(ocfg, W, lat, taus, text, mask, np.float32)
    _check("attention-only block pair output", out, ref)


def test_full_sampling_loop_batch_composition(af, full):
    """25-step CFG sampling of 4 images (transformer batch 8): every image's
    trajectory matches sampling it alone (to the bf16 bar: the attention splits
    the work of the last partial round of query tiles over key ranges, and
    which tiles are split depends on the batch size, so the fp32 summation
    order of those tiles differs), and the loop equals the explicit forward +
    Euler-CFG composition bit for bit."""
    import torch
    cfg, m = full
    Bp, T = 4, 256
    x0 = seeded_inputs.latents(Bp, 4, 128, 128)
    text_u = seeded_inputs.text_embeddings(Bp, T, 2048, first_index=100)
    text_c = seeded_inputs.text_embeddings(Bp, T, 2048, first_index=200)
    len_u = seeded_inputs.valid_lengths(Bp, 16, T, seed=5)
    len_c = seeded_inputs.valid_lengths(Bp, 16, T, seed=6)
    text = np.concatenate([text_u, text_c])
    mask = seeded_inputs.length_mask(np.concatenate([len_u, len_c]), T)
    x = to_dev(x0)
    m.sample(x, to_dev(text), to_dev(mask), num_steps=25, shift=1.73, guidance=3.5)
    xb = x.cpu().numpy()
    assert np.isfinite(xb).all()
    i = 2
    xi = to_dev(x0[i:i + 1])
    ti = np.concatenate([text_u[i:i + 1], text_c[i:i + 1]])
    mi = np.concatenate([mask[i:i + 1], mask[Bp + i:Bp + i + 1]])
    m.sample(xi, to_dev(ti), to_dev(mi), num_steps=25, shift=1.73, guidance=3.5)
    alone = xi.cpu().numpy()[0]
    e, c = rel_max(alone, xb[i]), cosine(alone, xb[i])
    print(f"image {i} alone vs in batch 8 after 25 steps: rel {e:.3e} cos {c:.6f}")
    assert e <= TOL and c >= COS, (e, c)
    # The loop's step is the explicit forward + Euler-CFG composition (one step).
    sig1 = af.af_sigma_schedule(1, 1.73)
    xin = to_dev(np.concatenate([x0, x0]))
    xs1 = to_dev(x0)
    v1 = m.forward(xin, to_dev(np.full(2 * Bp, sig1[0], np.float32)), to_dev(text), to_dev(mask))
    af.af_flow_euler_cfg_step(xs1, v1, float(sig1[0]), float(sig1[1]), 3.5)
    x1 = to_dev(x0)
    m.sample(x1, to_dev(text), to_dev(mask), num_steps=1, shift=1.73, guidance=3.5)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(x1.cpu().numpy(), xs1.cpu().numpy())
