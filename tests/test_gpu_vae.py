"""GPU parity of the VAE decode (the AutoencoderKL decoder, random weights): the HIP
path through the C-ABI (include/vae.h) against the oracle (oracle/vae.py) on the
same seeded weights (bf16-rounded on both sides) and latents.

Checked per stage: the activation after conv_in, after the mid block and after each
up level (the library's NHWC taps against the oracle's NCHW taps), and the image.
Each up level is also checked on its own: the oracle's level applied to the GPU's
previous tap, against the GPU's tap, so an error in one level cannot hide behind
the agreement of the chain. Bars: max|d|/max|ref| <= 2e-2 and cosine >= 0.999 (the
GPU rounds each convolution's operand -- the GroupNorm + SiLU output -- and the
attention's q, k, v and probabilities to bf16, 8 significant bits, so each product
carries a relative error near 2^-9 per rounding, against the float32 oracle).
"""
import numpy as np
import pytest

import seeded_inputs
from helpers import cosine, rel_max, to_dev
from oracle import vae as V

pytestmark = pytest.mark.gpu

TOL = 2e-2
COS = 0.999
SMALL = dict(block_out_channels=(128, 128, 256, 256), layers_per_block=1)
STAGES = ("conv_in", "mid", "up0", "up1", "up2", "up3")


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _ocfg(c):
    return V.VAEConfig(latent_channels=c.latent_channels, out_channels=c.out_channels,
                       block_out_channels=tuple(c.block_out_channels), layers_per_block=c.layers_per_block,
                       norm_groups=c.norm_groups, norm_eps=float(c.norm_eps), scaling_factor=float(c.scaling_factor))


def _decoder(af, kw, B, h, w):
    _torch()
    m = af.VAEDecoder(af.vae_make_config(max_batch=B, max_latent_h=h, max_latent_w=w, **kw))
    m.load_seeded_weights(threads=16)
    return m


def _weights(ocfg):
    return V.VAEWeights.seeded(ocfg, seeded_inputs.SEED_VAE_WEIGHTS, bf16=True)


def _nchw(x):
    return np.ascontiguousarray(np.asarray(x).transpose(0, 3, 1, 2))


def _level(ocfg, W, l, x):
    """The oracle's up level l (its ResNet blocks, then the upsampling conv) on NCHW x."""
    for r in range(ocfg.layers_per_block + 1):
        x = V.resnet_block(x, W, f"up{l}.res{r}", ocfg, np.float32)
    if l + 1 < len(ocfg.up_channels):
        x = V.conv2d(V.upsample_nearest2x(x), W[f"up{l}.upsample.w"], W[f"up{l}.upsample.b"])
    return x


def _report(name, got, ref):
    e, c = rel_max(got, ref), cosine(got, ref)
    print(f"{name}: rel {e:.3e} cos {c:.6f}", flush=True)
    return name, e, c


def _run_case(af, kw, B, h, w, seed_index):
    torch = _torch()
    m = _decoder(af, kw, B, h, w)
    ocfg = _ocfg(m.cfg)
    lat = seeded_inputs.latents(B, ocfg.latent_channels, h, w, first_index=seed_index)
    d = to_dev(lat)
    got = {i: _nchw(m.decode_taps(d, i).cpu().numpy()) for i in range(6)}
    img = m.decode(d).cpu().numpy()
    img2 = m.decode(d).cpu().numpy()
    torch.cuda.synchronize()
    m.close()
    assert img.shape == (B, ocfg.out_channels, 8 * h, 8 * w) and np.isfinite(img).all()
    np.testing.assert_array_equal(img, img2)
    W = _weights(ocfg)
    taps = {}
    ref = V.decode(ocfg, W, lat, np.float32, taps=lambda n, x: taps.__setitem__(n, x.copy()))
    results = [_report(f"{STAGES[i]} (chain)", got[i], taps[STAGES[i]]) for i in range(6)]
    for l in range(4):
        # got[1 + l] is the input of up level l (the mid block's output for l = 0)
        results.append(_report(f"up{l} (own level)", got[2 + l], _level(ocfg, W, l, got[1 + l])))
    results.append(_report("image", img, ref))
    for name, e, c in results:
        assert e <= TOL and c >= COS, (name, e, c)


def test_small_decoder_every_stage(af):
    """Narrow decoder (widths 128/128/256/256, two ResNet blocks per level), B = 2,
    8 x 8 latents (64 pixels: the attention's keys padded to 128)."""
    _run_case(af, SMALL, 2, 8, 8, 40)


def test_small_decoder_odd_latent_and_batch(af):
    """Narrow decoder, B = 3, a 7 x 9 latent (63 attention keys padded to 128; image 56 x 72,
    so no level's pixel count is a multiple of a GEMM tile or of a GroupNorm chunk)."""
    _run_case(af, SMALL, 3, 7, 9, 70)


def test_full_width_decoder_non_square(af):
    """The default decoder widths (512/512/256/128, three ResNet blocks per level) on
    a 12 x 20 latent (96 x 160 image; 240 attention keys padded to 256), B = 1."""
    _run_case(af, {}, 1, 12, 20, 50)


def test_full_size_mid_block_and_batch_independence(af):
    """1024 x 1024 images (128 x 128 latents), B = 2: the mid block (the attention
    over 16384 pixels) against the oracle for sample 0; the image finite and
    deterministic, and each sample equal bit for bit to its decode alone."""
    torch = _torch()
    B, h, w = 2, 128, 128
    m = _decoder(af, {}, B, h, w)
    ocfg = _ocfg(m.cfg)
    lat = seeded_inputs.latents(B, ocfg.latent_channels, h, w, first_index=60)
    d = to_dev(lat)
    mid = _nchw(m.decode_taps(d, 1).cpu().numpy())
    img = m.decode(d).cpu().numpy()
    img2 = m.decode(d).cpu().numpy()
    alone = m.decode(to_dev(lat[1:2])).cpu().numpy()
    torch.cuda.synchronize()
    m.close()
    assert img.shape == (B, 3, 1024, 1024) and np.isfinite(img).all()
    np.testing.assert_array_equal(img, img2)
    np.testing.assert_array_equal(img[1:2], alone)
    W = _weights(ocfg)
    f = lambda n: W[n]
    z = lat[:1] / np.float32(ocfg.scaling_factor)
    z = V.conv2d(z, f("post_quant.w"), f("post_quant.b"))
    x = V.conv2d(z, f("conv_in.w"), f("conv_in.b"))
    x = V.resnet_block(x, W, "mid.res0", ocfg, np.float32)
    x = V.attention_block(x, W, "mid.attn", ocfg, np.float32)
    x = V.resnet_block(x, W, "mid.res1", ocfg, np.float32)
    name, e, c = _report("1024^2 mid block, sample 0", mid[:1], x)
    assert e <= TOL and c >= COS, (name, e, c)


def test_full_size_image_against_stored_oracle_decode(af):
    """One 1024 x 1024 image (the first latent of the 4-image sampling workload) decoded
    whole on the GPU and compared with the oracle's decode of the same latent, stored in
    tests/golden/vae_oracle.npz (written by tests/golden/make_vae_golden.py from the oracle
    alone): the central 256 x 256 crop, the four 64 x 64 corners (zero-padding edges at
    every level) and the per-channel means of the whole image."""
    import importlib.util
    import os
    torch = _torch()
    here = os.path.dirname(os.path.abspath(__file__))
    spec = importlib.util.spec_from_file_location("mkv", os.path.join(here, "golden", "make_vae_golden.py"))
    mkv = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mkv)
    g = np.load(os.path.join(here, "golden", "vae_oracle.npz"))
    lat = mkv.latent()
    assert float(lat.astype(np.float64).sum()) == float(g["full1024_checksum"])
    m = _decoder(af, {}, 1, 128, 128)
    img = m.decode(to_dev(lat)).cpu().numpy()
    torch.cuda.synchronize()
    m.close()
    c, k, mean = mkv.crops(img)
    results = [_report("1024^2 image, centre 256 x 256", c, g["full1024_center"]),
               _report("1024^2 image, corners", k, g["full1024_corners"])]
    dm = np.abs(mean - g["full1024_mean"]).max() / np.abs(img).max()
    print(f"per-channel means: max difference {dm:.3e} of max|image|", flush=True)
    for name, e, c_ in results:
        assert e <= TOL and c_ >= COS, (name, e, c_)
    assert dm <= TOL


def test_decode_before_the_weights_are_complete(af):
    """A decode before every weight float is loaded returns AF_E_STATE (raised as AfError),
    and succeeds once the rest is loaded."""
    import seeded_inputs as si
    torch = _torch()
    m = af.VAEDecoder(af.vae_make_config(max_batch=1, max_latent_h=8, max_latent_w=8, **SMALL))
    lat = torch.zeros((1, 4, 8, 8), dtype=torch.float32, device="cuda")
    name, rows, cols, off = m.weights[0]
    m.load_weights(si.normal(si.SEED_VAE_WEIGHTS, 0, (rows * cols,), 0.02), off)
    with pytest.raises(af.AfError) as e:
        m.decode(lat)
    assert e.value.status == af.AF_E_STATE
    m.load_seeded_weights(threads=16)
    out = m.decode(lat)
    torch.cuda.synchronize()
    assert np.isfinite(out.cpu().numpy()).all()
    m.close()


def test_decode_argument_errors(af):
    torch = _torch()
    m = _decoder(af, SMALL, 2, 8, 8)
    lat = torch.zeros((3, 4, 8, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        m.decode(lat)                                    # B > max_batch
    with pytest.raises(ValueError):
        m.decode(torch.zeros((1, 4, 8, 9), dtype=torch.float32, device="cuda"))   # w > max_latent_w
    with pytest.raises(ValueError):
        m.decode_taps(torch.zeros((1, 4, 8, 8), dtype=torch.float32, device="cuda"), 6)
    assert m.decode(torch.zeros((0, 4, 8, 8), dtype=torch.float32, device="cuda")).shape == (0, 3, 64, 64)
    m.close()
