"""Host-side checks of the C-ABI library (no GPU): exported symbols, input
validation, the canonical weight list and the sigma schedule."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(af_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol(af):
    lib = ctypes.CDLL(af._LIB_PATH)
    names = _declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(af.EXPORTED) == names


def _cfg(af, **kw):
    return af.make_config(**kw)


def test_default_config_matches_pages(af):
    c = af.af_config_default()
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "auraflow_config.json")))["default"]
    for k in ("patch_size", "in_channels", "out_channels", "num_mmdit_layers", "num_single_dit_layers",
              "attention_head_dim", "num_attention_heads", "joint_attention_dim", "caption_projection_dim"):
        assert getattr(c, k) == g[k], k
    assert c.pos_embed_max_size == 96 * 96 and c.num_register_tokens == 8


@pytest.mark.parametrize("B,H,W,T,ok", [
    (2, 128, 128, 256, True), (0, 128, 128, 256, True), (2, 128, 128, 0, True), (1, 2, 2, 1, True),
    (2, 127, 128, 256, False), (2, 128, 129, 256, False), (3, 128, 128, 256, False),
    (2, 128, 128, 257, False), (2, 130, 128, 256, False), (-1, 128, 128, 1, False),
])
def test_check_shapes(af, B, H, W, T, ok):
    c = _cfg(af)
    if ok:
        af.af_check_shapes(c, B, H, W, T)
    else:
        with pytest.raises(ValueError):
            af.af_check_shapes(c, B, H, W, T)


def test_check_shapes_grid_limit(af):
    c = _cfg(af, max_latent_h=256, max_latent_w=256)
    af.af_check_shapes(c, 1, 192, 192, 8)                  # 96 x 96 uses the whole PE grid
    with pytest.raises(ValueError, match="position"):
        af.af_check_shapes(c, 1, 194, 64, 8)               # 97 rows of patches > 96


@pytest.mark.parametrize("field,value,status", [
    ("caption_projection_dim", 2048, 2), ("pos_embed_max_size", 9000, 2), ("attention_head_dim", 128, 3),
    ("compute_dtype", 7, 1), ("num_attention_heads", 0, 1), ("ln_eps", 0.0, 1),
])
def test_config_errors(af, field, value, status):
    c = _cfg(af, **{field: value})
    if field == "attention_head_dim":
        c.caption_projection_dim = c.num_attention_heads * value
    with pytest.raises(ValueError) as e:
        af.af_check_shapes(c, 1, 64, 64, 8)
    assert e.value.status == status
    assert af._lib.af_last_error().decode() != ""


def test_fp32_path_limits(af):
    c = _cfg(af, compute_dtype=af.AF_F32, num_attention_heads=4, attention_head_dim=8,
             caption_projection_dim=32, joint_attention_dim=32, pos_embed_max_size=64)
    af.af_check_shapes(c, 1, 16, 16, 8)
    c.attention_head_dim, c.caption_projection_dim = 128, 512
    with pytest.raises(ValueError):
        af.af_check_shapes(c, 1, 16, 16, 8)


def _oracle_cfg(c):
    return oracle.AuraFlowConfig(
        in_channels=c.in_channels, out_channels=c.out_channels, patch_size=c.patch_size,
        num_mmdit_layers=c.num_mmdit_layers, num_single_dit_layers=c.num_single_dit_layers,
        num_attention_heads=c.num_attention_heads, attention_head_dim=c.attention_head_dim,
        joint_attention_dim=c.joint_attention_dim, caption_projection_dim=c.caption_projection_dim,
        pos_embed_max_size=c.pos_embed_max_size, num_register_tokens=c.num_register_tokens)


@pytest.mark.parametrize("kw", [
    dict(),
    dict(num_mmdit_layers=1, num_single_dit_layers=1),
    dict(compute_dtype=0, num_attention_heads=4, attention_head_dim=8, caption_projection_dim=32,
         joint_attention_dim=32, pos_embed_max_size=64, num_mmdit_layers=1, num_single_dit_layers=1),
])
def test_weight_list_matches_oracle_list(af, kw):
    c = _cfg(af, **kw)
    n, total = af.af_weight_count(c)
    specs = oracle.weight_specs(_oracle_cfg(c))
    assert n == len(specs)
    off = 0
    for i, (name, shape, _std) in enumerate(specs):
        lname, rows, cols, loff = af.af_weight_info(c, i)
        assert lname == name
        assert (rows, cols) == (shape[0], shape[1] if len(shape) > 1 else 1)
        assert loff == off
        off += int(np.prod(shape))
    assert total == off == oracle.count_parameters(_oracle_cfg(c))
    # The synthetic init scale is part of the input recipe; both sides agree on it.
    for name, _shape, std in specs:
        assert af.weight_std(name) == std


def test_sigma_schedule_library(af):
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "sigma_schedule.json")))
    s = af.af_sigma_schedule(4, 1.73)
    assert s[0] == 1.0 and s[-1] == 0.0
    assert abs(s[2] - g["sigma_at_u"]["0.5"]) < 1e-7 and abs(s[3] - g["sigma_at_u"]["0.25"]) < 1e-7
    np.testing.assert_allclose(af.af_sigma_schedule(25, 1.73), oracle.sigma_schedule(25, 1.73), atol=1e-7)
    with pytest.raises(ValueError):
        af.af_sigma_schedule(0, 1.73)
    with pytest.raises(ValueError):
        af.af_sigma_schedule(5, -1.0)


def test_euler_step_argument_errors_without_device(af):
    lib = af._lib
    assert lib.af_flow_euler_cfg_step(None, None, 0, 4, 8, 8, 1.0, 0.5, 3.5, None) == af.AF_OK   # empty
    assert lib.af_flow_euler_cfg_step(None, None, -1, 4, 8, 8, 1.0, 0.5, 3.5, None) == af.AF_E_INVALID_ARG
    assert lib.af_flow_euler_cfg_step(None, None, 1, 4, 8, 8, 1.0, 0.5, 3.5, None) == af.AF_E_INVALID_ARG
    assert lib.af_status_string(af.AF_E_SHAPE) == b"shape error"


def test_forward_rejects_null_model(af):
    lib = af._lib
    st = lib.af_transformer_forward(None, None, None, None, 0, None, 1, 16, 16, 8, None, None)
    assert st == af.AF_E_INVALID_ARG
    assert b"model" in lib.af_last_error()


def test_mxfp8_config_checks(af):
    # host-only: the MXFP8 compute type is accepted with the bf16 constraints
    af.af_check_shapes(af.make_config(compute_dtype=af.AF_MXFP8), 2, 128, 128, 256)
    with pytest.raises(ValueError):
        af.af_check_shapes(af.make_config(compute_dtype=3), 2, 128, 128, 256)
    with pytest.raises(ValueError):   # head dim other than 256 is not built for the bf16 / MXFP8 paths
        af.af_check_shapes(af.make_config(compute_dtype=af.AF_MXFP8, attention_head_dim=128,
                                          caption_projection_dim=1536), 2, 128, 128, 256)


# ----------------------------------------------------------------------------- text encoder (UMT5)

def test_umt5_weight_list_matches_oracle(af):
    from oracle import umt5 as U
    for ocfg, kw in ((U.UMT5_FULL, {}), (U.UMT5_SMALL, dict(d_model=256, num_heads=4, num_layers=2, d_ff=512,
                                                            vocab_size=1000))):
        cfg = af.umt5_make_config(**kw)
        n, total = af.af_umt5_weight_count(cfg)
        specs = U.umt5_weight_specs(ocfg)
        assert n == len(specs)
        off = 0
        for i, (name, shape, std, mean) in enumerate(specs):
            nm, r, c, o = af.af_umt5_weight_info(cfg, i)
            assert nm == name and o == off, (i, nm, name)
            assert (r, c) == (shape[0], shape[1] if len(shape) > 1 else 1)
            assert af.umt5_weight_recipe(nm) == (std, mean), nm
            off += int(np.prod(shape))
        assert total == off


@pytest.mark.parametrize("kw", [dict(num_heads=16), dict(d_model=2176, num_heads=34), dict(d_ff=5000),
                                dict(rel_buckets=64), dict(rel_max_distance=64), dict(max_tokens=513),
                                dict(eps=0.0), dict(vocab_size=0)])
def test_umt5_config_checks(af, kw):
    with pytest.raises(ValueError):
        af.af_umt5_weight_count(af.umt5_make_config(**kw))


def test_umt5_default_config_matches_pages(af):
    c = af.umt5_make_config()
    # [DEEP] 2.1 文本编码器: d_model 2048, 32 heads, 24 layers, d_ff 5120, vocab 32128, max distance 128
    assert (c.d_model, c.num_heads, c.num_layers, c.d_ff, c.vocab_size, c.rel_max_distance) == \
        (2048, 32, 24, 5120, 32128, 128)


# ----------------------------------------------------------------------------- binding argument checks
# Each bad argument raises ValueError in the binding, before the library is
# called (CPU tensors stand in; no model handle and no device are needed).

def _good(af, B=2, T=16, H=32, W=32):
    import torch
    cfg = _cfg(af)
    lat = torch.zeros((B, 4, H, W), dtype=torch.float32)
    tau = torch.zeros(B, dtype=torch.float32)
    text = torch.zeros((B, T, cfg.joint_attention_dim), dtype=torch.bfloat16)
    mask = torch.ones((B, T), dtype=torch.uint8)
    out = torch.zeros((B, 4, H, W), dtype=torch.float32)
    return cfg, lat, tau, text, mask, out


@pytest.mark.parametrize("bad", ["tau_len", "tau_dtype", "text_dim", "text_batch", "text_dtype", "mask_shape",
                                 "mask_dtype", "out_shape", "out_dtype", "lat_channels", "lat_rank", "noncontig"])
def test_forward_tensor_checks_raise_before_launch(af, bad):
    import torch
    cfg, lat, tau, text, mask, out = _good(af)
    if bad == "tau_len": tau = torch.zeros(3)
    if bad == "tau_dtype": tau = tau.double()
    if bad == "text_dim": text = torch.zeros((2, 16, 1024), dtype=torch.bfloat16)
    if bad == "text_batch": text = torch.zeros((1, 16, 2048), dtype=torch.bfloat16)
    if bad == "text_dtype": text = text.half()
    if bad == "mask_shape": mask = torch.ones((2, 15), dtype=torch.uint8)
    if bad == "mask_dtype": mask = mask.bool()
    if bad == "out_shape": out = torch.zeros((2, 4, 32, 16))
    if bad == "out_dtype": out = out.half()
    if bad == "lat_channels": lat = torch.zeros((2, 3, 32, 32))
    if bad == "lat_rank": lat = torch.zeros((2, 4, 32))
    if bad == "noncontig": lat = torch.zeros((2, 4, 32, 64))[..., ::2]
    with pytest.raises(ValueError) as e:
        af.check_forward_tensors(cfg, 0, lat, tau, text, mask, out, (2, 4, 32, 32))
    assert "cuda" not in str(e.value), e.value   # a shape/dtype error, reported before the device check


@pytest.mark.parametrize("where", ["latents", "tau", "text", "mask", "out"])
def test_forward_tensor_checks_reject_host_tensors(af, where):
    """Well-formed arguments that are not on the model's device are refused (a host
    pointer handed to a kernel would fault the GPU)."""
    cfg, lat, tau, text, mask, out = _good(af)
    with pytest.raises(ValueError, match="must be a tensor on cuda:0") as e:
        af.check_forward_tensors(cfg, 0, lat, tau, text, mask, out, (2, 4, 32, 32))
    assert "latents" in str(e.value)             # the first tensor checked is named


def test_euler_and_cfg_input_wrappers_check_sizes_before_launch(af):
    import torch
    x = torch.zeros((2, 4, 8, 8))
    with pytest.raises(ValueError, match="v must hold 2"):
        af.af_flow_euler_cfg_step(x, torch.zeros((2, 4, 8, 8)), 1.0, 0.5, 3.5)      # CFG needs [uncond; cond]
    with pytest.raises(ValueError, match="v must hold 1"):
        af.af_flow_euler_cfg_step(x, torch.zeros((4, 4, 8, 8)), 1.0, 0.5, 1.0)
    with pytest.raises(ValueError, match="must be a tensor on cuda"):
        af.af_flow_euler_cfg_step(x, torch.zeros((4, 4, 8, 8)), 1.0, 0.5, 3.5)      # sizes fine, host memory
    with pytest.raises(ValueError, match="x_in must be"):
        af.af_flow_cfg_inputs(x, 0.5, True, torch.zeros((2, 4, 8, 8)), torch.zeros(4))
    with pytest.raises(ValueError, match="tau must hold"):
        af.af_flow_cfg_inputs(x, 0.5, True, torch.zeros((4, 4, 8, 8)), torch.zeros(2))
    with pytest.raises(ValueError, match="must be a tensor on cuda"):
        af.af_flow_cfg_inputs(x, 0.5, False, torch.zeros((2, 4, 8, 8)), torch.zeros(2))


def test_cfg_inputs_library_argument_errors_without_device(af):
    """The library's own checks (NULL pointers, negative sizes, non-finite sigma,
    overlapping buffers) reject before anything is enqueued."""
    import ctypes as C
    lib = af._lib
    assert lib.af_flow_cfg_inputs(None, 0, 4, 8, 8, 0.5, 1, None, None, None) == af.AF_OK       # Bi = 0: no-op
    assert lib.af_flow_cfg_inputs(None, 1, 4, 8, 8, 0.5, 1, None, None, None) == af.AF_E_INVALID_ARG
    assert lib.af_flow_cfg_inputs(C.c_void_p(256), -1, 4, 8, 8, 0.5, 1, C.c_void_p(4096), C.c_void_p(8192),
                                  None) == af.AF_E_INVALID_ARG
    assert lib.af_flow_cfg_inputs(C.c_void_p(256), 1, 4, 8, 8, float("nan"), 1, C.c_void_p(1 << 20),
                                  C.c_void_p(1 << 21), None) == af.AF_E_INVALID_ARG
    # x_in starting inside latents (256 floats each) overlaps
    assert lib.af_flow_cfg_inputs(C.c_void_p(4096), 1, 4, 8, 8, 0.5, 0, C.c_void_p(4096 + 512), C.c_void_p(1 << 21),
                                  None) == af.AF_E_INVALID_ARG
    assert "overlaps" in af._lib.af_last_error().decode()


# ----------------------------------------------------------------------------- VAE decoder

def _vae_oracle_cfg(c):
    from oracle import vae as V
    return V.VAEConfig(latent_channels=c.latent_channels, out_channels=c.out_channels,
                       block_out_channels=tuple(c.block_out_channels), layers_per_block=c.layers_per_block,
                       norm_groups=c.norm_groups, norm_eps=float(c.norm_eps), scaling_factor=float(c.scaling_factor))


@pytest.mark.parametrize("kw", [{}, dict(block_out_channels=(128, 128, 256, 256), layers_per_block=1)])
def test_vae_weight_list_matches_oracle(af, kw):
    """Same names, element counts, order and init recipe as the oracle's decoder list, so
    seeded weights drawn per index are the same tensors on both sides."""
    from oracle import vae as V
    cfg = af.vae_make_config(**kw)
    specs = V.vae_weight_specs(_vae_oracle_cfg(cfg))
    n, total = af.af_vae_weight_count(cfg)
    assert n == len(specs)
    off = 0
    for i, (name, shape, kind) in enumerate(specs):
        nm, r, c, o = af.af_vae_weight_info(cfg, i)
        assert nm == name and o == off, (i, nm, name)
        assert r == shape[0] and r * c == int(np.prod(shape)), (nm, r, c, shape)
        assert af.vae_weight_recipe(nm) == V.vae_weight_recipe(kind), nm
        off += int(np.prod(shape))
    assert total == off


def test_vae_default_config_matches_oracle_reading(af):
    from oracle import vae as V
    c = af.vae_make_config()
    o = V.VAE_FULL
    assert (c.latent_channels, c.out_channels, tuple(c.block_out_channels), c.layers_per_block, c.norm_groups) == \
        (o.latent_channels, o.out_channels, o.block_out_channels, o.layers_per_block, o.norm_groups)
    assert c.norm_eps == np.float32(o.norm_eps) and c.scaling_factor == np.float32(o.scaling_factor)
    assert (c.max_batch, c.max_latent_h, c.max_latent_w) == (4, 128, 128)


@pytest.mark.parametrize("kw", [dict(block_out_channels=(128, 256, 512, 500)), dict(norm_groups=16),
                                dict(latent_channels=33), dict(out_channels=5), dict(norm_eps=0.0),
                                dict(scaling_factor=0.0), dict(block_out_channels=(128, 256, 512, 1152)),
                                dict(max_batch=-1)])
def test_vae_config_checks(af, kw):
    with pytest.raises(ValueError):
        af.af_vae_weight_count(af.vae_make_config(**kw))


def test_vae_decode_rejects_null_model(af):
    assert af._lib.af_vae_decode(None, None, 1, 8, 8, None, None) == af.AF_E_INVALID_ARG
    assert af._lib.af_vae_decode_taps(None, None, 1, 8, 8, 0, None, None) == af.AF_E_INVALID_ARG
