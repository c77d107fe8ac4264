"""ctypes binding of libauraflow.so: the C-ABI calls under the same names, plus a
small ``AuraFlowModel`` wrapper that marshals torch tensors (device memory and
the current HIP stream) into them. No arithmetic of the model happens here;
every step runs in the library's HIP kernels.

The library must have been built (``python -m flow_matching_mmdit_amd.build``);
importing this module without it raises ImportError.
"""
from __future__ import annotations

import ctypes as C
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
# torch first: its HIP runtime (same soname as /opt/rocm's) then serves the
# library too, so device pointers and streams from torch tensors are valid in it.
import torch  # noqa: F401

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libauraflow.so")

AF_OK, AF_E_INVALID_ARG, AF_E_SHAPE, AF_E_UNSUPPORTED, AF_E_OOM, AF_E_HIP, AF_E_STATE = range(7)
AF_F32, AF_BF16, AF_MXFP8 = 0, 1, 2


class AfConfig(C.Structure):
    _fields_ = [
        ("in_channels", C.c_int), ("out_channels", C.c_int), ("patch_size", C.c_int),
        ("num_mmdit_layers", C.c_int), ("num_single_dit_layers", C.c_int),
        ("num_attention_heads", C.c_int), ("attention_head_dim", C.c_int),
        ("joint_attention_dim", C.c_int), ("caption_projection_dim", C.c_int),
        ("pos_embed_max_size", C.c_int), ("num_register_tokens", C.c_int),
        ("compute_dtype", C.c_int), ("ln_eps", C.c_float), ("timestep_scale", C.c_float),
        ("max_batch", C.c_int), ("max_latent_h", C.c_int), ("max_latent_w", C.c_int),
        ("max_text_len", C.c_int),
    ]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class AfUmt5Config(C.Structure):
    _fields_ = [
        ("d_model", C.c_int), ("num_heads", C.c_int), ("num_layers", C.c_int), ("d_ff", C.c_int),
        ("vocab_size", C.c_int), ("rel_buckets", C.c_int), ("rel_max_distance", C.c_int), ("eps", C.c_float),
        ("max_batch", C.c_int), ("max_tokens", C.c_int),
    ]


class AfVaeConfig(C.Structure):
    _fields_ = [
        ("latent_channels", C.c_int), ("out_channels", C.c_int), ("block_out_channels", C.c_int * 4),
        ("layers_per_block", C.c_int), ("norm_groups", C.c_int), ("norm_eps", C.c_float),
        ("scaling_factor", C.c_float), ("max_batch", C.c_int), ("max_latent_h", C.c_int), ("max_latent_w", C.c_int),
    ]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with python -m flow_matching_mmdit_amd.build")
    lib = C.CDLL(_LIB_PATH)
    P, I, SZ, F, D, V = C.c_void_p, C.c_int, C.c_size_t, C.c_float, C.c_double, None
    cfgp = C.POINTER(AfConfig)
    ucfgp = C.POINTER(AfUmt5Config)
    vcfgp = C.POINTER(AfVaeConfig)
    sig = {
        "af_config_default": (I, [cfgp]),
        "af_check_shapes": (I, [cfgp, I, I, I, I]),
        "af_weight_count": (I, [cfgp, C.POINTER(I), C.POINTER(SZ)]),
        "af_weight_info": (I, [cfgp, I, C.c_char_p, I, C.POINTER(C.c_int64), C.POINTER(C.c_int64), C.POINTER(SZ)]),
        "af_create": (I, [cfgp, I, C.POINTER(P)]),
        "af_load_weights": (I, [P, P, SZ, SZ, P]),
        "af_init_weights": (I, [P, P, SZ, P]),
        "af_transformer_forward": (I, [P, P, P, P, I, P, I, I, I, I, P, P]),
        "af_transformer_forward_taps": (I, [P, P, P, P, I, P, I, I, I, I, I, P, P]),
        "af_flow_euler_cfg_step": (I, [P, P, I, I, I, I, F, F, F, P]),
        "af_flow_cfg_inputs": (I, [P, I, I, I, I, F, I, P, P, P]),
        "af_attention_workspace_size": (SZ, [I, I, I, I]),
        "af_attention": (I, [P, P, P, P, I, I, I, I, F, P, P, SZ, P]),
        "af_attention_noalloc": (I, [P, P, P, P, I, I, I, I, F, P, P]),
        "af_attention_noalloc_max_bytes": (SZ, []),
        "af_sigma_schedule": (I, [I, D, C.POINTER(F)]),
        "af_destroy": (V, [P]),
        "af_status_string": (C.c_char_p, [I]),
        "af_last_error": (C.c_char_p, []),
        "af_umt5_config_default": (I, [ucfgp]),
        "af_umt5_weight_count": (I, [ucfgp, C.POINTER(I), C.POINTER(SZ)]),
        "af_umt5_weight_info": (I, [ucfgp, I, C.c_char_p, I, C.POINTER(C.c_int64), C.POINTER(C.c_int64),
                                    C.POINTER(SZ)]),
        "af_umt5_create": (I, [ucfgp, I, C.POINTER(P)]),
        "af_umt5_load_weights": (I, [P, P, SZ, SZ, P]),
        "af_umt5_encode": (I, [P, P, P, I, I, P, P]),
        "af_umt5_encode_taps": (I, [P, P, P, I, I, I, P, P]),
        "af_umt5_destroy": (V, [P]),
        "af_vae_config_default": (I, [vcfgp]),
        "af_vae_weight_count": (I, [vcfgp, C.POINTER(I), C.POINTER(SZ)]),
        "af_vae_weight_info": (I, [vcfgp, I, C.c_char_p, I, C.POINTER(C.c_int64), C.POINTER(C.c_int64),
                                   C.POINTER(SZ)]),
        "af_vae_create": (I, [vcfgp, I, C.POINTER(P)]),
        "af_vae_load_weights": (I, [P, P, SZ, SZ, P]),
        "af_vae_decode": (I, [P, P, I, I, I, P, P]),
        "af_vae_decode_taps": (I, [P, P, I, I, I, I, P, P]),
        "af_vae_destroy": (V, [P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
EXPORTED = (
    "af_config_default", "af_check_shapes", "af_weight_count", "af_weight_info", "af_create",
    "af_load_weights", "af_init_weights", "af_transformer_forward", "af_transformer_forward_taps",
    "af_flow_euler_cfg_step", "af_flow_cfg_inputs", "af_attention_workspace_size", "af_attention",
    "af_attention_noalloc", "af_attention_noalloc_max_bytes",
    "af_sigma_schedule", "af_destroy", "af_status_string",
    "af_last_error", "af_umt5_config_default", "af_umt5_weight_count", "af_umt5_weight_info",
    "af_umt5_create", "af_umt5_load_weights", "af_umt5_encode", "af_umt5_encode_taps", "af_umt5_destroy",
    "af_vae_config_default", "af_vae_weight_count", "af_vae_weight_info", "af_vae_create", "af_vae_load_weights",
    "af_vae_decode", "af_vae_decode_taps", "af_vae_destroy")


class AfError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_lib.af_status_string(status).decode()}: {msg}")
        self.status = status


def _check(status):
    if status != AF_OK:
        msg = _lib.af_last_error().decode()
        if status in (AF_E_INVALID_ARG, AF_E_SHAPE, AF_E_UNSUPPORTED):
            e = ValueError(f"{_lib.af_status_string(status).decode()}: {msg}")
            e.status = status
            raise e
        raise AfError(status, msg)


# ----------------------------------------------------------------------------- plain C-ABI calls

def af_config_default() -> AfConfig:
    c = AfConfig()
    _check(_lib.af_config_default(C.byref(c)))
    return c


def af_check_shapes(cfg: AfConfig, B: int, H: int, W: int, T: int) -> None:
    _check(_lib.af_check_shapes(C.byref(cfg), B, H, W, T))


def af_weight_count(cfg: AfConfig):
    n, tot = C.c_int(), C.c_size_t()
    _check(_lib.af_weight_count(C.byref(cfg), C.byref(n), C.byref(tot)))
    return n.value, tot.value


def af_weight_info(cfg: AfConfig, index: int):
    name = C.create_string_buffer(128)
    r, c, o = C.c_int64(), C.c_int64(), C.c_size_t()
    _check(_lib.af_weight_info(C.byref(cfg), index, name, 128, C.byref(r), C.byref(c), C.byref(o)))
    return name.value.decode(), r.value, c.value, o.value


def af_sigma_schedule(num_steps: int, shift: float) -> np.ndarray:
    out = (C.c_float * (num_steps + 1))()
    _check(_lib.af_sigma_schedule(num_steps, shift, out))
    return np.frombuffer(out, dtype=np.float32).copy()


def _need(cond, msg):
    """Argument check on the host, before anything is enqueued (a failed check
    raises ValueError, as the library's own shape errors do)."""
    if not cond:
        raise ValueError(msg)


def _on_device(t, name, device):
    _need(t.is_cuda and (device is None or t.device.index == device),
          f"{name} must be a tensor on cuda:{'' if device is None else device}")


def af_flow_euler_cfg_step(latents, v, sigma: float, sigma_next: float, guidance: float, stream=None):
    """x <- x + (sigma_next - sigma) * v_hat in place; v holds [uncond; cond] (2 Bi
    samples) when guidance > 1, else Bi samples."""
    import torch
    _need(latents.dtype == torch.float32 and v.dtype == torch.float32, "latents and v must be float32")
    _need(latents.is_contiguous() and v.is_contiguous(), "latents and v must be contiguous")
    _need(latents.dim() == 4, "latents must be [Bi, C, H, W]")
    per = 2 if guidance > 1.0 else 1
    _need(v.numel() == per * latents.numel(),
          f"v must hold {per} x latents.numel() values (guidance {guidance})")
    _on_device(latents, "latents", None)
    _on_device(v, "v", latents.device.index)
    Bi, Cc, H, W = latents.shape
    _check(_lib.af_flow_euler_cfg_step(C.c_void_p(latents.data_ptr()), C.c_void_p(v.data_ptr()), Bi, Cc, H, W,
                                       sigma, sigma_next, guidance, _stream_ptr(stream)))


def af_flow_cfg_inputs(latents, sigma: float, cfg_on: bool, x_in, tau, stream=None):
    """x_in = [latents; latents] (cfg_on) or latents, tau[:] = sigma (one CFG step's
    transformer inputs)."""
    import torch
    _need(latents.dtype == torch.float32 and x_in.dtype == torch.float32 and tau.dtype == torch.float32,
          "latents, x_in and tau must be float32")
    _need(latents.is_contiguous() and x_in.is_contiguous() and tau.is_contiguous(), "tensors must be contiguous")
    _need(latents.dim() == 4, "latents must be [Bi, C, H, W]")
    per = 2 if cfg_on else 1
    Bi, Cc, H, W = latents.shape
    _need(tuple(x_in.shape) == (per * Bi, Cc, H, W), "x_in must be [(2 if cfg_on else 1) * Bi, C, H, W]")
    _need(tau.numel() == per * Bi, "tau must hold one value per x_in sample")
    _on_device(latents, "latents", None)
    for t, name in ((x_in, "x_in"), (tau, "tau")):
        _on_device(t, name, latents.device.index)
    _check(_lib.af_flow_cfg_inputs(C.c_void_p(latents.data_ptr()), Bi, Cc, H, W, sigma, 1 if cfg_on else 0,
                                   C.c_void_p(x_in.data_ptr()), C.c_void_p(tau.data_ptr()), _stream_ptr(stream)))


def af_attention_workspace_size(B: int, S: int, H: int, head_dim: int = 256) -> int:
    return int(_lib.af_attention_workspace_size(B, S, H, head_dim))


def _attention_args(q, k, v, key_mask, num_heads, out):
    import torch
    _need(q.dim() == 3 and q.shape == k.shape == v.shape, "q, k, v must be [B, S, H * head_dim] of one shape")
    _need(all(t.dtype == torch.bfloat16 and t.is_contiguous() for t in (q, k, v)),
          "q, k, v must be contiguous bfloat16")
    B, S, D = q.shape
    _need(num_heads > 0 and D % num_heads == 0, "H * head_dim must equal the last dimension")
    if key_mask is not None:
        _need(key_mask.dtype == torch.uint8 and key_mask.is_contiguous() and tuple(key_mask.shape) == (B, S),
              "key_mask must be contiguous uint8 [B, S]")
    if out is not None:
        _need(out.dtype == torch.bfloat16 and out.is_contiguous() and out.shape == q.shape,
              "out must be contiguous bfloat16 of q's shape")
    _on_device(q, "q", None)
    for t, name in ((k, "k"), (v, "v"), (key_mask, "key_mask"), (out, "out")):
        if t is not None:
            _on_device(t, name, q.device.index)
    return B, S, D // num_heads


def af_attention(q, k, v, key_mask=None, num_heads: int = 12, eps: float = 1e-6, out=None, workspace=None,
                 stream=None):
    """QK-norm + joint attention on token-major bf16 q, k, v [B, S, H * 256] -> out of
    the same shape. `workspace` (a uint8 device tensor) is allocated here when not
    given."""
    import torch
    B, S, hd = _attention_args(q, k, v, key_mask, num_heads, out)
    if out is None:
        out = torch.empty_like(q)
    need = af_attention_workspace_size(B, S, num_heads, hd)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _need(workspace.dtype == torch.uint8 and workspace.is_contiguous(), "workspace must be a contiguous uint8 tensor")
    _on_device(workspace, "workspace", q.device.index)
    mptr = C.c_void_p(key_mask.data_ptr()) if key_mask is not None else None
    _check(_lib.af_attention(C.c_void_p(q.data_ptr()), C.c_void_p(k.data_ptr()), C.c_void_p(v.data_ptr()), mptr,
                             B, S, num_heads, hd, eps, C.c_void_p(out.data_ptr()),
                             C.c_void_p(workspace.data_ptr()), workspace.numel(), _stream_ptr(stream)))
    return out


def af_attention_noalloc(q, k, v, key_mask=None, num_heads: int = 12, eps: float = 1e-6, out=None, stream=None):
    """af_attention with the library's fixed per-device scratch: the call itself
    allocates nothing on the device (pass `out` to allocate nothing here either)."""
    import torch
    B, S, hd = _attention_args(q, k, v, key_mask, num_heads, out)
    if out is None:
        out = torch.empty_like(q)
    mptr = C.c_void_p(key_mask.data_ptr()) if key_mask is not None else None
    _check(_lib.af_attention_noalloc(C.c_void_p(q.data_ptr()), C.c_void_p(k.data_ptr()), C.c_void_p(v.data_ptr()),
                                     mptr, B, S, num_heads, hd, eps, C.c_void_p(out.data_ptr()), _stream_ptr(stream)))
    return out


def af_attention_noalloc_max_bytes() -> int:
    return int(_lib.af_attention_noalloc_max_bytes())


def _stream_ptr(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


# ----------------------------------------------------------------------------- model wrapper

def make_config(**kw) -> AfConfig:
    """Full AuraFlow defaults with any field overridden by keyword."""
    c = af_config_default()
    for k, v in kw.items():
        if not hasattr(c, k):
            raise KeyError(k)
        setattr(c, k, v)
    return c


def weight_std(name: str) -> float:
    """Synthetic init recipe: position table N(0, 0.1), every other tensor N(0, 0.02)."""
    return 0.1 if name == "pos_embed" else 0.02


class AuraFlowModel:
    """One model handle on one device; tensors in, tensors out."""

    def __init__(self, cfg: AfConfig, device: int = 0):
        self.cfg = cfg
        self.device = device
        h = C.c_void_p()
        _check(_lib.af_create(C.byref(cfg), device, C.byref(h)))
        self._h = h
        n, total = af_weight_count(cfg)
        self.weights = [af_weight_info(cfg, i) for i in range(n)]
        self.total_floats = total

    def close(self):
        if getattr(self, "_h", None):
            _lib.af_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def inner_dim(self):
        return self.cfg.num_attention_heads * self.cfg.attention_head_dim

    def load_weights(self, host: np.ndarray, offset: int = 0, stream=None):
        a = np.ascontiguousarray(host, dtype=np.float32).ravel()
        _check(_lib.af_load_weights(self._h, C.c_void_p(a.ctypes.data), offset, a.size, _stream_ptr(stream)))

    def load_seeded_weights(self, seed: int = 0, overrides: dict | None = None, threads: int = 8):
        """Draws every canonical tensor from seeded_inputs (stream (seed, index)) and loads it."""
        import seeded_inputs
        overrides = overrides or {}

        def draw(i):
            name, rows, cols, off = self.weights[i]
            if name in overrides:
                a = np.asarray(overrides[name], np.float32).reshape(rows * cols)
            else:
                a = seeded_inputs.normal(seed, i, (rows, cols) if cols > 1 else (rows,), weight_std(name))
            return off, a

        # Bounded window of tensors in flight: the full model is ~27 GB as fp32.
        n = len(self.weights)
        win = 2 * max(1, threads)
        with ThreadPoolExecutor(max(1, threads)) as ex:
            for w0 in range(0, n, win):
                for off, a in ex.map(draw, range(w0, min(n, w0 + win))):
                    self.load_weights(a, off)

    def _common(self, latents, tau, text, mask, out=None, out_shape=None):
        """Host-side checks of the tensor arguments (dtype, layout, shape, device)
        before anything is enqueued; returns the ABI's size arguments."""
        return check_forward_tensors(self.cfg, self.device, latents, tau, text, mask, out, out_shape)

    def forward(self, latents, tau, text, mask=None, out=None, stream=None):
        import torch
        B, Cc, H, W = latents.shape if latents.dim() == 4 else (0, 0, 0, 0)
        oshape = (B, self.cfg.out_channels, H, W)
        B, Cc, H, W, T, tdt, mptr = self._common(latents, tau, text, mask, out, oshape)
        if out is None:
            out = torch.empty(oshape, dtype=torch.float32, device=latents.device)
        _check(_lib.af_transformer_forward(self._h, C.c_void_p(latents.data_ptr()), C.c_void_p(tau.data_ptr()),
                                           C.c_void_p(text.data_ptr()), tdt, mptr, B, H, W, T,
                                           C.c_void_p(out.data_ptr()), _stream_ptr(stream)))
        return out

    def forward_taps(self, latents, tau, text, mask=None, stop_after_block: int = 0, out=None, stream=None):
        import torch
        _need(latents.dim() == 4 and text.dim() == 3, "latents must be [B, C, H, W] and text [B, T, D]")
        B, Cc, H, W = latents.shape
        S = self.cfg.num_register_tokens + text.shape[1] + (H // self.cfg.patch_size) * (W // self.cfg.patch_size)
        oshape = (B, S, self.inner_dim)
        B, Cc, H, W, T, tdt, mptr = self._common(latents, tau, text, mask, out, oshape)
        if out is None:
            out = torch.empty(oshape, dtype=torch.float32, device=latents.device)
        _check(_lib.af_transformer_forward_taps(self._h, C.c_void_p(latents.data_ptr()), C.c_void_p(tau.data_ptr()),
                                                C.c_void_p(text.data_ptr()), tdt, mptr, B, H, W, T,
                                                stop_after_block, C.c_void_p(out.data_ptr()), _stream_ptr(stream)))
        return out

    def sample(self, x, text, mask=None, num_steps: int = 25, shift: float = 1.73, guidance: float = 3.5,
               stream=None):
        """Flow-matching Euler sampling loop with CFG. x: [B', C, H, W] (updated in place);
        text/mask: [2B', ...] = [uncond; cond] when guidance > 1, else [B', ...].
        Every step runs as three library calls on one stream: the step's inputs
        (latents duplicated for CFG, tau = sigma_i), the forward and the CFG + Euler
        update. With `stream` given, the buffers are also allocated on it."""
        import contextlib
        import torch
        sig = af_sigma_schedule(num_steps, shift)
        Bp = x.shape[0]
        cfg_on = guidance > 1.0
        Bt = 2 * Bp if cfg_on else Bp
        _need(text.shape[0] == Bt, f"text must hold {Bt} rows ([uncond; cond] when guidance > 1)")
        ctx = torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()
        with ctx:
            s = torch.cuda.current_stream()
            xin = torch.empty((Bt,) + tuple(x.shape[1:]), dtype=torch.float32, device=x.device)
            tau = torch.empty(Bt, dtype=torch.float32, device=x.device)
            v = torch.empty_like(xin)
            for i in range(num_steps):
                af_flow_cfg_inputs(x, float(sig[i]), cfg_on, xin, tau, stream=s)
                self.forward(xin, tau, text, mask, out=v, stream=s)
                af_flow_euler_cfg_step(x, v, float(sig[i]), float(sig[i + 1]), guidance, stream=s)
        return x


def check_forward_tensors(cfg: AfConfig, device: int, latents, tau, text, mask=None, out=None, out_shape=None):
    """Checks the tensor arguments of a forward against the model's config: dtype,
    contiguity and shape of every tensor first, then that every tensor (out
    included) lives on cuda:`device`. Raises ValueError before anything is
    enqueued; returns (B, C, H, W, T, text dtype code, mask pointer or None)."""
    import torch
    _need(latents.dim() == 4, "latents must be [B, C, H, W]")
    B, Cc, H, W = latents.shape
    _need(latents.dtype == torch.float32 and latents.is_contiguous(), "latents must be contiguous float32")
    _need(Cc == cfg.in_channels, f"latents must have {cfg.in_channels} channels")
    _need(tau.dtype == torch.float32 and tau.is_contiguous() and tau.numel() == B,
          "tau must be contiguous float32 with one value per sample")
    _need(text.dim() == 3 and text.shape[0] == B and text.shape[2] == cfg.joint_attention_dim,
          f"text must be [B, T, {cfg.joint_attention_dim}]")
    _need(text.dtype in (torch.bfloat16, torch.float32) and text.is_contiguous(),
          "text must be contiguous bfloat16 or float32")
    T = text.shape[1]
    if mask is not None:
        _need(mask.dtype == torch.uint8 and mask.is_contiguous() and tuple(mask.shape) == (B, T),
              "mask must be contiguous uint8 [B, T]")
    if out is not None:
        _need(out.dtype == torch.float32 and out.is_contiguous(), "out must be contiguous float32")
        _need(out_shape is None or tuple(out.shape) == tuple(out_shape), f"out must have shape {tuple(out_shape)}")
    named = [(latents, "latents"), (tau, "tau"), (text, "text")]
    if mask is not None:
        named.append((mask, "mask"))
    if out is not None:
        named.append((out, "out"))
    for t, name in named:
        _on_device(t, name, device)
    tdt = AF_BF16 if text.dtype == torch.bfloat16 else AF_F32
    mptr = C.c_void_p(mask.data_ptr()) if mask is not None else None
    return B, Cc, H, W, T, tdt, mptr


# ----------------------------------------------------------------------------- diagnostics
AF_K_NAMES = ("gemm_qkv", "gemm_out", "gemm_ffn_up", "gemm_ffn_down", "attention", "ln_modulate",
              "adaln", "embed", "final")

_lib.af_profile.restype = C.c_int
_lib.af_profile.argtypes = [C.c_void_p, C.c_int]
_lib.af_profile_read.restype = C.c_int
_lib.af_profile_read.argtypes = [C.c_void_p, C.c_int, C.POINTER(C.c_double), C.POINTER(C.c_int64)]
EXPORTED = EXPORTED + ("af_profile", "af_profile_read")


def af_profile(model: "AuraFlowModel", enable: bool) -> None:
    _check(_lib.af_profile(model._h, 1 if enable else 0))


def af_profile_read(model: "AuraFlowModel") -> dict:
    """{class name: (total kernel ms, launches)} since the last af_profile(model, True)."""
    out = {}
    for i, name in enumerate(AF_K_NAMES):
        ms, n = C.c_double(), C.c_int64()
        _check(_lib.af_profile_read(model._h, i, C.byref(ms), C.byref(n)))
        out[name] = (ms.value, n.value)
    return out


# ----------------------------------------------------------------------------- text encoder (UMT5)

def umt5_make_config(**kw) -> AfUmt5Config:
    """The pages' encoder configuration with any field overridden by keyword."""
    c = AfUmt5Config()
    _check(_lib.af_umt5_config_default(C.byref(c)))
    for k, v in kw.items():
        if not hasattr(c, k):
            raise KeyError(k)
        setattr(c, k, v)
    return c


def af_umt5_weight_count(cfg: AfUmt5Config):
    n, tot = C.c_int(), C.c_size_t()
    _check(_lib.af_umt5_weight_count(C.byref(cfg), C.byref(n), C.byref(tot)))
    return n.value, tot.value


def af_umt5_weight_info(cfg: AfUmt5Config, index: int):
    name = C.create_string_buffer(128)
    r, c, o = C.c_int64(), C.c_int64(), C.c_size_t()
    _check(_lib.af_umt5_weight_info(C.byref(cfg), index, name, 128, C.byref(r), C.byref(c), C.byref(o)))
    return name.value.decode(), r.value, c.value, o.value


def umt5_weight_recipe(name: str):
    """Synthetic init recipe (std, mean): embedding N(0, 1); norm weights N(1, 0.1^2);
    q and k projections N(0, 0.01^2); relative-position tables N(0, 0.5^2); every
    other matrix N(0, 0.02^2)."""
    t = name.split(".")[-1]
    if t == "embed":
        return 1.0, 0.0
    if t in ("ln1", "ln2", "final_ln"):
        return 0.1, 1.0
    if t in ("wq", "wk"):
        return 0.01, 0.0
    if t == "rel_bias":
        return 0.5, 0.0
    return 0.02, 0.0


class UMT5Encoder:
    """One text-encoder handle on one device; token ids in, embeddings out."""

    def __init__(self, cfg: AfUmt5Config, device: int = 0):
        self.cfg = cfg
        self.device = device
        h = C.c_void_p()
        _check(_lib.af_umt5_create(C.byref(cfg), device, C.byref(h)))
        self._h = h
        n, total = af_umt5_weight_count(cfg)
        self.weights = [af_umt5_weight_info(cfg, i) for i in range(n)]
        self.total_floats = total

    def close(self):
        if getattr(self, "_h", None):
            _lib.af_umt5_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def load_weights(self, host: np.ndarray, offset: int = 0, stream=None):
        a = np.ascontiguousarray(host, dtype=np.float32).ravel()
        _check(_lib.af_umt5_load_weights(self._h, C.c_void_p(a.ctypes.data), offset, a.size, _stream_ptr(stream)))

    def load_seeded_weights(self, seed: int | None = None, threads: int = 8):
        """Draws every canonical tensor from seeded_inputs (stream (seed, index)) and loads it."""
        import seeded_inputs
        seed = seeded_inputs.SEED_ENCODER_WEIGHTS if seed is None else seed

        def draw(i):
            name, rows, cols, off = self.weights[i]
            std, mean = umt5_weight_recipe(name)
            return off, seeded_inputs.normal(seed, i, (rows, cols) if cols > 1 else (rows,), std, mean)

        n = len(self.weights)
        win = 2 * max(1, threads)
        with ThreadPoolExecutor(max(1, threads)) as ex:
            for w0 in range(0, n, win):
                for off, a in ex.map(draw, range(w0, min(n, w0 + win))):
                    self.load_weights(a, off)

    def _args(self, ids, mask):
        import torch
        _need(ids.dtype == torch.int32 and ids.is_contiguous() and ids.dim() == 2, "ids must be contiguous int32 [B, T]")
        B, T = ids.shape
        mptr = None
        if mask is not None:
            _need(mask.dtype == torch.uint8 and mask.is_contiguous() and tuple(mask.shape) == (B, T),
                  "mask must be contiguous uint8 [B, T]")
            mptr = C.c_void_p(mask.data_ptr())
        _on_device(ids, "ids", self.device)
        if mask is not None:
            _on_device(mask, "mask", self.device)
        return B, T, mptr

    def _check_out(self, out, B, T):
        import torch
        _need(out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (B, T, self.cfg.d_model),
              "out must be contiguous float32 [B, T, d_model]")
        _on_device(out, "out", self.device)

    def encode(self, ids, mask=None, out=None, stream=None):
        import torch
        B, T, mptr = self._args(ids, mask)
        if out is None:
            out = torch.empty((B, T, self.cfg.d_model), dtype=torch.float32, device=ids.device)
        self._check_out(out, B, T)
        _check(_lib.af_umt5_encode(self._h, C.c_void_p(ids.data_ptr()), mptr, B, T, C.c_void_p(out.data_ptr()),
                                   _stream_ptr(stream)))
        return out

    def encode_taps(self, ids, mask=None, stop_after_layer: int = 0, out=None, stream=None):
        import torch
        B, T, mptr = self._args(ids, mask)
        if out is None:
            out = torch.empty((B, T, self.cfg.d_model), dtype=torch.float32, device=ids.device)
        self._check_out(out, B, T)
        _check(_lib.af_umt5_encode_taps(self._h, C.c_void_p(ids.data_ptr()), mptr, B, T, stop_after_layer,
                                        C.c_void_p(out.data_ptr()), _stream_ptr(stream)))
        return out


# ----------------------------------------------------------------------------- VAE decode

def vae_make_config(**kw) -> AfVaeConfig:
    """The AutoencoderKL decoder defaults with any field overridden by keyword
    (block_out_channels as a 4-sequence)."""
    c = AfVaeConfig()
    _check(_lib.af_vae_config_default(C.byref(c)))
    for k, v in kw.items():
        if not hasattr(c, k):
            raise KeyError(k)
        if k == "block_out_channels":
            v = (C.c_int * 4)(*v)
        setattr(c, k, v)
    return c


def af_vae_weight_count(cfg: AfVaeConfig):
    n, tot = C.c_int(), C.c_size_t()
    _check(_lib.af_vae_weight_count(C.byref(cfg), C.byref(n), C.byref(tot)))
    return n.value, tot.value


def af_vae_weight_info(cfg: AfVaeConfig, index: int):
    name = C.create_string_buffer(128)
    r, c, o = C.c_int64(), C.c_int64(), C.c_size_t()
    _check(_lib.af_vae_weight_info(C.byref(cfg), index, name, 128, C.byref(r), C.byref(c), C.byref(o)))
    return name.value.decode(), r.value, c.value, o.value


def vae_weight_recipe(name: str):
    """Synthetic init (std, mean) by the tensor's suffix: kernels, matrices (.w) and
    biases (.b) N(0, 0.02^2); GroupNorm scales (.g) N(1, 0.1^2); GroupNorm shifts
    (.n) N(0, 0.02^2)."""
    return {"w": (0.02, 0.0), "b": (0.02, 0.0), "g": (0.1, 1.0), "n": (0.02, 0.0)}[name.rsplit(".", 1)[1]]


class VAEDecoder:
    """One VAE-decoder handle on one device; latents in, images out."""

    def __init__(self, cfg: AfVaeConfig, device: int = 0):
        self.cfg = cfg
        self.device = device
        h = C.c_void_p()
        _check(_lib.af_vae_create(C.byref(cfg), device, C.byref(h)))
        self._h = h
        n, total = af_vae_weight_count(cfg)
        self.weights = [af_vae_weight_info(cfg, i) for i in range(n)]
        self.total_floats = total

    def close(self):
        if getattr(self, "_h", None):
            _lib.af_vae_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def load_weights(self, host: np.ndarray, offset: int = 0, stream=None):
        a = np.ascontiguousarray(host, dtype=np.float32).ravel()
        _check(_lib.af_vae_load_weights(self._h, C.c_void_p(a.ctypes.data), offset, a.size, _stream_ptr(stream)))

    def load_seeded_weights(self, seed: int | None = None, threads: int = 8):
        """Draws every canonical tensor from seeded_inputs (stream (seed, index)) and loads it."""
        import seeded_inputs
        seed = seeded_inputs.SEED_VAE_WEIGHTS if seed is None else seed

        def draw(i):
            name, rows, cols, off = self.weights[i]
            std, mean = vae_weight_recipe(name)
            return off, seeded_inputs.normal(seed, i, (rows * cols,), std, mean)

        n = len(self.weights)
        win = 2 * max(1, threads)
        with ThreadPoolExecutor(max(1, threads)) as ex:
            for w0 in range(0, n, win):
                for off, a in ex.map(draw, range(w0, min(n, w0 + win))):
                    self.load_weights(a, off)

    def _args(self, latents, out, out_shape):
        import torch
        _need(latents.dtype == torch.float32 and latents.is_contiguous() and latents.dim() == 4
              and latents.shape[1] == self.cfg.latent_channels,
              "latents must be contiguous float32 [B, latent_channels, h, w]")
        if out is not None:
            _need(out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == tuple(out_shape),
                  f"out must be contiguous float32 {list(out_shape)}")
        _on_device(latents, "latents", self.device)
        if out is not None:
            _on_device(out, "out", self.device)
        B, _, h, w = latents.shape
        return B, h, w

    def decode(self, latents, out=None, stream=None):
        """latents [B, latent_channels, h, w] -> image [B, out_channels, 8h, 8w] (fp32)."""
        import torch
        B, _, h, w = latents.shape if latents.dim() == 4 else (0, 0, 0, 0)
        shape = (B, self.cfg.out_channels, 8 * h, 8 * w)
        B, h, w = self._args(latents, out, shape)
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=latents.device)
        _check(_lib.af_vae_decode(self._h, C.c_void_p(latents.data_ptr()), B, h, w, C.c_void_p(out.data_ptr()),
                                  _stream_ptr(stream)))
        return out

    def tap_shape(self, B: int, h: int, w: int, stop_after: int):
        """NHWC shape of the activation af_vae_decode_taps writes after stage stop_after."""
        ch = list(self.cfg.block_out_channels)[::-1]
        if stop_after <= 1:
            return (B, h, w, ch[0])
        lvl = stop_after - 2
        f = 2 ** min(lvl + 1, 3)
        return (B, f * h, f * w, ch[lvl])

    def decode_taps(self, latents, stop_after: int, out=None, stream=None):
        """The fp32 NHWC activation after stage stop_after (0 conv_in, 1 mid, 2 + l up level l)."""
        import torch
        _need(0 <= stop_after <= 5, "stop_after must be in 0 .. 5")
        B, _, h, w = latents.shape if latents.dim() == 4 else (0, 0, 0, 0)
        shape = self.tap_shape(B, h, w, stop_after)
        B, h, w = self._args(latents, out, shape)
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=latents.device)
        _check(_lib.af_vae_decode_taps(self._h, C.c_void_p(latents.data_ptr()), B, h, w, stop_after,
                                       C.c_void_p(out.data_ptr()), _stream_ptr(stream)))
        return out
