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


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with python -m flow_matching_mmdit_amd.build")
    lib = C.CDLL(_LIB_PATH)
    P, I, SZ, F, D, V = C.c_void_p, C.c_int, C.c_size_t, C.c_float, C.c_double, None
    cfgp = C.POINTER(AfConfig)
    ucfgp = C.POINTER(AfUmt5Config)
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
    "af_flow_euler_cfg_step", "af_sigma_schedule", "af_destroy", "af_status_string",
    "af_last_error", "af_umt5_config_default", "af_umt5_weight_count", "af_umt5_weight_info",
    "af_umt5_create", "af_umt5_load_weights", "af_umt5_encode", "af_umt5_encode_taps", "af_umt5_destroy")


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


def af_flow_euler_cfg_step(latents, v, sigma: float, sigma_next: float, guidance: float, stream=None):
    import torch
    assert latents.dtype == torch.float32 and v.dtype == torch.float32
    assert latents.is_contiguous() and v.is_contiguous() and latents.dim() == 4
    Bi, Cc, H, W = latents.shape
    _check(_lib.af_flow_euler_cfg_step(C.c_void_p(latents.data_ptr()), C.c_void_p(v.data_ptr()), Bi, Cc, H, W,
                                       sigma, sigma_next, guidance, _stream_ptr(stream)))


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

    def _common(self, latents, tau, text, mask):
        import torch
        B, Cc, H, W = latents.shape
        T = text.shape[1]
        assert latents.dtype == torch.float32 and latents.is_contiguous() and latents.is_cuda
        assert tau.dtype == torch.float32 and tau.is_contiguous() and tau.numel() == B
        assert text.is_contiguous() and text.shape[0] == B and text.shape[2] == self.cfg.joint_attention_dim
        tdt = AF_BF16 if text.dtype == torch.bfloat16 else AF_F32
        assert text.dtype in (torch.bfloat16, torch.float32)
        mptr = None
        if mask is not None:
            assert mask.dtype == torch.uint8 and mask.is_contiguous() and tuple(mask.shape) == (B, T)
            mptr = C.c_void_p(mask.data_ptr())
        return B, Cc, H, W, T, tdt, mptr

    def forward(self, latents, tau, text, mask=None, out=None, stream=None):
        import torch
        B, Cc, H, W, T, tdt, mptr = self._common(latents, tau, text, mask)
        if out is None:
            out = torch.empty((B, self.cfg.out_channels, H, W), dtype=torch.float32, device=latents.device)
        _check(_lib.af_transformer_forward(self._h, C.c_void_p(latents.data_ptr()), C.c_void_p(tau.data_ptr()),
                                           C.c_void_p(text.data_ptr()), tdt, mptr, B, H, W, T,
                                           C.c_void_p(out.data_ptr()), _stream_ptr(stream)))
        return out

    def forward_taps(self, latents, tau, text, mask=None, stop_after_block: int = 0, out=None, stream=None):
        import torch
        B, Cc, H, W, T, tdt, mptr = self._common(latents, tau, text, mask)
        S = self.cfg.num_register_tokens + T + (H // self.cfg.patch_size) * (W // self.cfg.patch_size)
        if out is None:
            out = torch.empty((B, S, self.inner_dim), dtype=torch.float32, device=latents.device)
        _check(_lib.af_transformer_forward_taps(self._h, C.c_void_p(latents.data_ptr()), C.c_void_p(tau.data_ptr()),
                                                C.c_void_p(text.data_ptr()), tdt, mptr, B, H, W, T,
                                                stop_after_block, C.c_void_p(out.data_ptr()), _stream_ptr(stream)))
        return out

    def sample(self, x, text, mask=None, num_steps: int = 25, shift: float = 1.73, guidance: float = 3.5,
               stream=None):
        """Flow-matching Euler sampling loop with CFG. x: [B', C, H, W] (updated in place);
        text/mask: [2B', ...] = [uncond; cond] when guidance > 1, else [B', ...]."""
        import torch
        sig = af_sigma_schedule(num_steps, shift)
        Bp = x.shape[0]
        cfg_on = guidance > 1.0
        Bt = 2 * Bp if cfg_on else Bp
        xin = torch.empty((Bt,) + tuple(x.shape[1:]), dtype=torch.float32, device=x.device)
        tau = torch.empty(Bt, dtype=torch.float32, device=x.device)
        v = torch.empty_like(xin)
        for i in range(num_steps):
            xin[:Bp].copy_(x)
            if cfg_on:
                xin[Bp:].copy_(x)
            tau.fill_(float(sig[i]))
            self.forward(xin, tau, text, mask, out=v, stream=stream)
            af_flow_euler_cfg_step(x, v, float(sig[i]), float(sig[i + 1]), guidance, stream)
        return x


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
        assert ids.dtype == torch.int32 and ids.is_contiguous() and ids.is_cuda and ids.dim() == 2
        B, T = ids.shape
        mptr = None
        if mask is not None:
            assert mask.dtype == torch.uint8 and mask.is_contiguous() and tuple(mask.shape) == (B, T)
            mptr = C.c_void_p(mask.data_ptr())
        return B, T, mptr

    def encode(self, ids, mask=None, out=None, stream=None):
        import torch
        B, T, mptr = self._args(ids, mask)
        if out is None:
            out = torch.empty((B, T, self.cfg.d_model), dtype=torch.float32, device=ids.device)
        _check(_lib.af_umt5_encode(self._h, C.c_void_p(ids.data_ptr()), mptr, B, T, C.c_void_p(out.data_ptr()),
                                   _stream_ptr(stream)))
        return out

    def encode_taps(self, ids, mask=None, stop_after_layer: int = 0, out=None, stream=None):
        import torch
        B, T, mptr = self._args(ids, mask)
        if out is None:
            out = torch.empty((B, T, self.cfg.d_model), dtype=torch.float32, device=ids.device)
        _check(_lib.af_umt5_encode_taps(self._h, C.c_void_p(ids.data_ptr()), mptr, B, T, stop_after_layer,
                                        C.c_void_p(out.data_ptr()), _stream_ptr(stream)))
        return out
