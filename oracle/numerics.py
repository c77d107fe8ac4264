"""bfloat16 and MXFP8 rounding for the oracle (TEST INFRASTRUCTURE ONLY).

Weights (the position table excepted) and text embeddings are rounded to
bfloat16 with round-to-nearest-even before the oracle computes in float32; the
GPU path stores the same tensors in bfloat16. bfloat16 is the top 16 bits of an
IEEE float32, so RNE rounding adds 0x7FFF plus the lowest kept bit to the 32-bit
pattern and truncates. NaN is not expected in inputs and is not special-cased.
"""
from __future__ import annotations

import numpy as np


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    r &= np.uint32(0xFFFF0000)
    return r.view(np.float32)


# ----------------------------------------------------------------------------- MXFP8
# Microscaling FP8 (the OCP "MX" block format with E4M3 elements): every 32
# consecutive values along the contraction axis share one power-of-two scale
# X = 2^(floor(log2(amax)) - 8), amax being the block's largest magnitude and 8
# the exponent of E4M3's largest normal (448 = 1.75 * 2^8); an all-zero block
# takes X = 2^-127. Elements are v / X clamped to [-448, 448] and rounded to
# the nearest E4M3 value, ties to the even code. The scale exponent is kept in
# [-127, 127] (an 8-bit biased exponent).

E4M3_MAX = 448.0


def round_e4m3(x: np.ndarray) -> np.ndarray:
    """Round float32 values in [-448, 448] to the nearest OCP E4M3 value (ties to
    even); returns float32. Normal values (|x| >= 2^-6) keep 3 mantissa bits;
    below that the grid is uniform with step 2^-9."""
    x = np.asarray(x, dtype=np.float32)
    ax = np.abs(x).astype(np.float64)
    # exponent of the grid step at |x|: 2^(e - 3) for |x| in [2^e, 2^(e+1)), e >= -6
    e = np.frexp(np.where(ax > 0, ax, 1.0))[1] - 1.0     # floor(log2 |x|), exact
    e = np.maximum(e, -6.0)
    step = np.exp2(e - 3.0)
    r = np.rint(ax / step) * step            # np.rint rounds half to even
    return (np.sign(x) * r).astype(np.float32)


def mxfp8_qdq(x: np.ndarray, block: int = 32) -> np.ndarray:
    """Quantize to MXFP8 along the last axis and dequantize (float32 result)."""
    x = np.asarray(x, dtype=np.float32)
    K = x.shape[-1]
    assert K % block == 0, "last axis must be a multiple of the block size"
    xb = x.reshape(x.shape[:-1] + (K // block, block))
    amax = np.abs(xb).max(axis=-1, keepdims=True).astype(np.float64)
    E = np.frexp(np.where(amax > 0, amax, 1.0))[1] - 1.0   # floor(log2 amax), exact
    e = np.where(amax > 0, E - 8.0, -127.0)
    e = np.clip(e, -127.0, 127.0)
    v = np.clip(xb.astype(np.float64) * np.exp2(-e), -E4M3_MAX, E4M3_MAX).astype(np.float32)
    q = round_e4m3(v).astype(np.float64) * np.exp2(e)
    return q.astype(np.float32).reshape(x.shape)
