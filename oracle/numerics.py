"""bfloat16 rounding for the oracle's inputs (TEST INFRASTRUCTURE ONLY).

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
