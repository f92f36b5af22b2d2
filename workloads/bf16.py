"""bfloat16 storage helpers (NumPy has no bf16 dtype).

bf16 values are kept as uint16 bit patterns. Rounding from float32 is
round-to-nearest-even on the upper 16 bits, which is also what PyTorch's
float32 -> bfloat16 cast does for finite values and infinities.
"""
from __future__ import annotations

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even); return the uint16 bit patterns."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    with np.errstate(over="ignore"):
        rounded = bits + np.uint32(0x7FFF) + lsb
    is_nan = np.isnan(np.asarray(x, dtype=np.float32))
    out = (rounded >> np.uint32(16)).astype(np.uint16)
    out[is_nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bf16, returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))
