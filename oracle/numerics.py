"""bfloat16 rounding for the oracle's mirror of the bf16 path.

On the bf16 path the weights and the KV cache are bfloat16: K and V are
rounded to bfloat16 (round to nearest, ties to even) when they are written to
the cache.  Activations are not rounded (float32 on the GPU, float64 here).
This module is the oracle's own implementation of that rounding.  (The pages
fix no precision; this is the build's reading.)
"""
from __future__ import annotations

import numpy as np


def round_bf16(x) -> np.ndarray:
    """Round to the nearest bfloat16 value (ties to even); returns float64.

    The value is first rounded to float32 (the GPU holds it in float32), then
    the low 16 bits of the float32 pattern are rounded away.  Finite inputs
    only.
    """
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode raw bfloat16 bit patterns (uint16) to float64."""
    u = (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16))
    return u.view(np.float32).astype(np.float64)
