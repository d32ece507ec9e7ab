"""Number formats used by the oracle.

bfloat16 is the top 16 bits of an IEEE float32.  Rounding a float32 to bfloat16 here
is round-to-nearest, ties to even, on the bit pattern: add 0x7FFF plus the lowest kept
bit, then drop the low 16 bits.  NaN stays NaN.  The result is returned as float32
(or float64) values that are exactly representable in bfloat16.
"""
from __future__ import annotations

import numpy as np


def round_bf16(x) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even).  float64 input is first rounded to
    float32 (the kernels hold the value in float32 before narrowing it)."""
    a = np.asarray(x)
    f = a.astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    out = (r & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32)
    out = np.where(np.isnan(f), np.float32(np.nan), out)
    return out.astype(a.dtype if a.dtype in (np.float32, np.float64) else np.float32)


def round_f32(x) -> np.ndarray:
    """Round to float32 and carry the result in float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    return (np.asarray(u16, dtype=np.uint32) << np.uint32(16)).view(np.float32)
