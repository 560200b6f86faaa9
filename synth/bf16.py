"""fp32 -> bf16 rounding (round to nearest, ties to even) as raw uint16 bits.

Both sides receive the same bf16 bit patterns, so the input rounding is never
a parity term.  Only finite inputs are expected (Gaussian draws).
"""

import numpy as np


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (RNE) and return the uint16 bit patterns."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if not np.all(np.isfinite(a)):
        raise ValueError("bf16 conversion expects finite values")
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)
