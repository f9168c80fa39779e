"""Rounding to the bf16 storage dtype, for intermediates a path stores in bf16.

TEST INFRASTRUCTURE ONLY (see the package docstring).

bf16 keeps the sign, the 8 exponent bits and the top 7 fraction bits of an
IEEE-754 binary32 value. Rounding is to nearest, ties to even, applied to the
value first rounded to binary32 (as a device storing an fp32 accumulator in
bf16 does). Finite inputs only.
"""
from __future__ import annotations

import numpy as np


def round_bf16_ref(x) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even); returns fp64."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lower = u & 0xFFFF
    upper = u >> 16
    round_up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    upper = upper + round_up.astype(np.uint64)
    out = (upper << 16).astype(np.uint32).view(np.float32)
    return out.astype(np.float64)
