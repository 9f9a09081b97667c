"""bf16 helpers of the oracle (test infrastructure only; see the package docstring).

bf16 is the top half of an IEEE binary32 pattern, so widening is exact.  Narrowing
rounds to nearest-even on the bit pattern (the mode the pages leave open for the
output conversion of the merge kernels: "@mlx-bun/inference 1.0.0" diff page 50,
paged.ts paged_attention_merge and kvq4-decode.ts merge, which convert with a plain
``OutT(num / den)``).  The affine scale is rounded *up* to bf16, the reading this
build takes for the quantizer the pages call but do not show.
"""
from __future__ import annotations

import numpy as np


def to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float32 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def rne(x) -> np.ndarray:
    """Finite float32 values -> nearest bf16 (ties to even), as uint16 bit patterns."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def next_up(bits: np.ndarray) -> np.ndarray:
    """The next bf16 above a finite bf16 value (bit patterns in, bit patterns out)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    neg = (b & 0x8000) != 0
    is_zero = (b & 0x7FFF) == 0
    up = np.where(neg, b - 1, b + 1)
    up = np.where(is_zero, 1, up)          # +-0 -> smallest positive subnormal
    return up.astype(np.uint16)


def roundup(x) -> np.ndarray:
    """Finite float32 values -> the smallest bf16 >= x, as uint16 bit patterns."""
    x32 = np.asarray(x, dtype=np.float32)
    r = rne(x32)
    below = to_f32(r) < x32
    return np.where(below, next_up(r), r).astype(np.uint16)
