"""Element formats, decoded exactly (test infrastructure only).

bfloat16 is the upper half of an IEEE-754 binary32: a stored 16-bit pattern
``h`` means the float32 whose bits are ``h << 16``.  Every bf16 value is
therefore exactly representable in float64 and upcasting loses nothing.
"""

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 patterns -> float64 values (exact)."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("bf16 data must be given as uint16 bit patterns")
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 values -> uint16 bf16 patterns, round to nearest, ties to even.

    Adding 0x7FFF plus the lowest kept bit and truncating is the textbook
    integer form of round-half-to-even on the dropped 16 bits.  NaN stays NaN
    (a quiet NaN pattern); infinities stay infinities.
    """
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    return np.where(nan, np.uint16(0x7FC0), rounded).astype(np.uint16)


def to_f64(data: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> float64.  ``dtype`` is 'f32' (float32 values) or
    'bf16' (uint16 patterns)."""
    if dtype == "bf16":
        return bf16_bits_to_f64(data)
    if dtype == "f32":
        data = np.asarray(data)
        if data.dtype != np.float32:
            raise TypeError("f32 data must be float32")
        return data.astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")
