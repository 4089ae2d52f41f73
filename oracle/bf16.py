"""Exact widening of bfloat16 bit patterns to float64 (oracle side).

A bfloat16 value is the upper 16 bits of an IEEE binary32 value, so shifting
the bits left by 16 and reinterpreting as binary32 gives the value exactly, and
binary32 -> binary64 is exact. The oracle therefore adds no rounding to its
bf16 inputs.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """uint16 array of bf16 bit patterns -> float64 array of the same shape."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
