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


def f64_to_bf16_bits(x):
    """float64 array -> uint16 bf16 bit patterns, rounded to nearest, ties to even,
    directly from the float64 value (one rounding). Values whose magnitude rounds
    past the largest bf16 become infinities; values below the smallest normal
    bfloat16 (2^-126) are rounded through binary32 (not reached by the callers)."""
    x = np.asarray(x, dtype=np.float64)
    bits = x.view(np.uint64).copy()
    # keep 7 of the 52 fraction bits: add half an ulp minus one plus the lowest kept
    # bit (ties to even), then clear the dropped bits
    keep = (bits >> np.uint64(45)) & np.uint64(1)
    bits = (bits + np.uint64((1 << 44) - 1) + keep) & ~np.uint64((1 << 45) - 1)
    r = bits.view(np.float64)
    small = np.abs(x) < 2.0 ** -126
    with np.errstate(over="ignore"):
        r32 = np.where(small, x, r).astype(np.float32)
    out = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out = np.where(nan, np.uint16(0x7FC0), out)
    return out
