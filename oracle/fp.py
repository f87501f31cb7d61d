"""Floating-point rounding helpers for the oracle (test infrastructure only).

numpy has IEEE fp16 with round-to-nearest-even casts but no bfloat16, so the
fp32 -> bf16 rounding is written out on the bit pattern: add 0x7FFF plus the
lowest kept bit, then truncate (round half to even).  NaN inputs map to a quiet
NaN of the same sign.  This is the textbook definition; it is pinned in
``tests/test_oracle_fp.py`` against torch's CPU bfloat16 conversion.
"""

import numpy as np


def f32_to_bf16_bits(a):
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(np.asarray(a, dtype=np.float32))
    if np.any(nan):
        sign = ((u >> np.uint64(16)) & np.uint64(0x8000)).astype(np.uint16)
        r = np.where(nan, sign | np.uint16(0x7FC0), r).astype(np.uint16)
    return r


def bf16_bits_to_f32(b):
    """Exact widening of bf16 bit patterns (uint16) to fp32 values."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_f16(a):
    """Round fp32 values to fp16 (numpy's cast is IEEE round-to-nearest-even;
    magnitudes past the fp16 range become infinities)."""
    with np.errstate(over="ignore"):
        return np.asarray(a, dtype=np.float32).astype(np.float16)


def round_to(a32, dtype):
    """Round fp32 values to the 16-bit type named by ``dtype`` ("f16" | "bf16").

    Returns uint16 bit patterns for both types so callers can compare bits.
    """
    if dtype == "f16":
        return f32_to_f16(a32).view(np.uint16)
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    raise ValueError(dtype)


def bits_to_f64(bits, dtype):
    """Exact value of 16-bit patterns of ``dtype`` as fp64."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f32(bits).astype(np.float64)
    raise ValueError(dtype)
