"""bfloat16 storage with float32 arithmetic, written from the IEEE-754 definitions.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this package; the product path never does.

bfloat16 is the upper half of a binary32 word (1 sign, 8 exponent, 7
fraction bits), so widening is exact: the 16 bits move to the top of a 32-bit
word. Narrowing rounds the dropped 16 bits to nearest, ties to even, which on
the bit pattern of a finite value is: add 0x7FFF plus the lowest kept bit,
then shift right by 16 (a carry out of the fraction bumps the exponent, and
the largest finite values round to infinity exactly as IEEE rounding does).
A NaN is kept a NaN: its sign and top payload bits are kept and the quiet bit
is set.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of uint16 bfloat16 patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    is_nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    quiet = ((u >> np.uint64(16)) | np.uint64(0x0040)) & np.uint64(0xFFFF)
    return np.where(is_nan, quiet, rounded).astype(np.uint16)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value, returned as float32 (exactly representable)."""
    return bf16_to_f32(f32_to_bf16(x))


ELEM_BYTES = {"f32": 4, "bf16": 2, "u8": 1}         # u8: raw bytes (all-to-all payloads only)


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage values -> float32 working values."""
    if dtype == "f32":
        return np.array(x, dtype=np.float32, copy=True)
    if dtype == "bf16":
        return bf16_to_f32(x)
    raise ValueError(dtype)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 working values that are already representable -> storage values."""
    if dtype == "f32":
        return np.array(x, dtype=np.float32, copy=True)
    return f32_to_bf16(x)
