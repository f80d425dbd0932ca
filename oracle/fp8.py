"""FP8 payload for the MoE dispatch (oracle side).

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this package; the product path never does.

"Networks and Collective Communication", section 7.4: DeepSeek-V3 sends the
dispatch all-to-all in FP8 and keeps the combine in BF16. The pages name the
format only; the readings taken here:

R15  element format: FP8 E4M3 with no infinities (the OCP 8-bit E4M3
     encoding, also gfx950's native FP8): sign bit, 4 exponent bits with bias
     7, 3 mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6;
     S.1111.111 is NaN; the largest finite value is 1.75 * 2^8 = 448.
     Rounding to nearest, ties to even.
R16  scaling: every row is cut into groups of 128 consecutive elements; a
     group's scale is the power of two 2^k with k the smallest integer such
     that amax <= 448 * 2^k (amax = largest finite |x| of the group), k
     clamped to [-126, 126], and 2^0 for a group with no non-zero finite
     value. The code of x is E4M3(x * 2^-k); a power-of-two scale makes the
     product exact for every normal result and needs no saturation.
     Non-finite inputs (none occur in the workloads) encode as NaN, 0x7F.
R17  row layout: a row of H elements (H a multiple of 128) travels as H code
     bytes followed by H/128 float32 scales (little-endian), H + H/32 bytes.
"""
from __future__ import annotations

import numpy as np

GROUP = 128
MAX_E4M3 = 448.0


def row_bytes(hidden: int) -> int:
    return hidden + 4 * (hidden // GROUP)


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """float32 values with |y| <= 448 (or non-finite) -> E4M3 codes (uint8),
    round to nearest even, from the format's definition (R15)."""
    y = np.asarray(y, dtype=np.float32)
    out = np.zeros(y.shape, dtype=np.uint8)
    sign = (np.signbit(y)).astype(np.uint8) << 7
    a = np.abs(y).astype(np.float64)                 # exact copy of the float32 magnitude
    finite = np.isfinite(y)
    nz = finite & (a > 0)
    # binade of a: a in [2^e, 2^(e+1))
    e = np.zeros(y.shape, dtype=np.int64)
    e[nz] = np.floor(np.log2(a[nz])).astype(np.int64)
    # guard against log2 rounding at exact powers of two
    lo = nz & (a < np.ldexp(1.0, e))
    e[lo] -= 1
    hi = nz & (a >= np.ldexp(1.0, e + 1))
    e[hi] += 1
    sub = nz & (e < -6)
    nor = nz & (e >= -6)
    code = np.zeros(y.shape, dtype=np.int64)
    # subnormals (and the step up to 2^-6): multiples of 2^-9
    code[sub] = np.rint(np.ldexp(a[sub], 9)).astype(np.int64)       # 0..8; 8 is 2^-6, field 1 / mant 0
    # normals: 1.mmm * 2^e -> q = a / 2^(e-3) in [8, 16]
    q = np.rint(np.ldexp(a[nor], -(e[nor] - 3))).astype(np.int64)
    en = e[nor].copy()
    carry = q == 16
    q[carry] = 8
    en[carry] += 1
    code[nor] = ((en + 7) << 3) | (q - 8)
    out[:] = code.astype(np.uint8)
    out |= sign
    out[~finite] = 0x7F
    return out


def e4m3_decode(c: np.ndarray) -> np.ndarray:
    """E4M3 codes -> float32 values (R15)."""
    c = np.asarray(c, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = c & 7
    val = np.where(ef == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, ef - 7))
    val = s * val
    val[(c & 0x7F) == 0x7F] = np.nan
    return val.astype(np.float32)


def group_exponent(amax: float) -> int:
    """R16: smallest k with amax <= 448 * 2^k, clamped; 0 for amax == 0."""
    amax = float(amax)                               # exact; compare in float64
    if amax == 0:
        return 0
    k = int(np.ceil(np.log2(amax / MAX_E4M3)))
    while amax > MAX_E4M3 * 2.0 ** k:               # correct any log2 rounding
        k += 1
    while k > -126 and amax <= MAX_E4M3 * 2.0 ** (k - 1):
        k -= 1
    return max(-126, min(126, k))


def quantize_rows(x: np.ndarray) -> np.ndarray:
    """float32 rows [R, H] -> byte rows [R, H + H/32] (R16, R17)."""
    x = np.asarray(x, dtype=np.float32)
    R, H = x.shape
    if H % GROUP:
        raise ValueError("hidden size must be a multiple of 128")
    G = H // GROUP
    out = np.zeros((R, row_bytes(H)), dtype=np.uint8)
    scales = np.zeros((R, G), dtype=np.float32)
    for r in range(R):
        for g in range(G):
            v = x[r, g * GROUP:(g + 1) * GROUP]
            fin = v[np.isfinite(v)]
            amax = float(np.max(np.abs(fin))) if fin.size else 0.0
            k = group_exponent(amax)
            y = v * np.float32(2.0 ** -k)             # exact power-of-two scaling in float32
            out[r, g * GROUP:(g + 1) * GROUP] = e4m3_encode(y)
            scales[r, g] = np.float32(2.0 ** k)
    out[:, H:] = scales.view(np.uint8).reshape(R, 4 * G)
    return out


def dequantize_rows(b: np.ndarray, hidden: int) -> np.ndarray:
    """Byte rows -> float32 rows: code value times its group's scale."""
    b = np.asarray(b, dtype=np.uint8)
    R = b.shape[0]
    G = hidden // GROUP
    codes = e4m3_decode(b[:, :hidden]).reshape(R, G, GROUP)
    scales = np.ascontiguousarray(b[:, hidden:]).view(np.float32).reshape(R, G, 1)
    return (codes * scales).reshape(R, hidden).astype(np.float32)
