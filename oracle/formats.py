"""Storage formats of the weight-quantized linear layer, decoded bit by bit.

Test infrastructure (see the package docstring): the HIP library never imports
this module.

Formats, as the pages name them:

* ``float8_e4m3fn`` weights and block scales (fp8_gemv page, summary and
  "Structure" paragraphs; fp4_matmul page, summary; Matmul2dFp8 page, the
  ``b_type`` member).  The pages give only the dtype name.  Reading taken: the
  OCP 8-bit E4M3 "FN" encoding -- 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits, subnormals at exponent field 0, no infinities, NaN only
  where exponent and mantissa fields are all ones (0x7F, 0xFF).
* packed NVFP4 E2M1 nibbles (fp4_matmul page, summary): ``uint8 [N, K//2]``,
  "lo-nibble".  Reading taken: byte j of a row holds k = 2j in bits 0..3 and
  k = 2j+1 in bits 4..7.  E2M1 = 1 sign bit (bit 3), 2 exponent bits with
  bias 1, 1 mantissa bit, subnormal at exponent field 0, no NaN/inf.
* ``bfloat16`` activations and outputs: the upper 16 bits of an IEEE binary32.

All decodes return float64 arrays, which hold every value of these formats
exactly.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "e4m3_to_f64",
    "e2m1_to_f64",
    "unpack_nibbles",
    "bf16_bits_to_f64",
    "f64_to_bf16_bits",
    "round_to_precision",
    "f64_to_e4m3_codes",
    "BF16_MAX",
    "E4M3_MAX",
]


def e4m3_to_f64(codes) -> np.ndarray:
    """Decode float8_e4m3fn bytes to float64, field by field.

    value = (-1)^s * 2^(e-7) * (1 + m/8)   for exponent field e in 1..15,
    value = (-1)^s * 2^-6 * (m/8)          for e = 0 (subnormal),
    NaN                                    for e = 15 and m = 7.
    The largest finite magnitude is 2^8 * 1.75 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = c >> 7
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp((8 + m).astype(np.float64), (e - 10).astype(np.int64))  # (1+m/8)*2^(e-7)
    subnormal = np.ldexp(m.astype(np.float64), -9)                            # (m/8)*2^-6
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e2m1_to_f64(nibbles) -> np.ndarray:
    """Decode 4-bit E2M1 codes (values 0..15) to float64, field by field.

    value = (-1)^s * 2^(e-1) * (1 + m/2)   for exponent field e in 1..3,
    value = (-1)^s * m/2                   for e = 0 (subnormal).
    Magnitudes by code 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6.
    """
    c = np.asarray(nibbles).astype(np.int64)
    if np.any((c < 0) | (c > 15)):
        raise ValueError("E2M1 codes are 4-bit")
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    normal = np.ldexp((2 + m).astype(np.float64), (e - 2).astype(np.int64))  # (1+m/2)*2^(e-1)
    subnormal = m.astype(np.float64) * 0.5
    mag = np.where(e == 0, subnormal, normal)
    return np.where(s == 1, -mag, mag)


def unpack_nibbles(packed) -> np.ndarray:
    """Unpack ``uint8 [..., K//2]`` into E2M1 codes ``[..., K]``.

    Byte j carries element k = 2j in its low nibble and k = 2j+1 in its high
    nibble (fp4_matmul page, summary: "uint8 [N, K//2] lo-nibble").
    """
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64: the bits are the top half of
    an IEEE binary32, so shifting them up 16 places gives that binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


# Largest finite bfloat16: (2 - 2^-7) * 2^127.
BF16_MAX = float(np.ldexp(2.0 - 2.0 ** -7, 127))


def round_to_precision(x, p: int, emin: int) -> np.ndarray:
    """Round float64 values to the nearest number with ``p`` significant bits
    whose exponent is at least ``emin`` (so subnormals are rounded on the grid
    2^(emin-p+1)), ties to even.  No overflow handling: the caller does that.

    Works by scaling each value so that one unit in the last place of the
    target grid is 1.0 (a power-of-two scaling, exact in float64) and calling
    ``np.rint``, which rounds half to even.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    sel = np.isfinite(x) & (x != 0)
    if np.any(sel):
        v = x[sel]
        _, E = np.frexp(v)                 # v = f * 2^E, 0.5 <= |f| < 1
        e = np.maximum(E - 1, emin)        # exponent of the leading bit, floored at emin
        shift = e - (p - 1)                # exponent of one ulp
        out[sel] = np.ldexp(np.rint(np.ldexp(v, -shift)), shift)
    return out


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bfloat16 (round to nearest, ties to even) in ONE
    rounding and return the bit patterns as uint16.

    bfloat16: 8 significant bits, minimum normal exponent -126, overflow to
    +-inf at and above (2 - 2^-8) * 2^127, NaN returned as the quiet 0x7FC0
    (sign kept).  Rounding straight from float64 avoids the double rounding of
    going through binary32 first.
    """
    x = np.asarray(x, dtype=np.float64)
    r = round_to_precision(x, 8, -126)
    r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, r), r)
    f32 = r.astype(np.float32)            # exact: r has <= 8 significant bits and is in range
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if np.any(nan):
        sign = (np.signbit(x) & nan).astype(np.uint16) << np.uint16(15)
        bits = np.where(nan, np.uint16(0x7FC0) | sign, bits)
    return bits.astype(np.uint16)


# Largest finite float8_e4m3fn magnitude: 1.75 * 2^8.
E4M3_MAX = 448.0


def f64_to_e4m3_codes(x) -> np.ndarray:
    """Round float64 values to float8_e4m3fn (round to nearest, ties to even)
    in one rounding and return the codes as uint8, field by field.

    4 significant bits, minimum normal exponent -6 (subnormals on the grid
    2^-9), sign kept (-0.0 and negative values that round to zero give 0x80).
    Magnitudes beyond 448 saturate to 448; the caller clamps in the precision
    it works in.  NaN is not accepted.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.isnan(x)):
        raise ValueError("NaN has no saturating E4M3 code here")
    r = round_to_precision(np.clip(x, -E4M3_MAX, E4M3_MAX), 4, -6)
    mag = np.abs(r)
    sign = np.signbit(r).astype(np.int64) << 7
    _, E = np.frexp(np.where(mag > 0, mag, 1.0))        # mag = f * 2^E, 0.5 <= f < 1
    e = E - 1                                            # exponent of the leading bit
    normal = mag >= 2.0 ** -6
    field_e = np.where(normal, e + 7, 0)
    mant = np.where(normal, np.ldexp(mag, -e) - 1.0, np.ldexp(mag, 9))   # 1.m -> m in [0,1); subnormal: m/8 * 2^-6
    field_m = np.where(normal, np.rint(mant * 8.0), np.rint(mant)).astype(np.int64)
    return (sign | (field_e.astype(np.int64) << 3) | field_m).astype(np.uint8)
