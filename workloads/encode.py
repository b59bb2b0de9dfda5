"""Storage encoders for synthetic inputs: fp32 -> bf16 and fp32 -> fp8 e4m3.

These only turn generated fp32 draws into the stored form the layer consumes
(bf16 bit patterns, or e4m3 codes plus one fp32 scale per output row).  They
take no part in the layer's arithmetic; decoding belongs to each consumer.

fp8 format: OCP E4M3FN (sign, 4 exponent bits with bias 7, 3 mantissa bits;
no infinities; the all-ones exponent+mantissa pattern is NaN; largest finite
magnitude 448; subnormals step 2**-9).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the uint16 bit patterns.  NaN/Inf inputs are not produced by the
    generators and are not handled specially.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_e4m3(a: np.ndarray) -> np.ndarray:
    """Encode float32 values as OCP e4m3 codes, RNE, saturating at +-448."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    sign = (a.view(np.uint32) >> np.uint32(31)).astype(np.uint8) << np.uint8(7)
    mag = np.minimum(np.abs(a), np.float32(E4M3_MAX))
    u = mag.view(np.uint32)
    # normal range: keep 3 mantissa bits with round-to-nearest-even on the
    # fp32 pattern, then rebias the exponent from 127 to 7 (120 << 3 = 960).
    lsb = (u >> np.uint32(20)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFFF) + lsb) >> np.uint32(20)).astype(np.int64) - 960
    # subnormal range (|a| < 2**-6): multiples of 2**-9, rint is ties-to-even
    sub = np.rint(mag * np.float32(512.0)).astype(np.int64)
    code = np.where(mag < np.float32(2.0 ** -6), sub, r)
    code = np.minimum(code, 0x7E)
    return (code.astype(np.uint8) | sign)


def e4m3_scales(w: np.ndarray) -> np.ndarray:
    """Per-row scale max|w_row| / 448 (rows of an [out, in] matrix); 1 for zero rows."""
    m = np.max(np.abs(w), axis=-1).astype(np.float32)
    s = m / np.float32(E4M3_MAX)
    return np.where(m > 0, s, np.float32(1.0)).astype(np.float32)


def quantize_rows_e4m3(w: np.ndarray):
    """Quantise an [..., out, in] float32 matrix to (codes, per-row scales)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    s = e4m3_scales(w)
    q = f32_to_e4m3(w / s[..., None])
    return q, s
