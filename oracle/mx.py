"""MX block formats in float64: E2M1 weights, E8M0 scales, MXFP8 activations.

Test infrastructure (see the package docstring). Plain NumPy, no shared code
with the GPU library.

Formats, as the sources use them:
  * E2M1 ("FP4"): 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent 0 is
    subnormal. Largest magnitude 6.0, the FLOAT4_E2M1_MAX that "SGLang
    CUTLASS MoE" (section 6, FP4 support) names.
  * E8M0 ("float8_e8m0fnu", the Marlin MXFP4 MoE page, section 2): an
    unsigned power-of-two exponent, value 2^(e-127); byte 255 is NaN.
  * One E8M0 scale per 32 consecutive K elements (the MX block). Two E2M1
    codes per byte; the low nibble holds the even K element.
  * MXFP8 (W4A8 activations): E4M3 ("fn": no infinities, 0x7F/0xFF NaN,
    largest 448) elements with one E8M0 per 32 K elements. The pages name
    "MXFP8 activation" for the decode MoE (section 7 of the Shape-template
    page) without its recipe; the recipe here is the OCP MX one: shared
    exponent floor(log2(amax)) - 8, elements rounded to nearest-even with
    saturation at +-448.
  * MXFP4 (W4A4 activations): E2M1 elements with one E8M0 per 32 K
    elements. "SGLang CUTLASS MoE" (section 6, FP4 support) quantises the
    activations to FP4 (E2M1) too and corrects E2M1's small range (largest
    6.0) with extra scales; with power-of-two E8M0 block scales the range
    is covered by the shared exponent, as in the OCP MX recipe: shared
    exponent floor(log2(amax)) - 2 (2 = the largest E2M1 exponent),
    elements rounded to the nearest E2M1 value, ties to the even code,
    saturating at +-6.
"""
from __future__ import annotations

import numpy as np

# Magnitudes of E2M1 codes 0..7 (sign bit clear).
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)

MX_BLOCK = 32
E4M3_MAX = 448.0


def e2m1_decode(codes) -> np.ndarray:
    """E2M1 codes (0..15) -> float64. Code 8 (negative zero) decodes to -0.0."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def e8m0_decode(e) -> np.ndarray:
    """E8M0 bytes -> 2^(e-127) in float64; byte 255 -> NaN."""
    e = np.asarray(e).astype(np.int64)
    v = np.ldexp(1.0, e - 127)
    return np.where(e == 255, np.nan, v)


def _unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] codes; low nibble = even K index."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


# The value of each of the 16 E2M1 codes (index = code), from e2m1_decode.
E2M1_VALUES = e2m1_decode(np.arange(16))


def dequant_mxfp4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 rows -> float64.

    packed [..., K/2] uint8, scales [..., K/32] uint8 -> W [..., K] with
    W[..., k] = E2M1(code k) * 2^(scales[..., k // 32] - 127): each code's
    value from the 16-entry table, times its block's scale.
    """
    codes = _unpack_nibbles(packed)
    k = codes.shape[-1]
    assert scales.shape[-1] * MX_BLOCK == k, (scales.shape, k)
    vals = E2M1_VALUES[codes].reshape(codes.shape[:-1] + (k // MX_BLOCK, MX_BLOCK))
    return (vals * e8m0_decode(scales)[..., None]).reshape(codes.shape)


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 (fn) codes -> float64; 0x7F/0xFF -> NaN."""
    c = np.asarray(codes).astype(np.int64)
    s = np.where((c & 0x80) != 0, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = c & 7
    sub = np.ldexp(m.astype(np.float64), -9)
    nrm = np.ldexp(1.0 + m / 8.0, ef - 7)
    v = s * np.where(ef == 0, sub, nrm)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def _e4m3_encode(a: np.ndarray) -> np.ndarray:
    """Round float64 values to E4M3 codes: nearest, ties to even, saturating.

    Every step below is exact in float64 (power-of-two scalings of the input
    and an integer rounding), so the code is the correctly rounded one.
    """
    neg = np.signbit(a)
    mag = np.minimum(np.abs(a), E4M3_MAX)
    codes = np.zeros(a.shape, dtype=np.int64)
    small = mag < 2.0 ** -6
    # Subnormal range: spacing 2^-9; a rounded count of 8 is the smallest normal,
    # whose code is also 8.
    codes[small] = np.round(mag[small] * 2.0 ** 9).astype(np.int64)
    big = ~small
    if np.any(big):
        _, ex = np.frexp(mag[big])  # mag = f * 2^ex, f in [0.5, 1)
        ex = ex - 1  # floor(log2(mag))
        q = np.round(np.ldexp(mag[big], 3 - ex)).astype(np.int64)  # in [8, 16]
        carry = q == 16
        ex = np.where(carry, ex + 1, ex)
        q = np.where(carry, 8, q)
        codes[big] = ((ex + 7) << 3) | (q - 8)
    codes = np.where(neg, codes | 0x80, codes)
    return codes.astype(np.uint8)


def quant_mxfp8(v: np.ndarray):
    """MXFP8 quantisation along the last axis (length a multiple of 32).

    Per 32-element block: amax = max |v|; if amax == 0 the scale byte is 0 and
    every element code is 0 (sign kept). Otherwise the shared exponent is
    floor(log2(amax)) - 8 (8 = the largest E4M3 exponent), stored biased by
    127 and clamped to [0, 254]; elements are v / 2^shared rounded to E4M3.
    Returns (codes uint8 [..., K], scales uint8 [..., K/32]).
    """
    v = np.asarray(v, dtype=np.float64)
    k = v.shape[-1]
    assert k % MX_BLOCK == 0
    blk = v.reshape(v.shape[:-1] + (k // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blk), axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    biased = np.clip((ex - 1) - 8 + 127, 0, 254)
    biased = np.where(amax > 0, biased, 0)
    scaled = blk / np.ldexp(1.0, biased - 127)[..., None]
    codes = _e4m3_encode(scaled).reshape(v.shape)
    return codes, biased.astype(np.uint8)


def dequant_mxfp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP8 codes + E8M0 scales -> float64."""
    return e4m3_decode(codes) * np.repeat(e8m0_decode(scales), MX_BLOCK, axis=-1)


def _e2m1_encode(a: np.ndarray) -> np.ndarray:
    """Round float64 values to E2M1 codes: the nearest of the eight
    magnitudes, a tie to the even code (the one whose mantissa bit is 0),
    magnitudes above 6 saturating to 6; the sign bit is the input's (so a
    negative value that rounds to zero gives code 8, -0)."""
    a = np.asarray(a, dtype=np.float64)
    mag = np.minimum(np.abs(a), 6.0)
    d = np.abs(mag[..., None] - E2M1_MAGNITUDES)  # distance to each of codes 0..7
    dmin = d.min(axis=-1, keepdims=True)
    # among the (one or two) nearest codes, take the even one if there are two
    cand = d == dmin
    even_pref = np.where(np.arange(8) % 2 == 0, 0, 1)  # even codes rank first
    score = np.where(cand, even_pref, 2)
    codes = np.argmin(score, axis=-1).astype(np.int64)
    codes = np.where(np.signbit(a), codes | 8, codes)
    return codes.astype(np.uint8)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., K] codes (0..15) -> [..., K/2] bytes; even K index in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def quant_mxfp4(v: np.ndarray):
    """MXFP4 quantisation along the last axis (length a multiple of 32).

    Per 32-element block: amax = max |v|; if amax == 0 the scale byte is 0 and
    every element is zero (sign kept). Otherwise the shared exponent is
    floor(log2(amax)) - 2, stored biased by 127 and clamped to [0, 254];
    elements are v / 2^shared rounded to E2M1 (_e2m1_encode).
    Returns (codes packed two per byte [..., K/2], scales uint8 [..., K/32]),
    the layout dequant_mxfp4 reads.
    """
    v = np.asarray(v, dtype=np.float64)
    k = v.shape[-1]
    assert k % MX_BLOCK == 0
    blk = v.reshape(v.shape[:-1] + (k // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blk), axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    biased = np.clip((ex - 1) - 2 + 127, 0, 254)
    biased = np.where(amax > 0, biased, 0)
    scaled = blk / np.ldexp(1.0, biased - 127)[..., None]
    codes = _e2m1_encode(scaled).reshape(v.shape)
    return pack_nibbles(codes), biased.astype(np.uint8)
