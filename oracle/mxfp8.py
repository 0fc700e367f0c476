"""MXFP8 (E4M3 elements, UE8M0 scale per 32) activation quantization, the
oracle's version (test infrastructure only).

The kernels the pages describe quantize activations to a block-scaled
format when the weights are block-scaled and no weight-only format is asked
for ([P3] commit notes: activation_format None = the weights' format,
"bf16" = weight-only; MXFP8 through row-wise quantizers).  The element and
scale encodings are [OCP]'s: E4M3 has a sign bit, four exponent bits with
bias 7 and three mantissa bits; exponent field 0 is subnormal (steps of
2^-9); the largest finite magnitude is 448 (S.1111.110) and S.1111.111 is
NaN (no infinities).

Readings (the pages fix none of this):
  * block scale: 2^e with e the smallest integer for which every |x| / 2^e
    is at most 448, i.e. e = ceil(log2(amax / 448)), clamped to [-127, 127]
    (amax = 0 gives -127) -- the same rule as the library's MXFP4 weight
    quantizer, with 448 in place of 6, so no element saturates;
  * element: the nearest E4M3 value to x / 2^e, ties to the even code;
  * hi + lo split: hi = q(x), lo = q(x - deq(hi)), each block with its own
    scale; x ~ deq(hi) + deq(lo).
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """float64 value of each 8-bit E4M3 code (0x7F / 0xFF are NaN)."""
    c = np.asarray(codes).astype(np.int64)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where((c & 0x80) != 0, -mag, mag)


def e4m3_round(v) -> np.ndarray:
    """Code of the nearest E4M3 value to each v (|v| <= 448), ties to the
    even code (even mantissa).  -0.0 and negatives that round to zero keep
    the sign bit."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > E4M3_MAX) or np.any(~np.isfinite(a)):
        raise ValueError("e4m3_round: |v| > 448 or non-finite")
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal (and zero): multiples of 2^-9; 8 * 2^-9 is the smallest normal
    q = np.rint(a[sub] * 2.0 ** 9)            # rint rounds halves to even
    code[sub] = q.astype(np.int64)
    n = ~sub
    an = a[n]
    e = np.floor(np.log2(an)).astype(np.int64)
    # guard log2 rounding at exact powers of two
    e = np.where(np.ldexp(1.0, e) > an, e - 1, e)
    e = np.where(np.ldexp(1.0, e + 1) <= an, e + 1, e)
    m = np.rint((an / np.ldexp(1.0, e) - 1.0) * 8.0).astype(np.int64)
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    code[n] = ((e + 7) << 3) | m
    sign = np.signbit(v)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def block_exponent(x: np.ndarray) -> np.ndarray:
    """e per 32-block along the last axis: the smallest integer with
    amax / 2^e <= 448, clamped to [-127, 127]."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    amax = a.reshape(a.shape[:-1] + (a.shape[-1] // BLOCK, BLOCK)).max(axis=-1)
    e = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    r = amax[nz] / E4M3_MAX
    en = np.ceil(np.log2(r)).astype(np.int64)
    # exact: the smallest e with r <= 2^e
    en = np.where(np.ldexp(1.0, en) < r, en + 1, en)
    en = np.where(np.ldexp(1.0, en - 1) >= r, en - 1, en)
    e[nz] = en
    return np.clip(e, -127, 127)


def quantize(x) -> tuple[np.ndarray, np.ndarray]:
    """float64/bf16-valued x [..., K] (K % 32 == 0) -> (codes uint8 [..., K],
    scales uint8 [..., K/32])."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    e = block_exponent(x)
    xs = x / np.repeat(np.ldexp(1.0, e), BLOCK, axis=-1)
    return e4m3_round(xs), (e + 127).astype(np.uint8)


def dequantize(codes, scales) -> np.ndarray:
    s = np.asarray(scales).astype(np.int64)
    return e4m3_decode(codes) * np.repeat(np.ldexp(1.0, s - 127), BLOCK, axis=-1)


def quantize_hi_lo(x):
    """(hi codes, hi scales, lo codes, lo scales) with lo quantizing the
    residual x - deq(hi)."""
    x = np.asarray(x, dtype=np.float64)
    hc, hs = quantize(x)
    lc, ls = quantize(x - dequantize(hc, hs))
    return hc, hs, lc, ls
