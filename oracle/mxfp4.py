"""MXFP4 encode/decode, the oracle's version (test infrastructure only).

MXFP4 as the pages use it: expert weights stored packed, two E2M1 codes per
byte, with one UE8M0 power-of-two scale per 32 consecutive elements along K
([P3] commit notes on the MXFP4 format pinning UE8M0 scales, on the group-32
divisibility guard and on regrouping GPT-OSS blocks into the packed weight).
The encodings themselves come from [OCP].
"""
from __future__ import annotations

import numpy as np

BLOCK = 32

#: E2M1 magnitudes for the low three bits of a code ([OCP] FP4 E2M1: one
#: sign bit, two exponent bits with bias 1, one mantissa bit; exponent 0
#: is subnormal).  The sign is bit 3.
E2M1_MAGNITUDE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e2m1_decode(codes) -> np.ndarray:
    """float64 value of each 4-bit code; code 8 is -0.0."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAGNITUDE[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def ue8m0_decode(scales) -> np.ndarray:
    """2**(s - 127) as float64; s = 255 is NaN ([OCP] E8M0)."""
    s = np.asarray(scales).astype(np.int64)
    out = np.ldexp(1.0, s - 127)
    return np.where(s == 255, np.nan, out)


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] 4-bit codes.  Reading: element 2i is the
    low nibble of byte i and element 2i+1 the high nibble (the GPT-OSS/OCP
    packing order; the pages only say "packed")."""
    b = np.asarray(codes, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = b & 0x0F
    out[..., 1::2] = b >> 4
    return out


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact float64 values of a packed MXFP4 tensor.

    codes  uint8 [..., K/2], scales uint8 [..., K/32] -> float64 [..., K]
    value(n, k) = e2m1(code(n, k)) * 2**(scales[n, k // 32] - 127).

    Every such value is exactly representable in float64, and in float32 and
    bf16 whenever it is finite there, so dequantisation has one correct
    answer ([P3] commit note: the dequantize converter is bit-equal to the
    implementation it replaces).
    """
    c = unpack_codes(codes)
    K = c.shape[-1]
    s = np.asarray(scales)
    if s.shape[-1] * BLOCK != K:
        raise ValueError(f"scales last dim {s.shape[-1]} does not match K={K}")
    with np.errstate(invalid="ignore"):
        return e2m1_decode(c) * np.repeat(ue8m0_decode(s), BLOCK, axis=-1)


def scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Shared exponent e of each block: the smallest integer with
    6 * 2**e >= amax, i.e. ceil(log2(amax / 6)), clamped to [-127, 127].

    Reading: the configs give ceil(log2(amax/6)); amax = 0 (log = -inf) and
    the clamp to the UE8M0 range are ours.  The value is found exactly: a
    float64 log2 gives a first guess, then the defining inequality fixes it,
    so powers of two never round the wrong way.
    """
    a = np.asarray(amax, dtype=np.float64)
    e = np.full(a.shape, -127, dtype=np.int64)
    pos = a > 0
    with np.errstate(divide="ignore"):
        guess = np.ceil(np.log2(a[pos] / 6.0)).astype(np.int64)
    guess = np.clip(guess, -130, 130)
    ap = a[pos]
    # smallest e with 6 * 2**e >= amax
    up = 6.0 * np.ldexp(1.0, guess) < ap
    guess = guess + up
    down = 6.0 * np.ldexp(1.0, guess - 1) >= ap
    guess = guess - down
    e[pos] = guess
    return np.clip(e, -127, 127)


def round_e2m1(y: np.ndarray) -> np.ndarray:
    """4-bit code of the E2M1 value nearest to y (|y| <= 6).

    Reading: ties go to the even code (round half to even on the mantissa
    bit, the [OCP] default conversion), so the midpoints 0.25, 0.75, 1.25,
    1.75, 2.5, 3.5 and 5 go to 0, 1, 1, 2, 2, 4 and 4.  The sign bit of y is
    kept, so small negatives (and -0.0) give code 8.
    """
    y = np.asarray(y, dtype=np.float64)
    mag = np.abs(y)
    best = np.zeros(mag.shape, dtype=np.int64)
    # Walk the seven midpoints between neighbouring magnitudes i and i+1:
    # above a midpoint the upper neighbour is nearer; exactly on it, the
    # even one of the two wins.
    for i in range(7):
        mid = 0.5 * (E2M1_MAGNITUDE[i] + E2M1_MAGNITUDE[i + 1])
        upper_even = (i + 1) % 2 == 0
        best += (mag > mid) | ((mag == mid) & upper_even)
    sign = np.signbit(y).astype(np.int64) << 3
    return (best | sign).astype(np.uint8)


def quantize(w: np.ndarray):
    """Row-wise MXFP4 quantisation of w [..., K] (K % 32 == 0).

    Per 32-block along K: amax = max |x|; e = scale_exponent(amax);
    code = round_e2m1(x / 2**e); scale byte = e + 127; codes packed two per
    byte, low nibble first.  ([P3] commit note on the row-wise MXFP4
    quantizers, one launch per tensor; the scale rule from the workload
    recipe, "UE8M0 scale = ceil(log2(amax/6))".)

    Returns (codes uint8 [..., K/2], scales uint8 [..., K/32]).
    NaN or Inf inputs are outside the contract.
    """
    x = np.asarray(w, dtype=np.float32).astype(np.float64)
    K = x.shape[-1]
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = x.reshape(x.shape[:-1] + (K // BLOCK, BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    e = scale_exponent(amax)
    y = blocks / np.ldexp(1.0, e)[..., None]
    c = round_e2m1(y).reshape(x.shape)
    packed = (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)
