"""Pins of the oracle's MXFP4 encode/decode against things other than itself:
the OCP code table (golden file), a bit-field closed form, torch's own E8M0
dtype, brute force over every (byte, scale) pair, a brute-force nearest
search and the round-trip and error-bound invariants."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import mxfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_pairs(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                a, b = line.split()
                rows.append((a, b))
    return rows


def _fields_value(code):
    """E2M1 from its bit fields: sign bit 3, exponent bits 2..1 (bias 1),
    mantissa bit 0; exponent 0 is subnormal (0.m * 2**0)."""
    sign = -1.0 if code & 8 else 1.0
    ex = (code >> 1) & 3
    man = code & 1
    if ex == 0:
        return sign * (man * 0.5)
    return sign * (2.0 ** (ex - 1)) * (1.0 + man / 2.0)


def test_e2m1_table_matches_ocp_golden():
    got = mxfp4.e2m1_decode(np.arange(16))
    for code, val in _read_pairs("e2m1_table.txt"):
        v = float(val)
        g = got[int(code)]
        assert g == v and math.copysign(1, g) == math.copysign(1, v), (code, g, v)


def test_e2m1_table_matches_bitfield_closed_form():
    got = mxfp4.e2m1_decode(np.arange(16))
    for c in range(16):
        ref = _fields_value(c)
        assert got[c] == ref and math.copysign(1, got[c]) == math.copysign(1, ref)


def test_ue8m0_matches_torch_e8m0_dtype():
    s = torch.arange(256, dtype=torch.uint8)
    ref = s.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = mxfp4.ue8m0_decode(np.arange(256))
    assert np.isnan(got[255]) and np.isnan(ref[255])
    np.testing.assert_array_equal(got[:255], ref[:255])


def test_dequant_every_byte_and_scale_brute_force():
    # one row of 32 bytes per scale value: the 256 bytes spread over 8 rows
    byte = np.arange(256, dtype=np.uint8).reshape(8, 32)
    for s in range(256):
        scales = np.full((8, 2), s, dtype=np.uint8)
        got = mxfp4.dequantize(byte, scales)
        for r in range(8):
            for i in range(32):
                b = int(byte[r, i])
                for half, code in ((0, b & 15), (1, b >> 4)):
                    ref = math.nan if s == 255 else math.ldexp(_fields_value(code), s - 127)
                    g = got[r, 2 * i + half]
                    if s == 255:
                        assert math.isnan(g)
                    else:
                        assert g == ref and math.copysign(1, g) == math.copysign(1, ref)


def test_nibble_order_low_first():
    # byte 0x21: element 0 is code 1 (0.5), element 1 is code 2 (1.0)
    codes = np.zeros((1, 16), dtype=np.uint8)
    codes[0, 0] = 0x21
    codes[0, 15] = 0xF7   # element 30 = code 7 (6.0), element 31 = code 15 (-6.0)
    v = mxfp4.dequantize(codes, np.full((1, 1), 127, np.uint8))
    assert v[0, 0] == 0.5 and v[0, 1] == 1.0
    assert v[0, 30] == 6.0 and v[0, 31] == -6.0
    assert np.all(v[0, 2:30] == 0)


def test_dequant_values_fit_fp32_and_bf16_exactly():
    # every dequantized value below 2**128 in magnitude is exactly a float32
    # and, having at most two significant bits, exactly a bf16 too; larger
    # ones (magnitude >= 4 at s = 253, >= 2 at s = 254) overflow to +-inf
    byte = np.arange(256, dtype=np.uint8).reshape(8, 32)
    for s in range(0, 255):
        v = mxfp4.dequantize(byte, np.full((8, 2), s, np.uint8))
        with np.errstate(over="ignore"):
            f = v.astype(np.float32)
        fin = np.abs(v) < 2.0 ** 128
        assert np.array_equal(f[fin].astype(np.float64), v[fin])
        assert np.all(np.isinf(f[~fin])) and np.array_equal(np.sign(f[~fin]), np.sign(v[~fin]))
        assert (s >= 253) == (not fin.all())
        bits = f.view(np.uint32)
        assert np.all((bits & 0xFFFF) == 0)  # bf16 = top 16 bits


def _brute_exponent(amax):
    if amax == 0:
        return -127
    e = -200
    while 6.0 * 2.0 ** e < amax:
        e += 1
    return max(-127, min(127, e))


def test_scale_exponent_brute_force():
    rng = np.random.default_rng(1)
    vals = [0.0, 6.0, 3.0, 12.0, 6.0000001, 5.9999999, 1e-40, 1e-45, 3e38, 0.75, 1.5]
    vals += [6.0 * 2.0 ** p for p in range(-130, 127, 7)]
    vals += list(np.abs(rng.standard_normal(200)) * 10.0 ** rng.integers(-30, 30, 200))
    vals = np.array(vals, dtype=np.float32).astype(np.float64)
    got = mxfp4.scale_exponent(vals)
    for a, e in zip(vals, got):
        assert e == _brute_exponent(a), (a, e)


def test_scale_exponent_invariant_on_normal_range():
    rng = np.random.default_rng(2)
    amax = np.abs(rng.standard_normal(10000)) * 10.0 ** rng.integers(-20, 20, 10000)
    e = mxfp4.scale_exponent(amax)
    r = amax / np.ldexp(1.0, e)
    assert np.all(r > 3.0) and np.all(r <= 6.0)


def test_rounding_golden_midpoints():
    for y, val in _read_pairs("e2m1_rounding.txt"):
        c = mxfp4.round_e2m1(np.array([float(y)]))[0]
        g = mxfp4.e2m1_decode(c)
        v = float(val)
        assert g == v and math.copysign(1, g) == math.copysign(1, v), (y, g, v)


def _brute_round(y):
    """Nearest of the 8 magnitudes by exhaustive search; on a tie, the one
    whose code (index) is even."""
    mags = [_fields_value(c) for c in range(8)]
    best = None
    for c, m in enumerate(mags):
        d = abs(abs(y) - m)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (8 if math.copysign(1, y) < 0 else 0)


def test_rounding_brute_force():
    rng = np.random.default_rng(3)
    ys = np.concatenate([np.linspace(-6, 6, 4801), rng.uniform(-6, 6, 2000),
                         [0.0, -0.0, 1e-30, -1e-30]])
    got = mxfp4.round_e2m1(ys)
    for y, c in zip(ys, got):
        assert c == _brute_round(float(y)), (y, c)


def test_quantize_round_trip_value_idempotent():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 256, (64, 48), dtype=np.uint8)
    scales = rng.integers(100, 150, (64, 3), dtype=np.uint8)
    v = mxfp4.dequantize(codes, scales)
    c2, s2 = mxfp4.quantize(v.astype(np.float32))
    np.testing.assert_array_equal(mxfp4.dequantize(c2, s2), v)


def test_quantize_grid_values_exact_and_bytes_stable():
    # blocks whose max magnitude code is 6.0 keep their codes and scale
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, (16, 16), dtype=np.uint8)
    codes[:, 0] = 0x07   # element 0 = +6.0 in every row's only block
    scales = rng.integers(110, 140, (16, 1), dtype=np.uint8)
    v = mxfp4.dequantize(codes, scales)
    c2, s2 = mxfp4.quantize(v.astype(np.float32))
    np.testing.assert_array_equal(s2, scales)
    # signed zeros survive too: code 8 is -0.0 and quantizes back to 8
    np.testing.assert_array_equal(c2, codes)


def test_quantize_error_bound():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((40, 256)) * 0.02).astype(np.float32)
    c, s = mxfp4.quantize(w)
    v = mxfp4.dequantize(c, s)
    e = s.astype(np.int64) - 127
    step = np.repeat(np.ldexp(1.0, e), 32, axis=1)
    err = np.abs(w.astype(np.float64) - v)
    # the widest gap in the E2M1 grid is 2 (between 4 and 6): half of it
    assert np.all(err <= step)
    # below magnitude 4 the gaps are at most 1: half-gap 0.5
    y = np.abs(w.astype(np.float64)) / step
    assert np.all(err[y < 3.5] <= 0.5 * step[y < 3.5])


def test_quantize_small_block_signs_and_zero_block():
    w = np.zeros((2, 32), np.float32)
    w[1, :] = -1e-9
    w[1, 0] = 6e-9
    c, s = mxfp4.quantize(w)
    assert s[0, 0] == 0      # amax = 0 -> e = -127
    v = mxfp4.dequantize(c, s)
    assert np.all(v[0] == 0)
    # -1e-9 / 2**e with amax 6e-9 rounds to -0.0 or a small negative code
    assert np.all(np.signbit(v[1, 1:]))


def test_quantize_rejects_ragged_k():
    with pytest.raises(ValueError):
        mxfp4.quantize(np.zeros((2, 48), np.float32))
