"""Pins of the oracle's MXFP8 activation quantizer (oracle/mxfp8.py):
the OCP E4M3 value table, brute-force nearest-value rounding with ties to
the even code, the block-scale rule and the hi + lo split's error."""
import os

import numpy as np
import pytest

from oracle import mxfp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_values.txt")

FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_decode_matches_the_ocp_table():
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        got = float(mxfp8.e4m3_decode(int(code, 16)))
        if val == "nan":
            assert np.isnan(got), code
        else:
            assert got == float(val) and np.signbit(got) == val.startswith("-"), (code, got, val)


def test_decode_closed_form_every_code():
    # sign * 2^(e-7) * (1 + m/8), subnormal sign * 2^-6 * m/8
    for c in FINITE.astype(int):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        ref = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        ref = -ref if s else ref
        assert mxfp8.e4m3_decode(c) == ref


def _brute(v):
    """Nearest finite code by exhaustive search, ties to the even mantissa."""
    vals = mxfp8.e4m3_decode(FINITE)
    out = []
    for x in np.atleast_1d(v):
        d = np.abs(vals - x)
        best = np.flatnonzero(d == d.min())
        cand = [int(FINITE[i]) for i in best]
        # among equidistant codes of the right sign, the one with an even mantissa
        cand = [c for c in cand if ((c & 0x80) != 0) == np.signbit(x)] or cand
        even = [c for c in cand if (c & 1) == 0]
        out.append((even or cand)[0])
    return np.array(out, dtype=np.uint8)


def test_round_matches_brute_force_on_random_and_midpoints():
    rng = np.random.default_rng(3)
    vals = np.sort(mxfp8.e4m3_decode(FINITE[FINITE < 0x7F]))       # non-negative grid
    mids = (vals[1:] + vals[:-1]) / 2
    samples = np.concatenate([mids, -mids, vals, -vals,
                              rng.uniform(-448, 448, 2000),
                              rng.standard_normal(2000) * 2.0 ** rng.integers(-12, 8, 2000)])
    samples = np.clip(samples, -448, 448)
    got = mxfp8.e4m3_round(samples)
    ref = _brute(samples)
    # +0 / -0 both decode to zero; compare values, then signs where non-zero
    gv, rv = mxfp8.e4m3_decode(got), mxfp8.e4m3_decode(ref)
    assert np.array_equal(gv, rv)
    nz = gv != 0
    assert np.array_equal(got[nz], ref[nz])


def test_round_refuses_out_of_range():
    with pytest.raises(ValueError):
        mxfp8.e4m3_round(np.array([449.0]))


def test_block_scale_rule():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((50, 64)) * 2.0 ** rng.integers(-30, 30, (50, 1))
    x[3, :32] = 0.0
    e = mxfp8.block_exponent(x)
    amax = np.abs(x).reshape(50, 2, 32).max(-1)
    nz = amax > 0
    # amax / 2^e <= 448 < amax / 2^(e - 1)
    assert np.all(amax[nz] / np.ldexp(1.0, e[nz]) <= 448)
    assert np.all(amax[nz] / np.ldexp(1.0, e[nz] - 1) > 448)
    assert e[3, 0] == -127


def test_quantize_error_bound_and_exact_round_trip():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((40, 96))
    c, s = mxfp8.quantize(x)
    y = mxfp8.dequantize(c, s)
    scale = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=-1)
    # at most half an E4M3 step: 2^-4 relative above the smallest normal,
    # 2^-10 absolute (in scale units) below it
    err = np.abs(x - y) / scale
    mag = np.abs(x) / scale
    bound = np.where(mag >= 2.0 ** -6, mag * 2.0 ** -4, 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-12))
    # values already on the grid survive unchanged
    c2, s2 = mxfp8.quantize(y)
    assert np.array_equal(mxfp8.dequantize(c2, s2), y)


def test_hi_lo_split_is_much_closer():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 2880))
    hc, hs, lc, ls = mxfp8.quantize_hi_lo(x)
    one = np.abs(x - mxfp8.dequantize(hc, hs)).max()
    two = np.abs(x - mxfp8.dequantize(hc, hs) - mxfp8.dequantize(lc, ls)).max()
    assert two < one * 2.0 ** -3


def test_forward_activation_formats():
    # "bf16" is the unquantized forward; the quantized formats change only the
    # gate_up input: equal to a forward on the dequantized activations with
    # the routing kept; hi + lo is far closer to bf16 than one MXFP8 pass
    import moe_synth as syn
    from layers import oracle_layer
    from oracle import moe
    s = syn.spec("tiny", T=40, H=128, I=96, E=4, k=2)
    L = oracle_layer(s)
    x = syn.tokens(s)
    r = moe.route(L, x)
    ref, _, _ = moe.forward(L, x, routing=r)
    same, _, _ = moe.forward(L, x, routing=r, act_format="bf16")
    assert np.array_equal(ref, same)
    xf = moe.bf16_to_f64(x)
    errs = {}
    for fmt in ("mxfp8", "mxfp8x2"):
        out, _, cache = moe.forward(L, x, routing=r, act_format=fmt)
        xq = moe.gate_up_input(xf, fmt)
        f = int(r.sorted_rows[0])
        e = int(np.searchsorted(r.offsets, 0, side="right") - 1)
        h = xq[f // s.k] @ L.gate_up(e).T + L.gu_b(e)
        np.testing.assert_allclose(cache[f][0], h, rtol=1e-12, atol=1e-14)
        errs[fmt] = np.abs(out - ref).max() / np.abs(ref).max()
    assert 0 < errs["mxfp8x2"] < errs["mxfp8"] * 1e-2
