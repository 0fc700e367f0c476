"""Pins of the oracle's MoE block against things other than itself: the
bf16 decode against its bit-field definition and torch's conversion over
all 65536 patterns, exact sums (math.fsum), brute-force top-k, scipy's softmax, a brute-force double
loop for the permutation, torch's silu, a per-token brute-force expert loop,
the dense-MLP special case (E = 1, k = 1) written with torch, closed forms
for zero weights and for bias perturbations, and float64 central finite
differences for every gradient the backward returns."""
import copy
import math

import numpy as np
import pytest
import scipy.special
import torch

import moe_synth as syn
from oracle import moe, mxfp4

from layers import oracle_layer

TINY = syn.spec("tiny")


@pytest.fixture(scope="module")
def tiny():
    return oracle_layer(TINY)


@pytest.fixture(scope="module")
def tiny_x():
    return syn.tokens(TINY)


# ------------------------------------------------------------- bf16 decode

def _bf16_closed_form(b):
    """Value of one bf16 bit pattern from its fields: sign bit 15, an 8-bit
    exponent (bits 14..7, bias 127) and a 7-bit fraction with a hidden 1
    unless the exponent field is 0 (subnormal); exponent 255 is Inf or
    NaN."""
    sign = -1.0 if b >> 15 else 1.0
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    if e == 0xFF:
        return sign * math.inf if m == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(m, -126 - 7)
    return sign * math.ldexp(128 + m, e - 127 - 7)


def _same_values(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))   # -0.0 stays -0.0


def test_bf16_decode_every_pattern_closed_form():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    _same_values(moe.bf16_to_f64(bits), [_bf16_closed_form(int(b)) for b in bits])


def test_bf16_decode_every_pattern_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    _same_values(moe.bf16_to_f64(bits), ref)
    # shapes are kept, and float64 input is taken as already decoded
    assert moe.bf16_to_f64(bits.reshape(256, 256)).shape == (256, 256)
    probe = np.array([0.1, -3.0])
    assert moe.bf16_to_f64(probe) is probe


# ------------------------------------------------------------------ router

def test_router_logits_exact_sum(tiny, tiny_x):
    # x decoded from its bit fields here, independently of bf16_to_f64
    x = np.array([[_bf16_closed_form(int(b)) for b in row] for row in tiny_x])
    got = moe.router_logits(tiny, tiny_x)
    for t in range(x.shape[0]):
        for e in range(tiny.E):
            terms = [float(a) * float(b) for a, b in zip(x[t], tiny.router_w[e].astype(np.float64))]
            terms.append(float(tiny.router_b[e]))
            assert got[t, e] == np.float32(math.fsum(terms))


def _brute_topk(row, k):
    order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
    return order[:k]


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(0)
    logits = np.round(rng.standard_normal((300, 9)) * 2) / 2   # many exact ties
    logits = logits.astype(np.float32)
    for k in (1, 2, 4, 9):
        idx, w = moe.topk_softmax(logits, k)
        for t in range(logits.shape[0]):
            assert list(idx[t]) == _brute_topk(logits[t], k)
        sel = np.take_along_axis(logits, idx, 1).astype(np.float64)
        np.testing.assert_allclose(w, scipy.special.softmax(sel, axis=1), rtol=1e-14, atol=0)
        assert np.all(np.abs(w.sum(1) - 1) <= k * 2.0 ** -52)


def test_topk_special_cases():
    eq = np.zeros((5, 8), np.float32)
    idx, w = moe.topk_softmax(eq, 3)
    assert np.all(idx == np.arange(3)) and np.all(w == 1 / 3)
    idx, w = moe.topk_softmax(np.random.default_rng(1).standard_normal((7, 8)).astype(np.float32), 1)
    assert np.all(w == 1.0)
    with pytest.raises(ValueError):
        moe.topk_softmax(eq, 9)


def test_router_zero_weights_routes_to_first_k(tiny, tiny_x):
    L = copy.copy(tiny)
    L.router_w = np.zeros_like(tiny.router_w)
    L.router_b = np.zeros_like(tiny.router_b)
    r = moe.route(L, tiny_x)
    assert np.all(r.idx == np.arange(L.k)) and np.all(r.w == 1.0 / L.k)


# ------------------------------------------------------------- permutation

def _brute_permutation(idx, E):
    flat = [int(v) for v in np.asarray(idx).reshape(-1)]
    offsets = [0]
    rows = []
    for e in range(E):
        for f, ef in enumerate(flat):
            if ef == e:
                rows.append(f)
        offsets.append(len(rows))
    return offsets, rows


@pytest.mark.parametrize("E,k,T", [(4, 2, 16), (32, 4, 200), (128, 4, 300), (7, 7, 5), (3, 1, 1)])
def test_permutation_brute_force(E, k, T):
    rng = np.random.default_rng(E * 1000 + T)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    off, rows = moe.permutation(idx, E)
    boff, brows = _brute_permutation(idx, E)
    assert list(off) == boff and list(rows) == brows
    assert sorted(rows) == list(range(T * k))          # bijection
    flat = idx.reshape(-1)
    for e in range(E):
        seg = rows[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


# -------------------------------------------------------------- activation

def test_swiglu_reduces_to_silu_without_clamp():
    g = torch.linspace(-12, 12, 1001, dtype=torch.float64)
    u = torch.linspace(-3, 3, 1001, dtype=torch.float64)
    ref = torch.nn.functional.silu(g) * (u + 1)
    got = moe.swiglu(g.numpy(), u.numpy(), 1.0, np.inf)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-13, atol=1e-300)


def test_swiglu_is_quick_gelu_times_up():
    # x * sigmoid(1.702 x) is the sigmoid approximation of GELU; with
    # u = 0 and no clamp the GLU is exactly that function of the gate
    g = np.linspace(-5, 5, 101)
    ref = torch.nn.functional.silu(torch.tensor(1.702 * g)).numpy() / 1.702
    np.testing.assert_allclose(moe.swiglu(g, np.zeros_like(g), 1.702, np.inf), ref, rtol=1e-13)


def test_swiglu_clamps():
    a, L = 1.702, 7.0
    assert moe.swiglu(10.0, 0.5, a, L) == moe.swiglu(7.0, 0.5, a, L)
    assert moe.swiglu(1.0, -9.0, a, L) == moe.swiglu(1.0, -7.0, a, L)
    assert moe.swiglu(1.0, 9.0, a, L) == moe.swiglu(1.0, 7.0, a, L)
    assert moe.swiglu(-8.0, 0.5, a, L) != moe.swiglu(-7.0, 0.5, a, L)   # gate: upper clamp only
    assert moe.swiglu(0.0, 3.0, a, L) == 0.0
    assert moe.swiglu(1.0, -1.0, a, L) == 0.0
    assert abs(moe.swiglu(-200.0, 0.0, a, L)) < 1e-100


def test_swiglu_backward_finite_differences():
    rng = np.random.default_rng(7)
    a, L = 1.702, 7.0
    g = rng.uniform(-10, 10, 4000)
    u = rng.uniform(-10, 10, 4000)
    keep = (np.abs(g - L) > 1e-3) & (np.abs(np.abs(u) - L) > 1e-3)
    g, u = g[keep], u[keep]
    da = rng.standard_normal(g.size)
    dg, du = moe.swiglu_backward(g, u, da, a, L)
    eps = 1e-6
    fg = (moe.swiglu(g + eps, u, a, L) - moe.swiglu(g - eps, u, a, L)) / (2 * eps) * da
    fu = (moe.swiglu(g, u + eps, a, L) - moe.swiglu(g, u - eps, a, L)) / (2 * eps) * da
    np.testing.assert_allclose(dg, fg, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(du, fu, rtol=1e-6, atol=1e-8)
    assert np.all(dg[g > L] == 0) and np.all(du[np.abs(u) > L] == 0)


# ----------------------------------------------------------------- forward

def _brute_forward(L, x_bits):
    """Per token, per selected expert, dense math on dequantized weights:
    no permutation and no per-expert batching."""
    x = moe.bf16_to_f64(x_bits)
    T = x.shape[0]
    logits = moe.router_logits(L, x_bits)
    out = np.zeros((T, L.H))
    for t in range(T):
        sel = _brute_topk(logits[t], L.k)
        ls = np.array([float(logits[t, e]) for e in sel])
        ws = np.exp(ls - ls.max())
        ws /= ws.sum()
        for j, e in enumerate(sel):
            Wgu = mxfp4.dequantize(L.gu_codes[e], L.gu_scales[e])
            Wd = mxfp4.dequantize(L.dn_codes[e], L.dn_scales[e])
            h = np.array([np.dot(Wgu[n], x[t]) for n in range(2 * L.I)]) + L.gu_b(e)
            if L.has_lora_gu:
                Ag = moe.bf16_to_f64(L.lora_gu_A[e])
                Bg = moe.bf16_to_f64(L.lora_gu_B[e])
                h = h + L.lora_scale * Bg @ (Ag @ x[t])
            act = moe.swiglu(h[0::2], h[1::2], L.alpha, L.limit)
            y = np.array([np.dot(Wd[m], act) for m in range(L.H)]) + L.dn_b(e)
            if L.has_lora:
                A = moe.bf16_to_f64(L.lora_A[e])
                B = moe.bf16_to_f64(L.lora_B[e])
                y = y + L.lora_scale * B @ (A @ act)
            out[t] += ws[j] * y
    return out


def test_forward_matches_per_token_brute_force(tiny, tiny_x):
    out, _, _ = moe.forward(tiny, tiny_x)
    np.testing.assert_allclose(out, _brute_forward(tiny, tiny_x), rtol=1e-12, atol=1e-14)


def test_forward_with_lora_matches_brute_force():
    s = syn.spec("tiny", lora_rank=8)
    L = oracle_layer(s)
    x = syn.tokens(s)
    out, _, _ = moe.forward(L, x)
    np.testing.assert_allclose(out, _brute_forward(L, x), rtol=1e-12, atol=1e-14)


def test_forward_dense_special_case_torch():
    s = syn.spec("tiny", E=1, k=1)
    L = oracle_layer(s)
    x = syn.tokens(s)
    out, r, _ = moe.forward(L, x)
    assert np.all(r.w == 1.0)
    xt = torch.tensor(moe.bf16_to_f64(x))
    h = torch.nn.functional.linear(xt, torch.tensor(L.gate_up(0)), torch.tensor(L.gu_b(0)))
    act = torch.tensor(moe.swiglu(h[:, 0::2].numpy(), h[:, 1::2].numpy(), L.alpha, L.limit))
    ref = torch.nn.functional.linear(act, torch.tensor(L.down(0)), torch.tensor(L.dn_b(0)))
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-14)


def test_forward_zero_codes_gives_weighted_down_bias(tiny, tiny_x):
    L = copy.copy(tiny)
    L.gu_codes = np.zeros_like(tiny.gu_codes)
    L.dn_codes = np.zeros_like(tiny.dn_codes)
    out, r, _ = moe.forward(L, tiny_x)
    ref = np.einsum("tj,tjh->th", r.w, moe.bf16_to_f64(L.dn_bias)[r.idx])
    np.testing.assert_allclose(out, ref, rtol=1e-14, atol=0)


def test_bias_reaches_both_projections(tiny, tiny_x):
    out0, r, _ = moe.forward(tiny, tiny_x)
    e = int(r.idx[0, 0])
    routed = np.any(r.idx == e, axis=1)
    # down bias: out changes by w[t, j] * delta exactly on the routed tokens
    L = copy.copy(tiny)
    L.dn_bias = tiny.dn_bias.copy()
    L.dn_bias[e, 3] = syn.bf16_bits(np.array([moe.bf16_to_f64(tiny.dn_bias[e, 3]) + 0.5]))[0]
    delta = moe.bf16_to_f64(L.dn_bias[e, 3]) - moe.bf16_to_f64(tiny.dn_bias[e, 3])
    out1, _, _ = moe.forward(L, tiny_x)
    wj = np.where(r.idx == e, r.w, 0.0).sum(1)
    np.testing.assert_allclose(out1[:, 3] - out0[:, 3], wj * delta, rtol=1e-9, atol=1e-15)
    # gate_up bias: only tokens routed to e move
    L = copy.copy(tiny)
    L.gu_bias = tiny.gu_bias.copy()
    L.gu_bias[e] = syn.bf16_bits(moe.bf16_to_f64(tiny.gu_bias[e]).astype(np.float32) + 0.25)
    out2, _, _ = moe.forward(L, tiny_x)
    moved = np.any(out2 != out0, axis=1)
    assert np.array_equal(moved, routed)


def test_forward_token_subset(tiny, tiny_x):
    full, _, cache = moe.forward(tiny, tiny_x)
    toks = np.array([0, 3, 15])
    part, _, cache2 = moe.forward(tiny, tiny_x, tokens=toks)
    np.testing.assert_allclose(part[toks], full[toks], rtol=1e-13, atol=1e-16)
    assert np.all(part[np.setdiff1d(np.arange(16), toks)] == 0)
    assert set(cache2) == {t * tiny.k + j for t in toks for j in range(tiny.k)}


def test_stacked_gate_up_is_not_interleaved(tiny, tiny_x):
    # the layout is a precondition: the same weights in stacked order
    # ([gate; up] halves) give a different block
    L = copy.copy(tiny)
    order = np.concatenate([np.arange(0, 2 * L.I, 2), np.arange(1, 2 * L.I, 2)])
    L.gu_codes = tiny.gu_codes[:, order]
    L.gu_scales = tiny.gu_scales[:, order]
    L.gu_bias = tiny.gu_bias[:, order]
    a, _, _ = moe.forward(tiny, tiny_x)
    b, _, _ = moe.forward(L, tiny_x)
    assert np.abs(a - b).max() > 1e-3 * np.abs(a).max()


# ---------------------------------------------------------------- backward

def _loss(L, x, dY):
    out, _, _ = moe.forward(L, x)
    return float(np.sum(dY * out))


def _fd_layer(s, x_scale=1.0, lora=False):
    L = oracle_layer(s)
    L.logit_dtype = np.float64
    if lora:
        for name in ("lora_A", "lora_B", "lora_gu_A", "lora_gu_B"):
            if getattr(L, name) is not None:
                setattr(L, name, moe.bf16_to_f64(getattr(L, name)))
    x = moe.bf16_to_f64(syn.tokens(s, scale=x_scale))
    dY = moe.bf16_to_f64(syn.upstream_grad(s))
    return L, x, dY


@pytest.mark.parametrize("x_scale", [1.0, 64.0])
def test_backward_dx_finite_differences(x_scale):
    L, x, dY = _fd_layer(TINY, x_scale)
    if x_scale > 1:
        # the scaled case must actually hit the clamps
        _, _, cache = moe.forward(L, x)
        h = np.stack([c[0] for c in cache.values()])
        assert np.any(h[:, 0::2] > L.limit) and np.any(np.abs(h[:, 1::2]) > L.limit)
    dX, _, _ = moe.backward_dx(L, x, dY)
    r0 = moe.route(L, x)
    rng = np.random.default_rng(11)
    checked = 0
    for _ in range(12):
        v = rng.standard_normal(x.shape)
        eps = 1e-4 * np.linalg.norm(x) / np.linalg.norm(v) / 64
        xp, xm = x + eps * v, x - eps * v
        if not (np.array_equal(moe.route(L, xp).idx, r0.idx) and np.array_equal(moe.route(L, xm).idx, r0.idx)):
            continue
        # keep away from the clamp kinks
        _, _, cp = moe.forward(L, xp)
        _, _, cm = moe.forward(L, xm)
        hp = np.stack([c[0] for c in cp.values()])
        hm = np.stack([c[0] for c in cm.values()])
        if np.any(np.sign(hp[:, 0::2] - L.limit) != np.sign(hm[:, 0::2] - L.limit)) or \
           np.any(np.sign(np.abs(hp[:, 1::2]) - L.limit) != np.sign(np.abs(hm[:, 1::2]) - L.limit)):
            continue
        fd = (_loss(L, xp, dY) - _loss(L, xm, dY)) / (2 * eps)
        an = float(np.sum(dX * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)) + 1e-7 * np.abs(dX).sum() * np.abs(v).max(), (fd, an)
        checked += 1
    assert checked >= 6


def test_backward_block_scaled_is_straight_through(monkeypatch):
    # Under a block-scaled activation format the backward is the exact
    # gradient of the forward with the quantization error c = x_q - x held
    # constant.  Central differences of that surrogate (gate_up input x + c;
    # the router and the adapter read x) must match dX and the down
    # adapter's gradients, and dX must differ from the bf16 backward's by
    # far more than the check's tolerance, so a backward that recomputed h
    # from the unquantized x would fail.  The format enters only through
    # gate_up_input (pinned in the MXFP8 tests); single-pass MXFP8 is the
    # one whose error the differences can see (the hi + lo pair is
    # accurate to about 2^-18 of a block's amax).  Elements spread over
    # 2^-16..1 give every block an error.
    fmt = "mxfp8"
    s = syn.spec("tiny", lora_rank=8)
    L, x, dY = _fd_layer(s, lora=True)
    x = x * 2.0 ** np.random.default_rng(14).integers(-16, 1, x.shape)
    dX, dA, dB = moe.backward_dx(L, x, dY, act_format=fmt)
    plain, _, _ = moe.backward_dx(L, x, dY)
    c = moe.gate_up_input(x, fmt) - x
    assert np.abs(c).max() > 0
    assert np.abs(dX - plain).max() > 1e-4 * np.abs(plain).max()
    monkeypatch.setattr(moe, "gate_up_input", lambda xx, f: xx + c)
    r0 = moe.route(L, x)
    rng = np.random.default_rng(13)
    checked = 0
    for _ in range(8):
        v = rng.standard_normal(x.shape)
        eps = 1e-6
        xp, xm = x + eps * v, x - eps * v
        if not (np.array_equal(moe.route(L, xp).idx, r0.idx) and
                np.array_equal(moe.route(L, xm).idx, r0.idx)):
            continue
        fd = (_loss(L, xp, dY) - _loss(L, xm, dY)) / (2 * eps)
        an = float(np.sum(dX * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (fd, an)
        checked += 1
    assert checked >= 4
    for name, grad in (("lora_A", dA), ("lora_B", dB)):
        base = getattr(L, name)
        for _ in range(4):
            pos = tuple(int(rng.integers(0, n)) for n in base.shape)
            eps = 1e-4
            Lp, Lm = copy.copy(L), copy.copy(L)
            P, M = base.copy(), base.copy()
            P[pos] += eps
            M[pos] -= eps
            setattr(Lp, name, P)
            setattr(Lm, name, M)
            fd = (_loss(Lp, x, dY) - _loss(Lm, x, dY)) / (2 * eps)
            assert abs(fd - grad[pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])


def test_backward_router_term_is_needed():
    # without the router path the gradient is wrong (finite differences
    # include it), and the expert path alone is non-zero: no silent gradient
    L, x, dY = _fd_layer(TINY)
    dX, _, _ = moe.backward_dx(L, x, dY)
    L0 = copy.copy(L)
    L0.router_w = np.zeros_like(L.router_w)
    L0.router_b = L.router_b
    # expert path: rebuild with router gradient removed by freezing routing
    r = moe.route(L, x)
    dX_expert, _, _ = moe.backward_dx(L0, x, dY, routing=r)
    assert np.abs(dX_expert).max() > 0
    assert np.abs(dX - dX_expert).max() > 1e-3 * np.abs(dX).max()


def test_backward_lora_finite_differences():
    s = syn.spec("tiny", lora_rank=8)
    L, x, dY = _fd_layer(s, lora=True)
    dX, dA, dB = moe.backward_dx(L, x, dY)
    rng = np.random.default_rng(12)
    for name, grad in (("lora_A", dA), ("lora_B", dB)):
        base = getattr(L, name)
        for _ in range(6):
            pos = tuple(int(rng.integers(0, n)) for n in base.shape)
            eps = 1e-4
            P = base.copy()
            P[pos] += eps
            Lp = copy.copy(L)
            setattr(Lp, name, P)
            M = base.copy()
            M[pos] -= eps
            Lm = copy.copy(L)
            setattr(Lm, name, M)
            fd = (_loss(Lp, x, dY) - _loss(Lm, x, dY)) / (2 * eps)
            assert abs(fd - grad[pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])
    # and dX with LoRA present
    v = rng.standard_normal(x.shape)
    eps = 1e-6
    fd = (_loss(L, x + eps * v, dY) - _loss(L, x - eps * v, dY)) / (2 * eps)
    assert abs(fd - np.sum(dX * v)) <= 1e-6 * max(1.0, abs(fd))


def test_backward_token_subset_matches_full():
    L = oracle_layer(TINY)
    x = syn.tokens(TINY)
    dY = syn.upstream_grad(TINY)
    full, _, _ = moe.backward_dx(L, x, dY)
    toks = np.array([1, 2, 9])
    part, _, _ = moe.backward_dx(L, x, dY, tokens=toks)
    np.testing.assert_allclose(part[toks], full[toks], rtol=1e-13, atol=1e-15)


def test_expert_subsets_partition_the_block():
    # the experts= restriction splits the expert loop: per-expert outputs
    # and adapter gradients add up to the unrestricted ones
    s = syn.spec("tiny", lora_rank=16)
    L = oracle_layer(s)
    L.lora_scale = 3.0
    x = syn.tokens(s)
    dY = syn.upstream_grad(s)
    out, r, _ = moe.forward(L, x)
    _, dA, dB = moe.backward_dx(L, x, dY)
    acc = np.zeros_like(out)
    for e in range(s.E):
        oe, _, _ = moe.forward(L, x, routing=r, experts=[e])
        acc += oe
        _, dAe, dBe = moe.backward_dx(L, x, dY, routing=r, experts=[e])
        np.testing.assert_allclose(dAe[e], dA[e], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(dBe[e], dB[e], rtol=1e-12, atol=1e-15)
        others = [i for i in range(s.E) if i != e]
        assert not np.any(dAe[others]) and not np.any(dBe[others])
    np.testing.assert_allclose(acc, out, rtol=1e-12, atol=1e-15)


def test_lora_gradients_against_scale_derivative():
    # The adapter delta enters y as s * (v B^T), so with the routing fixed
    # L(s) is affine in s and dL/ds = <dB, B> / s = <dA, A> / s: both inner
    # products equal s times the slope of the loss between two scales.
    s = syn.spec("tiny", lora_rank=16)
    L = oracle_layer(s)
    x = syn.tokens(s)
    dY = moe.bf16_to_f64(syn.upstream_grad(s))
    r = moe.route(L, x)
    sc = 2.5
    L.lora_scale = sc
    _, dA, dB = moe.backward_dx(L, x, syn.upstream_grad(s), routing=r)
    vals = []
    for s_ in (0.0, 1.0):
        L.lora_scale = s_
        out, _, _ = moe.forward(L, x, routing=r)
        vals.append(float(np.sum(dY * out)))
    slope = vals[1] - vals[0]
    A = moe.bf16_to_f64(L.lora_A)
    B = moe.bf16_to_f64(L.lora_B)
    ipA, ipB = float(np.sum(dA * A)), float(np.sum(dB * B))
    assert abs(slope) > 1e-6
    assert abs(ipB - sc * slope) <= 1e-10 * abs(sc * slope)
    assert abs(ipA - sc * slope) <= 1e-10 * abs(sc * slope)


# ------------------------------------------------ adapter on gate_up (both)

def test_forward_with_gate_up_lora_matches_brute_force():
    s = syn.spec("tiny", lora_rank=8, lora_gate_up=True)
    L = oracle_layer(s)
    L.lora_scale = 3.0
    x = syn.tokens(s)
    out, _, cache = moe.forward(L, x)
    np.testing.assert_allclose(out, _brute_forward(L, x), rtol=1e-12, atol=1e-14)
    # the cached vg is x A_gu^T of the row's token
    xf = moe.bf16_to_f64(x)
    r = moe.route(L, x)
    for f in r.sorted_rows[:5]:
        e = int(np.searchsorted(r.offsets, np.nonzero(r.sorted_rows == f)[0][0], side="right") - 1)
        ref = moe.bf16_to_f64(L.lora_gu_A[e]) @ xf[f // s.k]
        np.testing.assert_allclose(cache[int(f)][3], ref, rtol=1e-13, atol=1e-16)


def test_gate_up_adapter_changes_the_output():
    # the adapter term is not lost: switching it off moves the output
    s = syn.spec("tiny", lora_rank=16, lora_gate_up=True, lora_down=False)
    L = oracle_layer(s)
    L.lora_scale = 8.0
    x = syn.tokens(s)
    r = moe.route(L, x)
    out, _, _ = moe.forward(L, x, routing=r)
    L0 = copy.copy(L)
    L0.lora_gu_A = L0.lora_gu_B = None
    out0, _, _ = moe.forward(L0, x, routing=r)
    assert np.abs(out - out0).max() > 1e-3 * np.abs(out0).max()


@pytest.mark.parametrize("down", [False, True])
def test_backward_gate_up_lora_finite_differences(down):
    s = syn.spec("tiny", lora_rank=8, lora_gate_up=True, lora_down=down)
    L, x, dY = _fd_layer(s, lora=True)
    L.lora_scale = 2.0
    g = {}
    dX, dA, dB = moe.backward_dx(L, x, dY, gu_grads=g)
    assert (dA is not None) == down and (dB is not None) == down
    rng = np.random.default_rng(13)
    grads = [("lora_gu_A", g["dA_gu"]), ("lora_gu_B", g["dB_gu"])]
    if down:
        grads += [("lora_A", dA), ("lora_B", dB)]
    for name, grad in grads:
        base = getattr(L, name)
        assert grad.shape == base.shape
        for _ in range(6):
            pos = tuple(int(rng.integers(0, n)) for n in base.shape)
            eps = 1e-4
            P = base.copy()
            P[pos] += eps
            Lp = copy.copy(L)
            setattr(Lp, name, P)
            M = base.copy()
            M[pos] -= eps
            Lm = copy.copy(L)
            setattr(Lm, name, M)
            fd = (_loss(Lp, x, dY) - _loss(Lm, x, dY)) / (2 * eps)
            assert abs(fd - grad[pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])
    # dX carries the gate_up adapter's input gradient
    v = rng.standard_normal(x.shape)
    eps = 1e-6
    fd = (_loss(L, x + eps * v, dY) - _loss(L, x - eps * v, dY)) / (2 * eps)
    assert abs(fd - np.sum(dX * v)) <= 1e-6 * max(1.0, abs(fd))


def test_gate_up_adapter_gradients_partition_over_experts():
    s = syn.spec("tiny", lora_rank=16, lora_gate_up=True)
    L = oracle_layer(s)
    L.lora_scale = 3.0
    x = syn.tokens(s)
    dY = syn.upstream_grad(s)
    r = moe.route(L, x)
    g = {}
    moe.backward_dx(L, x, dY, routing=r, gu_grads=g)
    for e in range(s.E):
        ge = {}
        moe.backward_dx(L, x, dY, routing=r, experts=[e], gu_grads=ge)
        np.testing.assert_allclose(ge["dA_gu"][e], g["dA_gu"][e], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(ge["dB_gu"][e], g["dB_gu"][e], rtol=1e-12, atol=1e-15)
        others = [i for i in range(s.E) if i != e]
        assert not np.any(ge["dA_gu"][others]) and not np.any(ge["dB_gu"][others])


# ---------------------------------------------- base-weight gradients (dW)

@pytest.mark.parametrize("lora", [False, True])
def test_base_weight_gradients_finite_differences(lora):
    # gradients with respect to the dequantized weights and the biases:
    # perturb one entry of a float64 weight copy (or a bias) and difference
    # the loss
    s = syn.spec("tiny", lora_rank=8 if lora else 0, lora_gate_up=lora)
    L, x, dY = _fd_layer(s, lora=lora)
    L.lora_scale = 2.0
    L.gu_weight = np.stack([mxfp4.dequantize(L.gu_codes[e], L.gu_scales[e]) for e in range(s.E)])
    L.dn_weight = np.stack([mxfp4.dequantize(L.dn_codes[e], L.dn_scales[e]) for e in range(s.E)])
    L.gu_bias = moe.bf16_to_f64(L.gu_bias)
    L.dn_bias = moe.bf16_to_f64(L.dn_bias)
    g = {}
    moe.backward_dx(L, x, dY, base_grads=g)
    assert g["dW_gu"].shape == L.gu_weight.shape and g["dW_dn"].shape == L.dn_weight.shape
    rng = np.random.default_rng(14)
    for name, grad in (("gu_weight", g["dW_gu"]), ("dn_weight", g["dW_dn"]),
                       ("gu_bias", g["db_gu"]), ("dn_bias", g["db_dn"])):
        base = getattr(L, name)
        nz = 0
        for _ in range(8):
            pos = tuple(int(rng.integers(0, n)) for n in base.shape)
            eps = 1e-4
            P = base.copy()
            P[pos] += eps
            Lp = copy.copy(L)
            setattr(Lp, name, P)
            M = base.copy()
            M[pos] -= eps
            Lm = copy.copy(L)
            setattr(Lm, name, M)
            fd = (_loss(Lp, x, dY) - _loss(Lm, x, dY)) / (2 * eps)
            assert abs(fd - grad[pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])
            nz += grad[pos] != 0
        assert nz > 0, name


def test_base_weight_gradients_closed_form_dense():
    # E = 1, k = 1: w = 1 and every token goes to the one expert, so
    # dW_dn = dY^T a and dW_gu = dh^T x over all tokens (torch autograd on
    # the dense float64 MLP as the reference)
    s = syn.spec("tiny", E=1, k=1)
    L = oracle_layer(s)
    x = syn.tokens(s)
    dY = syn.upstream_grad(s)
    g = {}
    moe.backward_dx(L, x, dY, base_grads=g)
    xt = torch.from_numpy(moe.bf16_to_f64(x))
    Wg = torch.from_numpy(L.gate_up(0)).requires_grad_(True)
    Wd = torch.from_numpy(L.down(0)).requires_grad_(True)
    bg = torch.from_numpy(L.gu_b(0)).requires_grad_(True)
    bd = torch.from_numpy(L.dn_b(0)).requires_grad_(True)
    h = xt @ Wg.T + bg
    gte, up = h[:, 0::2].clamp(max=L.limit), h[:, 1::2].clamp(-L.limit, L.limit)
    act = gte * torch.sigmoid(L.alpha * gte) * (up + 1)
    y = act @ Wd.T + bd
    (y * torch.from_numpy(moe.bf16_to_f64(dY))).sum().backward()
    np.testing.assert_allclose(g["dW_gu"][0], Wg.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dW_dn"][0], Wd.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["db_gu"][0], bg.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["db_dn"][0], bd.grad.numpy(), rtol=1e-10, atol=1e-12)
