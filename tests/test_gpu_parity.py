"""GPU parity of the HIP path against the float64 oracle, through the C ABI.

Integers (quantised bytes, dequantised bits, routing indices, expert
offsets, the permutation) must match bit for bit; floating-point results
(routing weights, the saved h and a, out, dX) must reach
max|g - r| / max|r| <= 2e-2 and cosine >= 0.9999 against the oracle.
Full-size layers: the 2048-token gpt-oss-20b layer and its decode sizes are
compared whole (every token's out and dX, every routed row's saved h and a);
the skewed 120b layer compares every row of its hottest expert (dozens of
row tiles and a ragged last one) and of a single-tile expert, plus out and
dX of sampled tokens; the 16384-token LoRA layer runs the checkpointing
sequence (forward, recompute forward, backward) and checks the recompute
bit for bit and dX on 64 tokens.
"""
import math
import sys

import numpy as np
import pytest
import torch

import moe_synth as syn
from mxfp4_weight_mixture_02_amd import (Mxfp4Error, mxfp4_dequantize, mxfp4_moe_backward,
                                         mxfp4_moe_backward_dx, mxfp4_moe_forward, mxfp4_quantize,
                                         mxfp8_quantize)
from oracle import moe, mxfp4, mxfp8

from gpu_helpers import (DEV, assert_bytes_equal, assert_close, assert_routing_equal, bf16_tensor,
                         cache_dequant, device_layer, min_topk_gap, oracle_layer, to_f64)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# ------------------------------------------------------------ MXFP4 codec

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_dequantize_every_byte_and_scale(dtype):
    _say(f"dequantize exhaustive {dtype}")
    codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))          # [256 rows, 256 B]
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 16, 1)  # one scale per row
    got = mxfp4_dequantize(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                           dtype)
    torch.cuda.synchronize()
    ref = mxfp4.dequantize(codes, scales)
    with np.errstate(over="ignore"):
        ref32 = ref.astype(np.float32)
    g = got.float().cpu().numpy()
    nan = np.isnan(ref32)
    assert np.all(np.isnan(g[nan]))
    assert np.array_equal(g[~nan].view(np.uint32), ref32[~nan].view(np.uint32))


def _quant_cases():
    rng = np.random.default_rng(21)
    out = {
        "normal_0.02": (rng.standard_normal((64, 2880)) * 0.02).astype(np.float32),
        "wide_range": (rng.standard_normal((32, 256)) *
                       10.0 ** rng.integers(-38, 37, (32, 1))).astype(np.float32),
        "zeros_and_neg_zero": (np.zeros((4, 64)) * np.array([1, -1, 1, -1])[:, None]).astype(np.float32),
    }
    # exact E2M1 midpoints and neighbours times a power of two per block
    # (each block's amax is exactly 6 * 2^e, so the midpoints stay midpoints)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    m7 = mids[:7]
    blk = np.concatenate([mids, -mids, np.nextafter(m7, np.float32(0)),
                          np.nextafter(m7, np.float32(7)), [np.float32(-6.0), np.float32(4.0)]])
    assert blk.size == 32
    e = rng.integers(-100, 100, 16).astype(np.float32)
    out["midpoints"] = np.stack([blk * np.float32(2.0) ** ee for ee in e]).astype(np.float32)
    out["tiny_subnormal"] = (rng.standard_normal((8, 64)) * 1e-41).astype(np.float32)
    out["one_block"] = np.linspace(-6, 6, 32, dtype=np.float32)[None, :]
    return out


@pytest.mark.parametrize("name", list(_quant_cases().keys()))
def test_quantize_bytes_match_oracle(name):
    _say(f"quantize {name}")
    w = _quant_cases()[name]
    c, s = mxfp4_quantize(torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    rc, rs = mxfp4.quantize(w)
    assert np.array_equal(s.cpu().numpy(), rs), "scales differ"
    assert np.array_equal(c.cpu().numpy(), rc), "codes differ"


# ------------------------------------------------------------- small layers

def _run_layer(s, x_scale=1.0, with_bias=True, backward=True, T=None, lora_scale=1.0):
    T = s.T if T is None else T
    _say(f"layer {s.name} T={T} H={s.H} I={s.I} E={s.E} k={s.k} x_scale={x_scale} bias={with_bias}"
         f" lora_rank={s.lora_rank} lora_scale={lora_scale}")
    dl = device_layer(s, with_bias=with_bias)
    ol, _ = oracle_layer(s, with_bias=with_bias)
    dl.lora_scale = ol.lora_scale = lora_scale
    # the oracle's quantised bytes must equal the GPU's (all four tensors)
    assert_bytes_equal(dl, ol)
    xb = syn.tokens(s, T, scale=x_scale)
    x = bf16_tensor(xb).to(DEV)
    out, sv = mxfp4_moe_forward(dl, x, saved=True)
    torch.cuda.synchronize()
    ref, r, cache = moe.forward(ol, xb)
    assert_routing_equal(sv, r)
    assert_close(to_f64(out), ref, "out")
    # saved state, in sorted order
    rows = r.sorted_rows
    href = np.stack([cache[int(f)][0] for f in rows])
    aref = np.stack([cache[int(f)][1] for f in rows])
    assert_close(to_f64(sv.h), href, "saved h")
    assert_close(to_f64(sv.a), aref, "saved a")
    if ol.has_lora:
        ex = np.searchsorted(r.offsets, np.arange(T * s.k), side="right") - 1
        vref = np.stack([moe._lora_v(ol, ex[i], aref[i][None])[0] for i in range(T * s.k)])
        assert_close(to_f64(sv.lora_v), vref, "saved lora_v")
    if ol.has_lora_gu:
        vgref = np.stack([cache[int(f)][3] for f in rows])
        assert_close(to_f64(sv.lora_vg), vgref, "saved lora_vg")
    res = {"out": out, "saved": sv, "routing": r}
    if backward:
        dyb = syn.upstream_grad(s, T)
        got = mxfp4_moe_backward_dx(dl, sv, bf16_tensor(dyb).to(DEV), x=x)
        torch.cuda.synchronize()
        g = {}
        dref, dAref, dBref = moe.backward_dx(ol, xb, dyb, gu_grads=g)
        dx, dA, dB = got[:3]
        assert_close(to_f64(dx), dref, "dX")
        if ol.has_lora:
            assert_close(to_f64(dA), dAref, "dA")
            assert_close(to_f64(dB), dBref, "dB")
        if ol.has_lora_gu:
            assert len(got) == 5
            assert_close(to_f64(got[3]), g["dA_gu"], "dA_gu")
            assert_close(to_f64(got[4]), g["dB_gu"], "dB_gu")
        res["dx"] = dx
    return res


def test_tiny_forward_backward():
    _run_layer(syn.spec("tiny"))


def test_tiny_clamp_exercise():
    # activations x64 push |h| past the SwiGLU limit on both branches
    s = syn.spec("tiny")
    ol, _ = oracle_layer(s)
    _, _, cache = moe.forward(ol, syn.tokens(s, scale=64.0))
    h = np.stack([c[0] for c in cache.values()])
    assert np.any(h[:, 0::2] > 7) and np.any(np.abs(h[:, 1::2]) > 7)
    _run_layer(s, x_scale=64.0)


def test_tiny_without_biases():
    _run_layer(syn.spec("tiny"), with_bias=False)


@pytest.mark.parametrize("T", [1, 3, 17])
def test_ragged_token_counts(T):
    _run_layer(syn.spec("tiny"), T=T)


@pytest.mark.parametrize("T", [8, 9, 32, 33, 128, 129])
def test_kernel_dispatch_boundaries(T):
    # tiny layer, k = 2: R = T * k on both sides of every switch of the
    # forward -- the K-split decode kernel (R <= 16), the decode kernels'
    # activation groups of 8 (R <= 64) or 16, the decode kernels and the
    # general GEMMs (R <= 256), and the one-workgroup routing plan (R <= 256)
    _say(f"dispatch boundary T={T} R={2 * T}")
    _run_layer(syn.spec("tiny"), T=T)


def test_dense_special_case():
    _run_layer(syn.spec("tiny", E=1, k=1, T=40))


def test_multi_tile_ragged_tails():
    # >128 rows per expert (several row tiles, ragged last tile), gate_up
    # output 640 = 2.5 column tiles, down output 192 < one column tile,
    # three 64-wide K steps in gate_up and five in down
    _run_layer(syn.spec("tiny", T=300, H=192, I=320, E=3, k=2))


def test_many_experts_top8():
    _run_layer(syn.spec("tiny", T=64, H=128, I=128, E=64, k=8))


@pytest.mark.timeout(600)
def test_maximum_hidden_sizes():
    # H = I = 5120, the largest the library takes: 80 K-steps per GEMM, the
    # eight-wave gate_up, 160 h-chunks in the router, R = 320 > 256 routed
    # rows (the many-token routing path and the general GEMMs)
    _run_layer(syn.spec("tiny", T=160, H=5120, I=5120, E=3, k=2))


def test_256_experts_top8_many_tokens():
    # E = 256 (four experts per lane in the top-k), k = 8; T * E > 4096, so
    # the many-token routing path; R = 256 takes the decode GEMMs
    _run_layer(syn.spec("tiny", T=32, H=64, I=64, E=256, k=8))


def test_256_experts_top8_planned():
    # the one-workgroup routing plan with four experts per lane (T * E = 4096)
    _run_layer(syn.spec("tiny", T=16, H=64, I=64, E=256, k=8))


def test_wide_hidden_size():
    # H = 4160 > 4096: gate_up takes the eight-wave, 512-row workgroup shape
    # (the scale panel of a 256-row workgroup no longer fits its 80 KB), and
    # K = H = 65 steps of 64 leaves a ragged last group of the unrolled loop
    _run_layer(syn.spec("tiny", T=300, H=4160, I=192, E=3, k=2))


@pytest.mark.parametrize("lora_scale", [1.0, 32.0])
def test_lora_tiny(lora_scale):
    # scale 32 makes the adapter delta comparable to the base output
    _run_layer(syn.spec("tiny", lora_rank=16), lora_scale=lora_scale)


def test_lora_multi_tile_ragged_tails():
    _run_layer(syn.spec("tiny", T=300, H=192, I=320, E=3, k=2, lora_rank=16), lora_scale=8.0)


def test_lora_empty_expert_gets_zero_gradients():
    # E = 16 experts, 3 tokens, k = 2: most experts receive no rows; their
    # dA/dB must come back as zeros (overwritten, not left stale)
    s = syn.spec("tiny", T=3, E=16, k=2, lora_rank=16)
    dl = device_layer(s)
    x = bf16_tensor(syn.tokens(s)).to(DEV)
    _, sv = mxfp4_moe_forward(dl, x, saved=True)
    dy = bf16_tensor(syn.upstream_grad(s)).to(DEV)
    dA = torch.full(dl.lora_A.shape, float("nan"), dtype=torch.float32, device=DEV)
    dB = torch.full(dl.lora_B.shape, float("nan"), dtype=torch.float32, device=DEV)
    _, dA, dB = mxfp4_moe_backward_dx(dl, sv, dy, dA=dA, dB=dB)
    torch.cuda.synchronize()
    off = sv.expert_offsets.cpu().numpy()
    empty = np.nonzero(off[1:] == off[:-1])[0]
    assert len(empty) >= 8
    assert torch.isfinite(dA).all() and torch.isfinite(dB).all()
    assert not dA[empty].any() and not dB[empty].any()
    _run_layer(s, lora_scale=4.0)


@pytest.mark.parametrize("T,H,I", [
    (300, 96, 160),    # both odd multiples of 32, several row tiles: the GEMMs' half last K step
    (300, 2912, 224),  # 46 steps of 64 in gate_up and bwd_down, a half 46th; down N = 2912
    (300, 32, 32),     # a single half step everywhere
    (5, 96, 160),      # R = 10: the K-split decode kernel
    (40, 160, 96),     # R = 80: the streaming decode kernel
    (40, 160, 1248),   # R = 80, down K = 1248: staged in segments of 18 steps, a half 20th
])
def test_hidden_sizes_odd_multiples_of_32(T, H, I):
    _say(f"odd multiples of 32: T={T} H={H} I={I}")
    _run_layer(syn.spec("tiny", T=T, H=H, I=I, E=3, k=2))


@pytest.mark.parametrize("r", [8, 32, 64])
def test_lora_ranks(r):
    # every supported rank: 8 (one zero-padded 16-deep chunk), 32 (one full
    # 32-wide rank block), 64 (two), through the GEMM epilogues, the rank
    # projection and the adapter gradients
    _say(f"lora rank {r}")
    _run_layer(syn.spec("tiny", T=300, H=192, I=320, E=3, k=2, lora_rank=r), lora_scale=4.0)


@pytest.mark.parametrize("T,r", [(3, 16), (5, 64), (40, 8), (100, 32)])
def test_lora_at_decode_sizes(T, r):
    # R = T * k <= 256 routed rows: the decode kernels carry the adapter term
    # (R <= 16 the K-split kernel, else the streaming one); odd multiples of
    # 32 for H and I on the way
    _say(f"lora decode T={T} r={r}")
    _run_layer(syn.spec("tiny", T=T, H=96, I=160, E=3, k=2, lora_rank=r), lora_scale=4.0)


@pytest.mark.parametrize("T,r,down", [(300, 16, True), (300, 8, False), (100, 64, True),
                                      (5, 32, True), (40, 16, False)])
def test_lora_on_gate_up(T, r, down):
    # the adapter on gate_up, alone or with the down one: forward (saved vg,
    # the GEMM and decode epilogues), dX's adapter term in bwd_gate_up, and
    # dA_gu / dB_gu; T = 5 and 40 run the decode kernels
    _say(f"gate_up lora T={T} r={r} down={down}")
    _run_layer(syn.spec("tiny", T=T, H=192, I=320, E=3, k=2, lora_rank=r, lora_gate_up=True,
                        lora_down=down), lora_scale=4.0)


def _run_full_backward(s, lora_scale=1.0):
    """Forward (saved), then the full backward: dX, the adapter gradients and
    the base-weight and bias gradients against the oracle, whole tensors and
    expert by expert."""
    _say(f"full backward {s.name} T={s.T} H={s.H} I={s.I} E={s.E} k={s.k} r={s.lora_rank}")
    dl = device_layer(s)
    ol, _ = oracle_layer(s)
    dl.lora_scale = ol.lora_scale = lora_scale
    xb, dyb = syn.tokens(s), syn.upstream_grad(s)
    x = bf16_tensor(xb).to(DEV)
    _, sv = mxfp4_moe_forward(dl, x, saved=True)
    got = mxfp4_moe_backward(dl, sv, x, bf16_tensor(dyb).to(DEV))
    torch.cuda.synchronize()
    g, base = {}, {}
    dref, dAref, dBref = moe.backward_dx(ol, xb, dyb, gu_grads=g, base_grads=base)
    assert_close(to_f64(got["dx"]), dref, "dX")
    refs = dict(base, dA=dAref, dB=dBref, **g)
    off = sv.expert_offsets.cpu().numpy()
    for name in ("dW_gu", "dW_dn", "db_gu", "db_dn", "dA", "dB", "dA_gu", "dB_gu"):
        if refs.get(name) is None:
            assert name not in got
            continue
        gv = got[name].double().cpu().numpy()
        assert_close(gv, refs[name], name)
        if name.startswith("d") and name[1] in "Wb":
            for e in range(s.E):
                if off[e + 1] == off[e]:
                    assert not gv[e].any(), f"{name}[{e}]: expert without rows"
                else:
                    assert_close(gv[e], refs[name][e], f"{name}[{e}]", max_rel=3e-2)
    return got


@pytest.mark.parametrize("shape", [
    dict(),                                     # tiny: 4 experts, 16 tokens
    dict(T=300, H=192, I=320, E=3, k=2),        # several 64-row steps per expert, ragged
    dict(T=200, H=96, I=160, E=3, k=2),         # odd multiples of 32
    dict(T=260, H=320, I=288, E=5, k=2),        # 2I = 576, H = 320: partial 256 tiles
    dict(T=3, E=16, k=2),                       # most experts without rows
])
def test_full_backward_base_weight_gradients(shape):
    _run_full_backward(syn.spec("tiny", **shape))


@pytest.mark.parametrize("r,gu,dn", [(16, True, True), (8, False, True), (32, True, False)])
def test_full_backward_with_adapters(r, gu, dn):
    _run_full_backward(syn.spec("tiny", T=300, H=192, I=320, E=3, k=2, lora_rank=r,
                                lora_gate_up=gu, lora_down=dn), lora_scale=4.0)


def test_mxfp8_quantize_bytes_match_oracle():
    # row-wise MXFP8 (hi and the residual lo) against the oracle, byte for
    # byte: normal activations, wide exponent ranges, an all-zero block,
    # values on the E4M3 grid and its midpoints, subnormal-range values
    rng = np.random.default_rng(21)
    rows = [rng.standard_normal(256),
            rng.standard_normal(256) * 2.0 ** rng.integers(-40, 40, 256),
            np.zeros(256),
            np.repeat(mxfp8.e4m3_decode(rng.integers(0, 0x7E, 8)), 32) * 2.0 ** -3,
            rng.standard_normal(256) * 1e-3,
            np.linspace(-448, 448, 256)]
    x = np.stack(rows)
    xb = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)   # truncate to bf16 bits
    xt = bf16_tensor(xb).to(DEV)
    hc, hs, lc, ls = mxfp8_quantize(xt, lo=True)
    torch.cuda.synchronize()
    ref = mxfp8.quantize_hi_lo(moe.bf16_to_f64(xb))
    for name, g, r in zip(("codes", "scales", "lo codes", "lo scales"), (hc, hs, lc, ls), ref):
        gn = g.cpu().numpy()
        bad = np.flatnonzero(gn.ravel() != r.ravel())
        assert bad.size == 0, f"{name}: {bad.size} bytes differ, first at {bad[:5]}"


@pytest.mark.parametrize("fmt", ["mxfp8x2", "mxfp8"])
@pytest.mark.parametrize("shape", [dict(T=300, H=192, I=320, E=3, k=2),
                                   dict(T=40, H=128, I=96, E=4, k=2),
                                   dict(T=5, H=256, I=160, E=3, k=2)])
def test_block_scaled_activation_forward(fmt, shape):
    # the scaled-MFMA gate_up on the packed FP4 weights and MXFP8 token rows,
    # against the oracle's forward with the same quantized activations;
    # with the hi + lo pair it also meets the bar against the bf16 forward
    s = syn.spec("tiny", **shape)
    _say(f"block-scaled activations {fmt} {shape}")
    dl = device_layer(s)
    dl.act_format = fmt
    ol, _ = oracle_layer(s)
    xb = syn.tokens(s)
    out, sv = mxfp4_moe_forward(dl, bf16_tensor(xb).to(DEV), saved=True)
    torch.cuda.synchronize()
    ref, r, cache = moe.forward(ol, xb, act_format=fmt)
    assert_routing_equal(sv, r)
    assert_close(to_f64(out), ref, f"out ({fmt})")
    href = np.stack([cache[int(f)][0] for f in r.sorted_rows])
    assert_close(to_f64(sv.h), href, f"saved h ({fmt})")
    plain, _, _ = moe.forward(ol, xb, routing=r)
    g = to_f64(out)
    rel = np.abs(g - plain).max() / np.abs(plain).max()
    print(f"{fmt}: max_rel against the bf16 forward {rel:.3e}", flush=True)
    if fmt == "mxfp8x2":
        assert_close(g, plain, "out (mxfp8x2 vs bf16 oracle)")


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp8x2"])
@pytest.mark.parametrize("shape", [dict(T=300, H=192, I=320, E=3, k=2, lora_rank=16),
                                   dict(T=1, H=128, I=96, E=8, k=4),
                                   dict(T=40, H=128, I=96, E=4, k=2, lora_rank=8)])
def test_block_scaled_forward_then_backward(fmt, shape):
    # the dX backward run on a block-scaled forward's saved state (its h
    # came from the quantized activations; the backward is straight-through)
    # against the oracle's backward for the same format, with a down adapter
    # and at a one-token decode size; the forward's out as well
    s = syn.spec("tiny", **shape)
    _say(f"block-scaled forward + backward {fmt} {shape}")
    dl = device_layer(s)
    dl.act_format = fmt
    ol, _ = oracle_layer(s)
    dl.lora_scale = ol.lora_scale = 2.0
    xb = syn.tokens(s)
    dyb = syn.upstream_grad(s)
    out, sv = mxfp4_moe_forward(dl, bf16_tensor(xb).to(DEV), saved=True)
    dx, dA, dB = mxfp4_moe_backward_dx(dl, sv, bf16_tensor(dyb).to(DEV))
    torch.cuda.synchronize()
    ref, r, _ = moe.forward(ol, xb, act_format=fmt)
    assert_routing_equal(sv, r)
    assert_close(to_f64(out), ref, f"out ({fmt})")
    dref, dAref, dBref = moe.backward_dx(ol, xb, dyb, routing=r, act_format=fmt)
    assert_close(to_f64(dx), dref, f"dX ({fmt})")
    if ol.has_lora:
        assert_close(to_f64(dA), dAref, f"dA ({fmt})")
        assert_close(to_f64(dB), dBref, f"dB ({fmt})")


def test_forward_is_deterministic():
    s = syn.spec("tiny", T=200, H=128, I=192, E=8, k=4)
    dl = device_layer(s)
    x = bf16_tensor(syn.tokens(s)).to(DEV)
    o1, s1 = mxfp4_moe_forward(dl, x, saved=True)
    o2, s2 = mxfp4_moe_forward(dl, x, saved=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    for n in ("topk_idx", "topk_w", "expert_offsets", "sorted_rows", "h", "a"):
        assert torch.equal(getattr(s1, n).view(torch.uint8), getattr(s2, n).view(torch.uint8)), n


@pytest.mark.parametrize("shape", [dict(T=16), dict(T=64, H=128, I=128, E=64, k=8),
                                   dict(T=300, H=192, I=320, E=3, k=2),
                                   dict(T=40, E=16, k=4, lora_rank=16)])
def test_results_do_not_depend_on_buffer_contents(shape):
    # Every buffer the library reads must have been written by the same
    # call: with the workspace, the output and the saved state pre-filled
    # with NaN (bytes 0xFF), forward and backward reproduce the results of a
    # call on zeroed buffers bit for bit.
    from mxfp4_weight_mixture_02_amd import SavedState, Workspace
    s = syn.spec("tiny", **shape)
    _say(f"buffer-contents check {shape}")
    dl = device_layer(s)
    x = bf16_tensor(syn.tokens(s)).to(DEV)
    dy = bf16_tensor(syn.upstream_grad(s)).to(DEV)
    res = []
    for fill in (0x00, 0xFF, 0xFF):
        ws = Workspace()
        ws.get(1 << 24, x.device).fill_(fill)
        sv = SavedState.empty(dl, s.T, x.device)
        for n in ("topk_idx", "topk_w", "expert_offsets", "sorted_rows", "h", "a", "lora_v"):
            t = getattr(sv, n)
            if t is not None:
                t.view(torch.uint8).fill_(fill)
        out = torch.empty_like(x)
        out.view(torch.uint8).fill_(fill)
        mxfp4_moe_forward(dl, x, saved=sv, out=out, workspace=ws)
        ws.buf.fill_(fill)
        dx = torch.empty_like(x)
        dx.view(torch.uint8).fill_(fill)
        _, dA, dB = mxfp4_moe_backward_dx(dl, sv, dy, dx=dx, workspace=ws)
        torch.cuda.synchronize()
        res.append([out, sv.h, sv.a, dx] + ([dA, dB, sv.lora_v] if s.lora_rank else []))
    for r in res[1:]:
        for g, ref in zip(r, res[0]):
            assert torch.equal(g.view(torch.uint8), ref.view(torch.uint8))


def test_inference_forward_equals_saved_forward():
    s = syn.spec("tiny", T=77)
    dl = device_layer(s)
    x = bf16_tensor(syn.tokens(s)).to(DEV)
    o1, _ = mxfp4_moe_forward(dl, x, saved=None)
    o2, _ = mxfp4_moe_forward(dl, x, saved=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("shape", [dict(T=200, H=128, I=192, E=8, k=4),
                                   dict(T=4, E=8, k=2),
                                   dict(T=40, E=16, k=4, lora_rank=16)])
def test_graph_replay_matches_eager(shape):
    # Forward (saved) + backward captured once in a HIP graph.  Before each
    # of three replays an eager forward + backward on other tokens rewrites
    # every buffer the graph uses (outputs, saved state, workspaces); each
    # replay must then reproduce the eager results on the captured tokens
    # bit for bit.  T = 4 takes the decode-size path (plan + weight-
    # streaming GEMMs), the others the general path.
    from mxfp4_weight_mixture_02_amd import SavedState, Workspace
    s = syn.spec("tiny", **shape)
    _say(f"graph replay {shape}")
    dl = device_layer(s)
    x = bf16_tensor(syn.tokens(s)).to(DEV)
    x2 = x.flip(0).contiguous()
    dy = bf16_tensor(syn.upstream_grad(s)).to(DEV)
    sv = SavedState.empty(dl, s.T, DEV)
    out, dx = torch.empty_like(x), torch.empty_like(x)
    lora = dl.lora_A is not None
    dA = torch.empty(dl.lora_A.shape, dtype=torch.float32, device=DEV) if lora else None
    dB = torch.empty(dl.lora_B.shape, dtype=torch.float32, device=DEV) if lora else None
    wsf, wsb = Workspace(), Workspace()

    def run(xin):
        mxfp4_moe_forward(dl, xin, saved=sv, out=out, workspace=wsf)
        mxfp4_moe_backward_dx(dl, sv, dy, dx=dx, workspace=wsb, dA=dA, dB=dB)

    def results():
        return [out, dx, sv.h, sv.a] + ([dA, dB] if lora else [])

    run(x)
    torch.cuda.synchronize()
    ref = [t.clone() for t in results()]
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            run(x)
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    for rep in range(3):
        run(x2)
        torch.cuda.synchronize()
        assert not torch.equal(out.view(torch.int16), ref[0].view(torch.int16))
        g.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(results(), ref)):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), (rep, i)
    del g


def test_unsupported_shape_raises():
    s = syn.spec("tiny")
    dl = device_layer(s)
    x = bf16_tensor(syn.tokens(s)).to(DEV)
    dl.k = 5  # k > E
    with pytest.raises(Mxfp4Error):
        mxfp4_moe_forward(dl, x)


# --------------------------------------------------------- non-finite input

@pytest.mark.parametrize("T", [16, 200])
def test_non_finite_tokens_still_route_k_distinct_experts(T):
    # Tokens holding a NaN or an Inf give NaN or infinite logits.  The top-k
    # orders on a total key (NaN lowest, ties to the lower index, the order
    # of the oracle's stable sort), so such a token still takes k distinct
    # experts and adds exactly k rows: offsets[E] = T * k, the permutation
    # equals the oracle's and every other token's results are computed.
    # T = 16 takes the one-workgroup routing plan, T = 200 the many-token
    # path (R = 400 routed rows).
    s = syn.spec("tiny", T=T)
    _say(f"non-finite tokens T={T}")
    xb = syn.tokens(s, T).copy()
    xb[1, 5] = 0x7FC0                  # NaN: every logit NaN
    xb[3, 0] = 0x7F80                  # +Inf
    xb[6, :] = 0xFF80                  # -Inf everywhere: logits +-Inf and NaN
    xb[9, 7] = 0x7F80
    xb[9, 8] = 0xFF80                  # +Inf and -Inf in one token
    bad = np.array([1, 3, 6, 9])
    good = np.setdiff1d(np.arange(T), bad)
    dl = device_layer(s)
    ol, _ = oracle_layer(s)
    x = bf16_tensor(xb).to(DEV)
    out, sv = mxfp4_moe_forward(dl, x, saved=True)
    dyb = syn.upstream_grad(s, T)
    dx, _, _ = mxfp4_moe_backward_dx(dl, sv, bf16_tensor(dyb).to(DEV))
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore", over="ignore"):
        ref, r, _ = moe.forward(ol, xb)
        dref, _, _ = moe.backward_dx(ol, xb, dyb, tokens=good, routing=r)
    idx = sv.topk_idx.cpu().numpy()
    assert np.array_equal(idx, r.idx)
    assert all(len(set(row)) == s.k for row in idx)
    off = sv.expert_offsets.cpu().numpy()
    assert off[-1] == T * s.k and np.array_equal(off, r.offsets)
    assert np.array_equal(sv.sorted_rows.cpu().numpy(), r.sorted_rows)
    assert_close(to_f64(out)[good], ref[good], "out (finite tokens)")
    assert_close(to_f64(dx)[good], dref[good], "dX (finite tokens)")


# --------------------------------------------------------- full-size layers

def _device_and_routing(s, T):
    _say(f"full-size {s.name} T={T}: building device layer")
    dl = device_layer(s)
    xb = syn.tokens(s, T)
    rl = moe.Layer(router_w=syn.router_weight(s), router_b=syn.router_bias(s),
                   gu_codes=np.zeros((s.E, 2, 1), np.uint8), gu_scales=None, gu_bias=None,
                   dn_codes=None, dn_scales=None, dn_bias=None, k=s.k)
    r = moe.route(rl, xb)
    _say(f"min k/k+1 logit gap {min_topk_gap(r, s.k):.3e}")
    return dl, xb, r


def _sorted_positions(r, R):
    pos = np.empty(R, np.int64)
    pos[r.sorted_rows] = np.arange(R)
    return pos


def _whole_layer(name, T=None):
    """Every token and every routed row of the layer against the oracle."""
    s = syn.spec(name) if T is None else syn.spec(name, T=T)
    T = s.T
    dl, xb, r = _device_and_routing(s, T)
    x = bf16_tensor(xb).to(DEV)
    out, sv = mxfp4_moe_forward(dl, x, saved=True)
    dyb = syn.upstream_grad(s, T)
    dx, _, _ = mxfp4_moe_backward_dx(dl, sv, bf16_tensor(dyb).to(DEV))
    torch.cuda.synchronize()
    assert_routing_equal(sv, r)
    touched = np.unique(r.idx)
    _say(f"oracle: {len(touched)} experts, all {T} tokens")
    ol, _ = oracle_layer(s, experts=touched, threads=16)
    assert_bytes_equal(dl, ol, touched)
    cache_dequant(ol, touched)
    ref, _, cache = moe.forward(ol, xb, routing=r)
    assert_close(to_f64(out), ref, "out (all tokens)")
    rows = r.sorted_rows
    assert_close(to_f64(sv.h), np.stack([cache[int(f)][0] for f in rows]), "saved h (all rows)")
    assert_close(to_f64(sv.a), np.stack([cache[int(f)][1] for f in rows]), "saved a (all rows)")
    del cache
    _say("oracle backward")
    dref, _, _ = moe.backward_dx(ol, xb, dyb, routing=r)
    assert_close(to_f64(dx), dref, "dX (all tokens)")
    assert torch.isfinite(out.float()).all() and torch.isfinite(dx.float()).all()


@pytest.mark.timeout(900)
def test_gpt_oss_20b_layer_2048_tokens():
    _whole_layer("20b_2048")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [1, 8, 64])
def test_gpt_oss_20b_layer_decode(T):
    _whole_layer("20b_decode", T=T)


@pytest.mark.timeout(900)
def test_gpt_oss_120b_layer_zipf_8192_tokens():
    s = syn.spec("120b_8192_zipf")
    T = s.T
    dl, xb, r = _device_and_routing(s, T)
    x = bf16_tensor(xb).to(DEV)
    out, sv = mxfp4_moe_forward(dl, x, saved=True)
    dyb = syn.upstream_grad(s, T)
    dx, _, _ = mxfp4_moe_backward_dx(dl, sv, bf16_tensor(dyb).to(DEV))
    torch.cuda.synchronize()
    assert_routing_equal(sv, r)
    hist = np.diff(r.offsets)
    e_hot = int(np.argmax(hist))
    single = np.nonzero((hist > 32) & (hist <= 128))[0]
    e_one = int(single[0]) if len(single) else int(np.nonzero(hist > 0)[0][-1])
    assert hist[e_hot] > 20 * 128 and hist[e_hot] % 128 != 0
    rng = np.random.default_rng(0)
    toks = np.sort(rng.choice(T, size=4, replace=False))
    need = np.union1d(np.unique(r.idx[toks]), [e_hot, e_one])
    _say(f"hottest expert {e_hot} ({hist[e_hot]} rows), single-tile expert {e_one} "
         f"({hist[e_one]} rows); oracle over {len(need)} experts")
    ol, _ = oracle_layer(s, experts=need, threads=16)
    assert_bytes_equal(dl, ol, need)
    cache_dequant(ol, need)
    pos = _sorted_positions(r, T * s.k)
    h_gpu, a_gpu = to_f64(sv.h), to_f64(sv.a)
    for e in (e_hot, e_one):
        _, _, cache = moe.forward(ol, xb, routing=r, experts=[e])
        fl = np.array(sorted(cache.keys()))
        assert len(fl) == hist[e]
        p = pos[fl]
        assert_close(h_gpu[p], np.stack([cache[int(f)][0] for f in fl]), f"saved h (expert {e}, all rows)")
        assert_close(a_gpu[p], np.stack([cache[int(f)][1] for f in fl]), f"saved a (expert {e}, all rows)")
        del cache
    ref, _, _ = moe.forward(ol, xb, tokens=toks, routing=r)
    assert_close(to_f64(out)[toks], ref[toks], "out (sampled tokens)")
    dref, _, _ = moe.backward_dx(ol, xb, dyb, tokens=toks, routing=r)
    assert_close(to_f64(dx)[toks], dref[toks], "dX (sampled tokens)")
    assert torch.isfinite(out.float()).all() and torch.isfinite(dx.float()).all()


@pytest.mark.timeout(900)
def test_gpt_oss_20b_layer_16384_tokens_lora_checkpointing():
    # Gradient checkpointing: a forward whose activations are dropped, the
    # recompute forward that saves them, then dX + dA/dB.  The recompute
    # must reproduce the first pass bit for bit (routing, permutation, h, a,
    # the adapter projection v and out).
    from mxfp4_weight_mixture_02_amd import SavedState
    s = syn.spec("20b_16384_lora")
    T = s.T
    dl, xb, r = _device_and_routing(s, T)
    x = bf16_tensor(xb).to(DEV)
    _say("forward (activations dropped)")
    out0, _ = mxfp4_moe_forward(dl, x, saved=None)
    out1, sv1 = mxfp4_moe_forward(dl, x, saved=True)
    _say("recompute forward")
    sv2 = SavedState.empty(dl, T, DEV)
    out2, _ = mxfp4_moe_forward(dl, x, saved=sv2)
    torch.cuda.synchronize()
    assert torch.equal(out0.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    for n in ("topk_idx", "topk_w", "expert_offsets", "sorted_rows", "h", "a", "lora_v"):
        assert torch.equal(getattr(sv1, n).view(torch.uint8), getattr(sv2, n).view(torch.uint8)), n
    del sv1
    assert_routing_equal(sv2, r)
    _say("backward")
    dyb = syn.upstream_grad(s, T)
    dx, dA, dB = mxfp4_moe_backward_dx(dl, sv2, bf16_tensor(dyb).to(DEV))
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    toks = np.sort(rng.choice(T, size=64, replace=False))
    hist = np.diff(r.offsets)
    e_full = int(np.argmin(np.where(hist > 0, hist, np.iinfo(np.int64).max)))
    need = np.union1d(np.unique(r.idx[toks]), [e_full])
    _say(f"oracle over {len(need)} experts: 64 tokens, adapter gradients of expert {e_full} "
         f"({hist[e_full]} rows)")
    ol, _ = oracle_layer(s, experts=need, threads=16)
    assert_bytes_equal(dl, ol, need)
    cache_dequant(ol, need)
    ref, _, cache = moe.forward(ol, xb, tokens=toks, routing=r)
    assert_close(to_f64(out2)[toks], ref[toks], "out (64 tokens)")
    pos = _sorted_positions(r, T * s.k)
    fl = np.array(sorted(cache.keys()))
    aref = np.stack([cache[int(f)][1] for f in fl])
    assert_close(to_f64(sv2.a)[pos[fl]], aref, "saved a (64 tokens)")
    assert_close(to_f64(sv2.h)[pos[fl]], np.stack([cache[int(f)][0] for f in fl]), "saved h (64 tokens)")
    ef = np.searchsorted(r.offsets, pos[fl], side="right") - 1
    vref = np.stack([moe._lora_v(ol, ef[i], aref[i][None])[0] for i in range(len(fl))])
    assert_close(to_f64(sv2.lora_v)[pos[fl]], vref, "saved lora_v (64 tokens)")
    dref, _, _ = moe.backward_dx(ol, xb, dyb, tokens=toks, routing=r, want_lora=False)
    assert_close(to_f64(dx)[toks], dref[toks], "dX (64 tokens)")
    _, dAr, dBr = moe.backward_dx(ol, xb, dyb, routing=r, experts=[e_full])
    assert_close(to_f64(dA[e_full]), dAr[e_full], "dA (one expert, all rows)")
    assert_close(to_f64(dB[e_full]), dBr[e_full], "dB (one expert, all rows)")
    # every expert: <dA, A> = <dB, B> (both are s * dL/ds)
    ipA = float((dA.double() * dl.lora_A.double()).sum())
    ipB = float((dB.double() * dl.lora_B.double()).sum())
    assert abs(ipA - ipB) <= 1e-2 * max(abs(ipA), abs(ipB)), (ipA, ipB)
    assert torch.isfinite(out2.float()).all() and torch.isfinite(dx.float()).all()
