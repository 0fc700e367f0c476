"""Shared pieces of the GPU parity tests: device layers built from the
seeded generators (quantised by the HIP quantizer), oracle layers built
from the same fp32 draws (quantised by the oracle), and the comparison
rules."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import moe_synth as syn
from mxfp4_weight_mixture_02_amd import MoeLayer, mxfp4_quantize
from oracle import moe, mxfp4

DEV = "cuda:0"

# Tolerance for floating-point results against the float64 oracle:
# normwise max relative error and cosine over the flattened tensor.
MAX_REL = 2e-2
MIN_COS = 0.9999


def bf16_tensor(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(got, ref, what, max_rel=MAX_REL, min_cos=MIN_COS):
    g = np.asarray(got, dtype=np.float64).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    scale = np.abs(r).max()
    rel = np.abs(g - r).max() / scale if scale > 0 else np.abs(g).max()
    cos = float(g @ r / (np.linalg.norm(g) * np.linalg.norm(r))) if scale > 0 else 1.0
    print(f"{what}: max_rel={rel:.3e} cos={cos:.8f}", flush=True)
    assert rel <= max_rel and cos >= min_cos, f"{what}: max_rel={rel:.3e} cos={cos:.8f}"
    return rel, cos


def device_layer(s, with_bias=True, threads=8, experts=None):
    """Weights drawn per expert, quantised on the GPU by mxfp4_quantize."""
    E = s.E
    gu_c = torch.empty((E, 2 * s.I, s.H // 2), dtype=torch.uint8, device=DEV)
    gu_s = torch.empty((E, 2 * s.I, s.H // 32), dtype=torch.uint8, device=DEV)
    dn_c = torch.empty((E, s.H, s.I // 2), dtype=torch.uint8, device=DEV)
    dn_s = torch.empty((E, s.H, s.I // 32), dtype=torch.uint8, device=DEV)

    def draw(e):
        return syn.gate_up_weight(s, e), syn.down_weight(s, e)

    with ThreadPoolExecutor(threads) as ex:
        for e, (gw, dw) in enumerate(ex.map(draw, range(E))):
            c, sc = mxfp4_quantize(torch.from_numpy(gw).to(DEV))
            gu_c[e].copy_(c)
            gu_s[e].copy_(sc)
            c, sc = mxfp4_quantize(torch.from_numpy(dw).to(DEV))
            dn_c[e].copy_(c)
            dn_s[e].copy_(sc)
    L = MoeLayer(
        router_w=torch.from_numpy(syn.router_weight(s)).to(DEV),
        router_b=torch.from_numpy(syn.router_bias(s)).to(DEV),
        gu_codes=gu_c, gu_scales=gu_s,
        gu_bias=bf16_tensor(syn.gate_up_bias(s)).to(DEV) if with_bias else None,
        dn_codes=dn_c, dn_scales=dn_s,
        dn_bias=bf16_tensor(syn.down_bias(s)).to(DEV) if with_bias else None,
        k=s.k, alpha=s.swiglu_alpha, limit=s.swiglu_limit)
    if s.lora_rank and s.lora_down:
        L.lora_A = bf16_tensor(syn.lora_a(s)).to(DEV)
        L.lora_B = bf16_tensor(syn.lora_b(s)).to(DEV)
    if s.lora_rank and s.lora_gate_up:
        L.lora_gu_A = bf16_tensor(syn.lora_gu_a(s)).to(DEV)
        L.lora_gu_B = bf16_tensor(syn.lora_gu_b(s)).to(DEV)
    return L


def oracle_layer(s, experts=None, with_bias=True, threads=8):
    """Oracle-quantised layer; with ``experts`` only those experts are
    quantised (the rest stay zero and must not be used)."""
    E = s.E
    experts = list(range(E)) if experts is None else sorted(set(int(e) for e in experts))
    gu_c = np.zeros((E, 2 * s.I, s.H // 2), np.uint8)
    gu_s = np.zeros((E, 2 * s.I, s.H // 32), np.uint8)
    dn_c = np.zeros((E, s.H, s.I // 2), np.uint8)
    dn_s = np.zeros((E, s.H, s.I // 32), np.uint8)

    def one(e):
        return e, mxfp4.quantize(syn.gate_up_weight(s, e)), mxfp4.quantize(syn.down_weight(s, e))

    with ThreadPoolExecutor(threads) as ex:
        for e, (gc, gs), (dc, ds) in ex.map(one, experts):
            gu_c[e], gu_s[e], dn_c[e], dn_s[e] = gc, gs, dc, ds
    L = moe.Layer(router_w=syn.router_weight(s), router_b=syn.router_bias(s),
                  gu_codes=gu_c, gu_scales=gu_s,
                  gu_bias=syn.gate_up_bias(s) if with_bias else None,
                  dn_codes=dn_c, dn_scales=dn_s,
                  dn_bias=syn.down_bias(s) if with_bias else None,
                  k=s.k, alpha=s.swiglu_alpha, limit=s.swiglu_limit)
    if s.lora_rank and s.lora_down:
        L.lora_A = syn.lora_a(s)
        L.lora_B = syn.lora_b(s)
    if s.lora_rank and s.lora_gate_up:
        L.lora_gu_A = syn.lora_gu_a(s)
        L.lora_gu_B = syn.lora_gu_b(s)
    return L, experts


def cache_dequant(ol: moe.Layer, experts, threads=16):
    """Dequantize the given experts' weights once, in parallel, with the
    oracle's own ``dequantize``, and make ``ol.gate_up(e)`` / ``ol.down(e)``
    return those arrays (the forward and the backward would otherwise
    decode every expert again; the arithmetic is unchanged)."""
    experts = sorted(set(int(e) for e in experts))

    def one(e):
        return e, mxfp4.dequantize(ol.gu_codes[e], ol.gu_scales[e]), \
            mxfp4.dequantize(ol.dn_codes[e], ol.dn_scales[e])

    gu, dn = {}, {}
    with ThreadPoolExecutor(threads) as ex:
        for e, g, d in ex.map(one, experts):
            gu[e], dn[e] = g, d
    ol.gate_up = gu.__getitem__
    ol.down = dn.__getitem__
    return ol


def assert_bytes_equal(dl, ol, experts=None):
    """The GPU quantizer's codes and scales equal the oracle's, byte for
    byte, on every listed expert (all by default), for both projections."""
    experts = range(ol.E) if experts is None else experts
    for name in ("gu_codes", "gu_scales", "dn_codes", "dn_scales"):
        g = getattr(dl, name)
        r = getattr(ol, name)
        for e in experts:
            assert np.array_equal(g[e].cpu().numpy(), r[e]), f"{name}[{e}] differs"


def assert_routing_equal(saved, r: moe.Routing):
    """Indices, offsets and the permutation are integers: bit-exact.  The
    routing weights are floats: tolerance."""
    idx = saved.topk_idx.cpu().numpy()
    assert np.array_equal(idx, r.idx), f"topk_idx differs at {np.argwhere(idx != r.idx)[:5]}"
    assert np.array_equal(saved.expert_offsets.cpu().numpy(), r.offsets)
    assert np.array_equal(saved.sorted_rows.cpu().numpy(), r.sorted_rows)
    np.testing.assert_allclose(saved.topk_w.cpu().numpy(), r.w, rtol=2e-6, atol=1e-7)


def min_topk_gap(r: moe.Routing, k):
    """Smallest gap between the k-th and (k+1)-th logit (diagnostic)."""
    l = np.sort(r.logits.astype(np.float64), axis=1)[:, ::-1]
    if l.shape[1] <= k:
        return np.inf
    return float((l[:, k - 1] - l[:, k]).min())
