"""Builds oracle-side layers from the seeded generators (test helper)."""
import numpy as np

import moe_synth as syn
from oracle import moe, mxfp4


def quantized_experts(s, experts=None):
    """Oracle-quantized expert weights: (gu_codes, gu_scales, dn_codes,
    dn_scales), each with a leading expert axis over ``experts``."""
    experts = list(range(s.E)) if experts is None else list(experts)

    def one(e):
        gc, gs = mxfp4.quantize(syn.gate_up_weight(s, e))
        dc, ds = mxfp4.quantize(syn.down_weight(s, e))
        return gc, gs, dc, ds

    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(8) as ex:
        parts = list(ex.map(one, experts))
    return tuple(np.stack([p[i] for p in parts]) for i in range(4))


def oracle_layer(s, with_bias=True, **kw) -> moe.Layer:
    gc, gs, dc, ds = quantized_experts(s)
    L = moe.Layer(
        router_w=syn.router_weight(s), router_b=syn.router_bias(s),
        gu_codes=gc, gu_scales=gs, gu_bias=syn.gate_up_bias(s) if with_bias else None,
        dn_codes=dc, dn_scales=ds, dn_bias=syn.down_bias(s) if with_bias else None,
        k=s.k, alpha=s.swiglu_alpha, limit=s.swiglu_limit)
    if s.lora_rank and s.lora_down:
        L.lora_A = syn.lora_a(s)
        L.lora_B = syn.lora_b(s)
    if s.lora_rank and s.lora_gate_up:
        L.lora_gu_A = syn.lora_gu_a(s)
        L.lora_gu_B = syn.lora_gu_b(s)
    for key, v in kw.items():
        setattr(L, key, v)
    return L
