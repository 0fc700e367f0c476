"""Seeded synthetic inputs for the MXFP4 MoE expert block.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no quantisation, no routing, no expert math).  Both the
CPU oracle and the HIP path are fed from here, so that the two sides see the
same fp32 weights, the same bf16 activations and the same upstream gradients.

Shapes follow the GPT-OSS MoE layer the pages discuss (gpt-oss-20b: hidden
2880, intermediate 2880, 32 experts, top-4; gpt-oss-120b: 128 experts), as
listed in ``CONFIGS``.  Distributions:

* activations x and upstream gradient dY: N(0, 1), drawn in fp32 and rounded
  to bf16 (round to nearest even);
* router weight: N(0, 0.02) fp32 [E, H]; router bias zero, except the
  skewed-routing layer, whose bias is log of a Zipf(s) pmf over expert rank
  e + 1 (up to a constant): b[e] = -s * ln(e + 1);
* expert weights: N(0, 0.02) fp32, gate_up [E, 2I, H] with gate j at row 2j
  and up j at row 2j + 1 (the rows are simply drawn in that order), down
  [E, H, I]; they are handed out per expert so that no more than one expert's
  fp32 weights need to exist at a time;
* expert biases: N(0, 0.01), rounded to bf16, gate_up bias [E, 2I] (same
  interleaved row order) and down bias [E, H];
* LoRA adapters on the down projection: A [E, r, I] and B [E, H, r],
  N(0, 0.01), rounded to bf16.

Every tensor has its own PCG64 stream, keyed by (layer seed, tensor name,
expert), so any expert can be regenerated alone.
"""
from __future__ import annotations

import hashlib
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

__all__ = ["LayerSpec", "CONFIGS", "DECODE_TOKENS", "spec", "rng",
           "bf16_bits", "f32_from_bf16_bits", "router_weight", "router_bias",
           "gate_up_weight", "down_weight", "gate_up_bias", "down_bias",
           "lora_a", "lora_b", "lora_gu_a", "lora_gu_b", "tokens", "upstream_grad", "all_experts"]


@dataclass(frozen=True)
class LayerSpec:
    name: str
    T: int            # tokens
    H: int            # hidden size (K of gate_up, N of down)
    I: int            # intermediate size (gate_up has 2I rows)
    E: int            # experts
    k: int            # experts per token
    seed: int         # weight seed (decode shares the 20b layer's weights)
    zipf_s: float = 0.0      # router-bias skew; 0 = unbiased router
    lora_rank: int = 0       # LoRA rank; 0 = none
    lora_down: bool = True   # with lora_rank: an adapter on the down projection
    lora_gate_up: bool = False   # with lora_rank: an adapter on the gate_up projection
    swiglu_alpha: float = 1.702
    swiglu_limit: float = 7.0
    extra: dict = field(default_factory=dict, compare=False, hash=False)


_BASE = 0x4D5846

#: The five workloads: a tiny layer, the gpt-oss-20b layer at 2048 tokens,
#: the same layer at decode sizes, the gpt-oss-120b layer with skewed routing,
#: and the 20b layer at a 16384-token training step with a rank-16 LoRA.
CONFIGS = {
    "tiny": LayerSpec("tiny", T=16, H=64, I=64, E=4, k=2, seed=_BASE + 0),
    "20b_2048": LayerSpec("20b_2048", T=2048, H=2880, I=2880, E=32, k=4, seed=_BASE + 1),
    "20b_decode": LayerSpec("20b_decode", T=1, H=2880, I=2880, E=32, k=4, seed=_BASE + 1),
    "120b_8192_zipf": LayerSpec("120b_8192_zipf", T=8192, H=2880, I=2880, E=128, k=4,
                                seed=_BASE + 3, zipf_s=1.1),
    "20b_16384_lora": LayerSpec("20b_16384_lora", T=16384, H=2880, I=2880, E=32, k=4,
                                seed=_BASE + 1, lora_rank=16),
}
DECODE_TOKENS = (1, 8, 64)


def spec(name: str, **overrides) -> LayerSpec:
    """The named layer, optionally with fields replaced (e.g. T for decode)."""
    s = CONFIGS[name]
    if not overrides:
        return s
    d = {f: getattr(s, f) for f in s.__dataclass_fields__ if f != "extra"}
    d.update(overrides)
    return LayerSpec(**d)


def rng(seed: int, tensor: str, index: int = 0) -> np.random.Generator:
    """Independent PCG64 stream for (seed, tensor name, index)."""
    key = int.from_bytes(hashlib.sha256(tensor.encode()).digest()[:4], "little")
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, key, index])))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even.  Inputs here
    are finite draws, so NaN handling is not needed."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(seed, tensor, index, shape, std):
    g = rng(seed, tensor, index)
    return g.standard_normal(shape, dtype=np.float32) * np.float32(std)


def router_weight(s: LayerSpec) -> np.ndarray:
    return _normal(s.seed, "router_w", 0, (s.E, s.H), 0.02)


def router_bias(s: LayerSpec) -> np.ndarray:
    if s.zipf_s == 0.0:
        return np.zeros(s.E, dtype=np.float32)
    return (-s.zipf_s * np.log(np.arange(1, s.E + 1, dtype=np.float64))).astype(np.float32)


def gate_up_weight(s: LayerSpec, e: int) -> np.ndarray:
    """fp32 [2I, H] of expert e; row 2j is gate j, row 2j+1 is up j."""
    return _normal(s.seed, "gu_w", e, (2 * s.I, s.H), 0.02)


def down_weight(s: LayerSpec, e: int) -> np.ndarray:
    """fp32 [H, I] of expert e."""
    return _normal(s.seed, "dn_w", e, (s.H, s.I), 0.02)


def gate_up_bias(s: LayerSpec) -> np.ndarray:
    """bf16 bits [E, 2I], interleaved like the gate_up rows."""
    return bf16_bits(_normal(s.seed, "gu_b", 0, (s.E, 2 * s.I), 0.01))


def down_bias(s: LayerSpec) -> np.ndarray:
    return bf16_bits(_normal(s.seed, "dn_b", 0, (s.E, s.H), 0.01))


def lora_a(s: LayerSpec) -> np.ndarray:
    """bf16 bits [E, r, I]."""
    return bf16_bits(_normal(s.seed, "lora_A", 0, (s.E, s.lora_rank, s.I), 0.01))


def lora_b(s: LayerSpec) -> np.ndarray:
    """bf16 bits [E, H, r]."""
    return bf16_bits(_normal(s.seed, "lora_B", 0, (s.E, s.H, s.lora_rank), 0.01))


def lora_gu_a(s: LayerSpec) -> np.ndarray:
    """bf16 bits [E, r, H] (the gate_up adapter's A)."""
    return bf16_bits(_normal(s.seed, "lora_gu_A", 0, (s.E, s.lora_rank, s.H), 0.01))


def lora_gu_b(s: LayerSpec) -> np.ndarray:
    """bf16 bits [E, 2I, r] (rows in the interleaved gate|up order)."""
    return bf16_bits(_normal(s.seed, "lora_gu_B", 0, (s.E, 2 * s.I, s.lora_rank), 0.01))


def tokens(s: LayerSpec, T: int | None = None, scale: float = 1.0) -> np.ndarray:
    """bf16 bits [T, H] of N(0, scale^2) activations.  Each token count has
    its own stream (decode sizes do not share prefixes)."""
    T = s.T if T is None else T
    return bf16_bits(_normal(s.seed, "x", T, (T, s.H), scale))


def upstream_grad(s: LayerSpec, T: int | None = None) -> np.ndarray:
    T = s.T if T is None else T
    return bf16_bits(_normal(s.seed, "dY", T, (T, s.H), 1.0))


def all_experts(fn, s: LayerSpec, experts=None, threads: int = 8):
    """[fn(s, e) for e in experts], drawn on a small thread pool."""
    experts = range(s.E) if experts is None else experts
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(lambda e: fn(s, e), experts))
