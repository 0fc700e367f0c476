"""Host-side refusals of the Python binding (no GPU needed).

The C ABI receives only pointers, so a tensor of the wrong shape would make
the kernels read or write out of bounds; the binding therefore checks every
shape and dtype first, on any device, and only then that the tensors live
on the GPU.  These tests build layers from CPU tensors: a wrong shape must
be refused by name, and a right one must get as far as the device check.
"""
import pytest
import torch

from mxfp4_weight_mixture_02_amd import native
from mxfp4_weight_mixture_02_amd.native import MoeLayer, SavedState

E, H, I, K, R_LORA = 4, 64, 96, 2, 16


def _layer(lora=False, **repl):
    u8, bf = torch.uint8, torch.bfloat16
    t = dict(
        router_w=torch.zeros(E, H), router_b=torch.zeros(E),
        gu_codes=torch.zeros(E, 2 * I, H // 2, dtype=u8), gu_scales=torch.zeros(E, 2 * I, H // 32, dtype=u8),
        gu_bias=torch.zeros(E, 2 * I, dtype=bf),
        dn_codes=torch.zeros(E, H, I // 2, dtype=u8), dn_scales=torch.zeros(E, H, I // 32, dtype=u8),
        dn_bias=torch.zeros(E, H, dtype=bf))
    if lora:
        t["lora_A"] = torch.zeros(E, R_LORA, I, dtype=bf)
        t["lora_B"] = torch.zeros(E, H, R_LORA, dtype=bf)
    t.update(repl)
    return MoeLayer(k=K, **t)


def _saved(T, lora=False, **repl):
    R = T * K
    t = dict(topk_idx=torch.zeros(T, K, dtype=torch.int32), topk_w=torch.zeros(T, K),
             expert_offsets=torch.zeros(E + 1, dtype=torch.int32),
             sorted_rows=torch.zeros(R, dtype=torch.int32),
             h=torch.zeros(R, 2 * I, dtype=torch.bfloat16), a=torch.zeros(R, I, dtype=torch.bfloat16),
             lora_v=torch.zeros(R, R_LORA) if lora else None)
    t.update(repl)
    return SavedState(**t)


def _x(T=5):
    return torch.zeros(T, H, dtype=torch.bfloat16)


def _refused(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_well_formed_cpu_call_reaches_the_device_check():
    _refused("CUDA tensor", native.mxfp4_moe_forward, _layer(), _x())
    _refused("CUDA tensor", native.mxfp4_moe_backward_dx, _layer(), _saved(5), _x())


@pytest.mark.parametrize("name,bad", [
    ("router_w", torch.zeros(E, H + 1)),
    ("router_w", torch.zeros(E, H, dtype=torch.float64)),
    ("router_b", torch.zeros(E + 1)),
    ("gu_scales", torch.zeros(E, 2 * I, H // 32 + 1, dtype=torch.uint8)),
    ("gu_bias", torch.zeros(E, I, dtype=torch.bfloat16)),
    ("gu_bias", torch.zeros(E, 2 * I)),
    ("dn_codes", torch.zeros(E, H, I, dtype=torch.uint8)),
    ("dn_scales", torch.zeros(E, H - 1, I // 32, dtype=torch.uint8)),
    ("dn_bias", torch.zeros(E - 1, H, dtype=torch.bfloat16)),
])
def test_layer_parameter_shapes(name, bad):
    _refused(name, native.mxfp4_moe_forward, _layer(**{name: bad}), _x())


def test_gate_up_codes_define_the_layer():
    _refused("gu_codes", native.mxfp4_moe_forward,
             _layer(gu_codes=torch.zeros(E, 2 * I, dtype=torch.uint8)), _x())


def test_lora_shapes():
    _refused("lora_A and lora_B", native.mxfp4_moe_forward,
             _layer(lora_A=torch.zeros(E, R_LORA, I, dtype=torch.bfloat16)), _x())
    _refused("lora_B", native.mxfp4_moe_forward,
             _layer(lora=True, lora_B=torch.zeros(E, H, R_LORA + 1, dtype=torch.bfloat16)), _x())
    _refused("lora_A", native.mxfp4_moe_forward,
             _layer(lora=True, lora_A=torch.zeros(E, R_LORA, I + 32, dtype=torch.bfloat16)), _x())


def test_activation_shapes():
    L = _layer()
    _refused("x must be", native.mxfp4_moe_forward, L, torch.zeros(H, dtype=torch.bfloat16))
    _refused("x:", native.mxfp4_moe_forward, L, torch.zeros(5, H + 32, dtype=torch.bfloat16))
    _refused("x:", native.mxfp4_moe_forward, L, torch.zeros(5, H))
    _refused("out", native.mxfp4_moe_forward, L, _x(5), out=_x(6))
    _refused("dy:", native.mxfp4_moe_backward_dx, L, _saved(5), torch.zeros(5, H + 32, dtype=torch.bfloat16))
    _refused("dx", native.mxfp4_moe_backward_dx, L, _saved(5), _x(5), dx=_x(4))


@pytest.mark.parametrize("name,bad", [
    ("topk_idx", torch.zeros(5, K + 1, dtype=torch.int32)),
    ("topk_w", torch.zeros(5, K, dtype=torch.float64)),
    ("expert_offsets", torch.zeros(E, dtype=torch.int32)),
    ("sorted_rows", torch.zeros(5 * K - 1, dtype=torch.int32)),
    ("h", torch.zeros(5 * K, I, dtype=torch.bfloat16)),
    ("a", torch.zeros(5 * K, 2 * I, dtype=torch.bfloat16)),
])
def test_saved_state_shapes(name, bad):
    L = _layer()
    sv = _saved(5, **{name: bad})
    _refused(f"saved.{name}", native.mxfp4_moe_forward, L, _x(5), saved=sv)
    _refused(f"saved.{name}", native.mxfp4_moe_backward_dx, L, sv, _x(5))


def test_saved_state_must_match_the_token_count():
    # a backward whose dy has more tokens than the forward saved
    _refused("saved.topk_idx", native.mxfp4_moe_backward_dx, _layer(), _saved(5), _x(6))


def test_lora_saved_state_and_gradients():
    L = _layer(lora=True)
    _refused("saved.lora_v", native.mxfp4_moe_backward_dx, L, _saved(5), _x(5))
    sv = _saved(5, lora=True)
    _refused("dA", native.mxfp4_moe_backward_dx, L, sv, _x(5),
             dA=torch.zeros(E, R_LORA, I + 1))
    _refused("dB", native.mxfp4_moe_backward_dx, L, sv, _x(5),
             dB=torch.zeros(E, H, R_LORA, dtype=torch.float64))
    _refused("CUDA tensor", native.mxfp4_moe_backward_dx, L, sv, _x(5))
