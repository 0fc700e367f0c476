"""The forward that allocates nothing (mxfp4_moe_forward_noalloc, scratch in
a static device array of the library) against mxfp4_moe_forward with a
workspace, through the C ABI.  The two run the same kernels, so their
results must agree bit for bit.  Each case makes two calls in a row, the
second with fewer tokens: the static scratch keeps the first call's
contents, and none of them may leak into the second."""
import numpy as np
import pytest
import torch

import moe_synth as syn
from mxfp4_weight_mixture_02_amd import (Mxfp4Error, SavedState, Workspace, mxfp4_moe_forward,
                                         mxfp4_moe_forward_noalloc)

from gpu_helpers import DEV, bf16_tensor, device_layer

pytestmark = pytest.mark.gpu

SAVED = ("topk_idx", "topk_w", "expert_offsets", "sorted_rows", "h", "a", "lora_v")


def _same(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def _check(dl, s, T, saved):
    print(f"no-alloc forward {s.name} T={T} saved={saved}", flush=True)
    x = bf16_tensor(syn.tokens(s, T)).to(DEV)
    ref_sv = SavedState.empty(dl, T, DEV) if saved else None
    ref, _ = mxfp4_moe_forward(dl, x, saved=ref_sv, workspace=Workspace())
    out = torch.full_like(x, float("nan"))
    sv = SavedState.empty(dl, T, DEV) if saved else None
    if sv is not None:
        for n in SAVED:
            t = getattr(sv, n)
            if t is not None:
                t.view(torch.uint8).fill_(0xFF)
    got = mxfp4_moe_forward_noalloc(dl, x, out, saved=sv)
    torch.cuda.synchronize()
    assert got is out
    assert _same(out, ref), "out differs"
    if saved:
        for n in SAVED:
            if getattr(ref_sv, n) is not None:
                assert _same(getattr(sv, n), getattr(ref_sv, n)), n


@pytest.mark.parametrize("saved", [False, True])
def test_tiny_layer_two_calls(saved):
    s = syn.spec("tiny", T=40, E=16, k=4)
    dl = device_layer(s)
    _check(dl, s, 40, saved)
    _check(dl, s, 7, saved)


def test_tiny_lora_layer_two_calls():
    s = syn.spec("tiny", T=300, H=192, I=320, E=3, k=2, lora_rank=16)
    dl = device_layer(s)
    _check(dl, s, 300, True)
    _check(dl, s, 33, True)


def test_gpt_oss_20b_layer_decode_and_prefill_two_calls():
    s = syn.spec("20b_decode")
    dl = device_layer(s)
    _check(dl, s, 64, False)      # decode-size kernels
    _check(dl, s, 8, False)
    _check(dl, s, 300, True)      # general GEMMs, close to the scratch limit
    _check(dl, s, 1, True)
    # a forward whose scratch would exceed the static array is refused
    x = bf16_tensor(syn.tokens(s, 2048)).to(DEV)
    with pytest.raises(Mxfp4Error, match="EUNSUPPORTED"):
        mxfp4_moe_forward_noalloc(dl, x, torch.empty_like(x))
