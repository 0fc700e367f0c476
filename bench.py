#!/usr/bin/env python3
"""Throughput of the MXFP4 MoE expert block on one MI355X.

A step is one pass of the whole hot path on the gpt-oss-20b-shaped layer
(2048 tokens, hidden 2880, intermediate 2880, 32 experts, top-4, MXFP4
expert weights): the forward with saved state (router, permutation, gate_up
+ SwiGLU, down + weighted combine) followed by the dX backward.  Inputs
and weights are synthetic (seeded, the layer's real shapes) and resident in
HBM before the timed region.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode]

Prints one JSON line.  `value` is forward + dX TFLOP/s counting the expert
GEMMs' algorithmic flops (2 * T*k * 3 * H * I per pass, two passes); the
line also carries the forward-only rate, the decode-size weight-streaming
rates (GB/s over the packed weights and scales of the experts a step
touches, eight rotating weight copies so that nothing is served from the
last-level cache; timed as HIP-graph replays of eight forwards, with the
eager per-call time beside it), per-kernel times, the roofline entry of the dominant
kernel (timed with HIP events on the library's stream) and the CPU
oracle's rate on a bounded sample.
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("MoE layer TFLOP/s fwd & fwd+dX-bwd (gpt-oss-20b shape, 2048 tok); decode GB/s")
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=16)
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the 120b skewed-routing and 16384-token LoRA workloads")
    ap.add_argument("--act-format", default="bf16", choices=("bf16", "mxfp8", "mxfp8x2"),
                    help="what the gate_up product consumes in the timed step (the headline "
                         "is bf16; the block-scaled formats are for profiling runs)")
    ap.add_argument("--profile", action="store_true",
                    help="for rocprofv3 runs: one 256 MiB device-to-device copy (a known-size "
                         "calibration for the traffic counters), then warmup + steps of the "
                         "forward + dX step, nothing else")
    return ap.parse_args()


# HBM bytes per launch of the GEMM kernels from rocprofv3 FETCH_SIZE and
# WRITE_SIZE (scaled by the 256 MiB copy calibration: reads 2.0x, writes
# 1.0x), taken on the kernel source whose SHA-256 prefixes are recorded
# (the kernel's file and the shared device header); the figure is reported
# only while both are unchanged.
TRAFFIC = {
    # kernel: (source file, SHA-256 prefix of that file and of common.hpp, bytes per launch)
    "gate_up": ("gemm_fwd.hip", "1230d0aed3c0ae8b", "94b6aea9d96e712b", 610.8e6),
    "down": ("gemm_fwd.hip", "1230d0aed3c0ae8b", "94b6aea9d96e712b", 276.7e6),
    "bwd_down": ("gemm_bwd.hip", "e59007daef61b8b1", "94b6aea9d96e712b", 593.8e6),
    "bwd_gate_up": ("gemm_bwd.hip", "e59007daef61b8b1", "94b6aea9d96e712b", 787.2e6),
}


def counted_traffic(kernel):
    import hashlib
    entry = TRAFFIC.get(kernel)
    if entry is None:
        return None
    src, sha, sha_common, nbytes = entry
    csrc = os.path.join(ROOT, "mxfp4_weight_mixture_02_amd", "csrc")
    try:
        cur = hashlib.sha256(open(os.path.join(csrc, src), "rb").read()).hexdigest()[:16]
        cur_common = hashlib.sha256(open(os.path.join(csrc, "common.hpp"), "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    return nbytes if (cur, cur_common) == (sha, sha_common) else None


def kernel_times(lib):
    n = lib.mxfp4_moe_kernel_times(None, None, None, 0)
    names = (ctypes.c_char_p * n)()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int * n)()
    lib.mxfp4_moe_kernel_times(names, ms, cnt, n)
    return {names[i].decode(): (ms[i], cnt[i]) for i in range(n)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_synth as syn
    from mxfp4_weight_mixture_02_amd import (MoeLayer, SavedState, Workspace, lib,
                                             mxfp4_moe_backward_dx, mxfp4_moe_forward,
                                             mxfp4_quantize)

    L = lib()
    L.mxfp4_moe_kernel_timing.argtypes = [ctypes.c_int]
    L.mxfp4_moe_kernel_times.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int]
    dev = "cuda:0"
    s = syn.spec("20b_2048")
    T, H, I, E, k = s.T, s.H, s.I, s.E, s.k
    R = T * k

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- layer: fp32 draws quantised on the GPU, one expert at a time
    gu_c = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=dev)
    gu_s = torch.empty((E, 2 * I, H // 32), dtype=torch.uint8, device=dev)
    dn_c = torch.empty((E, H, I // 2), dtype=torch.uint8, device=dev)
    dn_s = torch.empty((E, H, I // 32), dtype=torch.uint8, device=dev)
    gws = syn.all_experts(syn.gate_up_weight, s)
    for e in range(E):
        c, sc = mxfp4_quantize(torch.from_numpy(gws[e]).to(dev))
        gu_c[e].copy_(c)
        gu_s[e].copy_(sc)
    del gws
    dws = syn.all_experts(syn.down_weight, s)
    for e in range(E):
        c, sc = mxfp4_quantize(torch.from_numpy(dws[e]).to(dev))
        dn_c[e].copy_(c)
        dn_s[e].copy_(sc)
    del dws
    layer = MoeLayer(torch.from_numpy(syn.router_weight(s)).to(dev),
                     torch.from_numpy(syn.router_bias(s)).to(dev), gu_c, gu_s,
                     bf(syn.gate_up_bias(s)), dn_c, dn_s, bf(syn.down_bias(s)), k=k)
    layer.act_format = args.act_format
    x = bf(syn.tokens(s))
    dy = bf(syn.upstream_grad(s))
    saved = SavedState.empty(layer, T, dev)
    out = torch.empty_like(x)
    dx = torch.empty_like(x)
    wsf, wsb = Workspace(), Workspace()

    def step():
        mxfp4_moe_forward(layer, x, saved=saved, out=out, workspace=wsf)
        mxfp4_moe_backward_dx(layer, saved, dy, dx=dx, workspace=wsb)

    flops_pass = 2.0 * R * 3 * H * I
    flops_step = 2 * flops_pass

    if args.profile:
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        for _ in range(args.warmup + args.steps):
            step()
        torch.cuda.synchronize()
        print(json.dumps({"profile_steps": args.steps, "copy_bytes": src.numel() * 4}), flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    value = flops_step / dt / 1e12

    # ---- per-step distribution (HIP events between consecutive steps on the
    # stream the library launches on) and the step as one HIP-graph replay
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per_step = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    step_stats = {"median": round(float(np.median(per_step)), 4),
                  "p10": round(float(np.percentile(per_step, 10)), 4),
                  "p90": round(float(np.percentile(per_step, 90)), 4)}
    gstep = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        with torch.cuda.graph(gstep, stream=cs):
            step()
    torch.cuda.current_stream().wait_stream(cs)
    for _ in range(3):
        gstep.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        gstep.replay()
    torch.cuda.synchronize()
    dt_graph = (time.perf_counter() - t0) / args.steps
    del gstep

    # ---- the same steps with per-kernel HIP events on the library's stream
    L.mxfp4_moe_kernel_timing(1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt_inst = (time.perf_counter() - t0) / args.steps
    kt = kernel_times(L)
    L.mxfp4_moe_kernel_timing(0)
    kernels = {n: round(ms / c * 1e3, 2) for n, (ms, c) in kt.items()}   # us per launch
    gemm_flops = {"gate_up": 2.0 * R * 2 * I * H, "down": 2.0 * R * H * I,
                  "bwd_down": 2.0 * R * H * I, "bwd_gate_up": 2.0 * R * 2 * I * H}
    dom = max(gemm_flops, key=lambda n: kt[n][0])
    avg_s = kt[dom][0] / kt[dom][1] / 1e3
    achieved = gemm_flops[dom] / avg_s / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": counted_traffic(dom), "traffic_unit": "bytes per launch",
                "avg_launch_us": round(avg_s * 1e6, 1),
                "flop_per_launch": gemm_flops[dom]}

    # ---- forward only (inference: no saved state)
    for _ in range(args.warmup):
        mxfp4_moe_forward(layer, x, out=out, workspace=wsf)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        mxfp4_moe_forward(layer, x, out=out, workspace=wsf)
    torch.cuda.synchronize()
    dt_fwd = (time.perf_counter() - t0) / args.steps
    fwd_tflops = flops_pass / dt_fwd / 1e12

    # ---- decode sizes, eight rotating copies of the expert weights
    decode = {}
    if not args.no_decode:
        copies = [layer]
        for _ in range(7):
            copies.append(MoeLayer(layer.router_w, layer.router_b, gu_c.clone(), gu_s.clone(),
                                   layer.gu_bias, dn_c.clone(), dn_s.clone(), layer.dn_bias, k=k))
        per_expert = (2 * I * H // 2 + 2 * I * H // 32) + (H * I // 2 + H * I // 32)
        for Td in syn.DECODE_TOKENS:
            xd = bf(syn.tokens(s, Td))
            wsd = Workspace()
            _, sv = mxfp4_moe_forward(layer, xd, saved=True, workspace=wsd)
            torch.cuda.synchronize()
            touched = int(torch.unique(sv.topk_idx).numel())
            od = torch.empty_like(xd)
            for i in range(16):
                mxfp4_moe_forward(copies[i % 8], xd, out=od, workspace=wsd)
            torch.cuda.synchronize()
            # eager: one Python call per forward (includes the host's launch cost)
            nrep = 8 * max(8, args.steps)
            t0 = time.perf_counter()
            for i in range(nrep):
                mxfp4_moe_forward(copies[i % 8], xd, out=od, workspace=wsd)
            torch.cuda.synchronize()
            dt_eager = (time.perf_counter() - t0) / nrep
            # per-kernel GPU time from the library's events (eager)
            L.mxfp4_moe_kernel_timing(1)
            for i in range(8):
                mxfp4_moe_forward(copies[i % 8], xd, out=od, workspace=wsd)
            kd = {n: round(ms / c * 1e3, 2) for n, (ms, c) in kernel_times(L).items()}
            L.mxfp4_moe_kernel_timing(0)
            # graph replay: the eight forwards (one per weight copy) captured once
            g = torch.cuda.CUDAGraph()
            cs = torch.cuda.Stream()
            cs.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cs):
                with torch.cuda.graph(g, stream=cs):
                    for i in range(8):
                        mxfp4_moe_forward(copies[i], xd, out=od, workspace=wsd)
            torch.cuda.current_stream().wait_stream(cs)
            for _ in range(3):
                g.replay()
            torch.cuda.synchronize()
            ref = od.clone()
            nrep_g = max(8, args.steps)
            t0 = time.perf_counter()
            for _ in range(nrep_g):
                g.replay()
            torch.cuda.synchronize()
            dtd = (time.perf_counter() - t0) / (8 * nrep_g)
            # the replayed result equals an eager forward on the last copy
            mxfp4_moe_forward(copies[7], xd, out=od, workspace=wsd)
            torch.cuda.synchronize()
            assert torch.equal(ref.view(torch.int16), od.view(torch.int16))
            del g
            decode[str(Td)] = {"us": round(dtd * 1e6, 2), "us_eager": round(dt_eager * 1e6, 1),
                               "experts": touched,
                               "GB/s": round(touched * per_expert / dtd / 1e9, 1),
                               "frac_hbm": round(touched * per_expert / dtd / 1e9 / PEAK_HBM_GBS, 4),
                               "kernel_us": kd}
        del copies

    # ---- the gate_up product per activation format (bf16 weight-only, the
    # block-scaled MXFP8 and hi + lo MXFP8 forms), same layer and tokens:
    # event-timed kernels over two passes in opposite orders (the clock
    # drifts), and each forward's distance from the bf16 one
    block_scaled = {}
    if not args.no_extra:
        fmts = ("bf16", "mxfp8", "mxfp8x2")
        acc = {f: {} for f in fmts}
        outs = {}
        for order in (fmts, fmts[::-1]):
            for f in order:
                layer.act_format = f
                for _ in range(5):
                    mxfp4_moe_forward(layer, x, saved=saved, out=out, workspace=wsf)
                torch.cuda.synchronize()
                L.mxfp4_moe_kernel_timing(1)
                for _ in range(10):
                    mxfp4_moe_forward(layer, x, saved=saved, out=out, workspace=wsf)
                torch.cuda.synchronize()
                for n, (ms, c) in kernel_times(L).items():
                    acc[f].setdefault(n, []).append(ms / c * 1e3)
                L.mxfp4_moe_kernel_timing(0)
                outs[f] = out.float().clone()
        layer.act_format = args.act_format
        ref = outs["bf16"]
        for f in fmts:
            g = outs[f]
            kt = {n: sum(v) / len(v) for n, v in acc[f].items()}
            block_scaled[f] = {
                "gate_up_kernel": "mx_gate_up" if f != "bf16" else "gate_up",
                "gate_up_us": round(kt.get("mx_gate_up", kt.get("gate_up", 0.0)), 1),
                "act_quantize_us": round(kt.get("act_quantize", 0.0), 1),
                "max_rel_vs_bf16": float(f"{float((g - ref).abs().max() / ref.abs().max()):.3e}"),
                "cos_vs_bf16": round(float((g * ref).sum() / (g.norm() * ref.norm())), 8)}

    # ---- the other full-size workloads (not the headline): the gpt-oss-120b
    # layer with Zipf-skewed routing (forward + dX) and the 16384-token LoRA
    # training step (forward, recompute forward, dX backward with dA/dB)
    extra = {}
    if not args.no_extra:
        del saved, wsf, wsb
        torch.cuda.empty_cache()
        extra["120b_8192_zipf_fwd_dx"] = extra_workload(
            syn.spec("120b_8192_zipf"), args, lora=False)
        extra["20b_16384_lora_train_step"] = extra_workload(
            syn.spec("20b_16384_lora"), args, lora=True)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(dt * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gpt-oss-20b MoE layer, 2048 tokens, forward (saved) + dX backward",
                   "T": T, "H": H, "I": I, "E": E, "k": k, "weights": "MXFP4 (E2M1 + UE8M0/32)",
                   "parallelism": "none (1 GPU)"},
        "fwd_tflops": round(fwd_tflops, 2), "fwd_ms": round(dt_fwd * 1e3, 4),
        "ms_per_step_stats": step_stats,
        "ms_per_step_graph": round(dt_graph * 1e3, 4),
        "ms_per_step_with_kernel_events": round(dt_inst * 1e3, 4),
        "kernel_us": kernels, "decode": decode, "roofline": roofline,
        "workloads": extra, "block_scaled_gate_up": block_scaled,
    }
    if args.act_format != "bf16":
        line["act_format"] = args.act_format

    # ---- CPU oracle on a bounded sample of the same workload
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(s, args.cpu_sample_tokens)
    print(json.dumps(line), flush=True)


def extra_workload(s, args, lora):
    """Throughput of one more full-size layer.  Expert weights ~N(0, 0.02)
    are drawn on the GPU (torch's generator, fixed seed) and quantised by the
    library; router weights, router bias (the Zipf skew), tokens and the
    upstream gradient come from the seeded generators.  Without LoRA a step
    is forward (saved) + dX; with LoRA it is the training step of a
    checkpointed layer: forward, recompute forward (saved), dX + dA/dB."""
    import numpy as np
    import torch

    import moe_synth as syn
    from mxfp4_weight_mixture_02_amd import (MoeLayer, SavedState, Workspace,
                                             mxfp4_moe_backward_dx, mxfp4_moe_forward,
                                             mxfp4_quantize)
    dev = "cuda:0"
    T, H, I, E, k = s.T, s.H, s.I, s.E, s.k
    R = T * k
    g = torch.Generator(device=dev).manual_seed(s.seed)
    gu_c = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=dev)
    gu_s = torch.empty((E, 2 * I, H // 32), dtype=torch.uint8, device=dev)
    dn_c = torch.empty((E, H, I // 2), dtype=torch.uint8, device=dev)
    dn_s = torch.empty((E, H, I // 32), dtype=torch.uint8, device=dev)
    for e in range(E):
        c, sc = mxfp4_quantize(torch.randn((2 * I, H), generator=g, device=dev) * 0.02)
        gu_c[e].copy_(c)
        gu_s[e].copy_(sc)
        c, sc = mxfp4_quantize(torch.randn((H, I), generator=g, device=dev) * 0.02)
        dn_c[e].copy_(c)
        dn_s[e].copy_(sc)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    layer = MoeLayer(torch.from_numpy(syn.router_weight(s)).to(dev),
                     torch.from_numpy(syn.router_bias(s)).to(dev), gu_c, gu_s,
                     (torch.randn((E, 2 * I), generator=g, device=dev) * 0.01).bfloat16(),
                     dn_c, dn_s, (torch.randn((E, H), generator=g, device=dev) * 0.01).bfloat16(),
                     k=k)
    if lora:
        layer.lora_A = bf(syn.lora_a(s))
        layer.lora_B = bf(syn.lora_b(s))
    x = bf(syn.tokens(s))
    dy = bf(syn.upstream_grad(s))
    sv = SavedState.empty(layer, T, dev)
    out = torch.empty_like(x)
    dx = torch.empty_like(x)
    wsf, wsb = Workspace(), Workspace()
    dA = dB = None
    if lora:
        dA = torch.empty(layer.lora_A.shape, dtype=torch.float32, device=dev)
        dB = torch.empty(layer.lora_B.shape, dtype=torch.float32, device=dev)

    def step():
        if lora:
            mxfp4_moe_forward(layer, x, out=out, workspace=wsf)
        mxfp4_moe_forward(layer, x, saved=sv, out=out, workspace=wsf)
        mxfp4_moe_backward_dx(layer, sv, dy, dx=dx, workspace=wsb, dA=dA, dB=dB)

    steps = max(3, args.steps // 4)
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    passes = 3 if lora else 2
    flops = passes * 2.0 * R * 3 * H * I
    if lora:
        flops += 6 * 2.0 * R * 16 * (H + I) / 2   # v, y delta, dv_u, da delta, dA, dB
    hist = torch.bincount(sv.topk_idx.flatten().long(), minlength=E)
    res = {"T": T, "E": E, "k": k, "ms_per_step": round(dt * 1e3, 3),
           "TFLOP/s": round(flops / dt / 1e12, 2), "steps": steps,
           "step": ("forward, recompute forward (saved), dX + dA/dB backward" if lora
                    else "forward (saved) + dX backward"),
           "max_rows_per_expert": int(hist.max()), "empty_experts": int((hist == 0).sum())}
    del layer, sv, wsf, wsb, gu_c, gu_s, dn_c, dn_s
    torch.cuda.empty_cache()
    return res


def cpu_baseline(s, n_tok):
    """The float64 oracle, as it stands, on the host cores: routing of all
    tokens, then forward and dX for a sample of n_tok tokens, each phase
    timed on its own; then the forward + dX of a quarter of the sample with
    the BLAS pool held to one thread (the per-core rate).  `value` is the
    sample's forward + dX flops over its forward + dX time (routing is
    reported apart).  The oracle's cost per token is dominated by
    dequantizing the weights of every expert the sample touches (about 0.5 s
    per expert on one core), so its rate grows with the sample."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import moe_synth as syn
    from oracle import moe, mxfp4

    xb = syn.tokens(s)
    dyb = syn.upstream_grad(s)
    toks = np.arange(n_tok)
    rl = moe.Layer(router_w=syn.router_weight(s), router_b=syn.router_bias(s),
                   gu_codes=np.zeros((s.E, 2, 1), np.uint8), gu_scales=None, gu_bias=None,
                   dn_codes=None, dn_scales=None, dn_bias=None, k=s.k)
    touched = sorted(set(int(e) for e in np.unique(moe.route(rl, xb).idx[toks])))
    gu_c = np.zeros((s.E, 2 * s.I, s.H // 2), np.uint8)
    gu_s = np.zeros((s.E, 2 * s.I, s.H // 32), np.uint8)
    dn_c = np.zeros((s.E, s.H, s.I // 2), np.uint8)
    dn_s = np.zeros((s.E, s.H, s.I // 32), np.uint8)
    from concurrent.futures import ThreadPoolExecutor

    def q(e):
        return e, mxfp4.quantize(syn.gate_up_weight(s, e)), mxfp4.quantize(syn.down_weight(s, e))

    with ThreadPoolExecutor(8) as ex:
        for e, (a, b), (c, d) in ex.map(q, touched):
            gu_c[e], gu_s[e], dn_c[e], dn_s[e] = a, b, c, d
    ol = moe.Layer(syn.router_weight(s), syn.router_bias(s), gu_c, gu_s, syn.gate_up_bias(s),
                   dn_c, dn_s, syn.down_bias(s), k=s.k)
    t0 = time.perf_counter()
    r = moe.route(ol, xb)
    t_route = time.perf_counter() - t0
    t0 = time.perf_counter()
    moe.forward(ol, xb, tokens=toks, routing=r)
    t_fwd = time.perf_counter() - t0
    t0 = time.perf_counter()
    moe.backward_dx(ol, xb, dyb, tokens=toks, routing=r)
    t_bwd = time.perf_counter() - t0
    per_tok = 2 * (2.0 * s.k * 3 * s.H * s.I)          # forward + dX flops per token
    n1 = max(1, n_tok // 4)
    with threadpool_limits(limits=1, user_api="blas"):
        t0 = time.perf_counter()
        moe.forward(ol, xb, tokens=toks[:n1], routing=r)
        moe.backward_dx(ol, xb, dyb, tokens=toks[:n1], routing=r)
        t_one = time.perf_counter() - t0
    blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"value": round(n_tok * per_tok / (t_fwd + t_bwd) / 1e12, 6), "unit": "TFLOP/s",
            "cores": cores, "blas_threads": max(blas) if blas else 1, "kind": "oracle",
            "seconds": {"route_all_tokens": round(t_route, 3), "forward": round(t_fwd, 2),
                        "backward_dx": round(t_bwd, 2)},
            "per_core": {"value": round(n1 * per_tok / t_one / 1e12, 6), "unit": "TFLOP/s",
                         "tokens": n1, "seconds": round(t_one, 2)},
            "sample": f"{n_tok} tokens ({n_tok * s.k} routed rows, {len(touched)} experts) of the "
                      f"2048-token gpt-oss-20b layer: routing of all {s.T} tokens, then forward + "
                      f"dX for the sample, float64 numpy on the host's cores (BLAS matmuls "
                      f"multi-threaded, dequant single-threaded); per_core: {n1} tokens, BLAS "
                      f"held to one thread"}


if __name__ == "__main__":
    main()
