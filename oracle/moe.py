"""The MoE expert block, the oracle's version (test infrastructure only).

Structure follows the eager reference path of [P1] "What this does": the
top-k router, then a per-expert loop in which each expert's packed MXFP4
weights are dequantized on the fly and the GPT-OSS expert math runs on them
(gate_up projection with bias, GLU, down projection with bias), then the
routing-weighted reduce ([P3] commit note on the per-expert ``bias=``
operand: ``_finish_down`` keeps only that reduce).  Everything is float64.

Layouts (row-major, last dim contiguous):
  x          bf16 bits [T, H]            activations
  router_w   fp32 [E, H], router_b fp32 [E]
  gu_codes   uint8 [E, 2I, H/2], gu_scales uint8 [E, 2I, H/32]
             rows interleaved: gate j at row 2j, up j at row 2j+1
             ([P3] commit note "store gate|up row-interleaved")
  gu_bias    bf16 bits [E, 2I] (same row order), or None
  dn_codes   uint8 [E, H, I/2], dn_scales uint8 [E, H, I/32]
  dn_bias    bf16 bits [E, H], or None
  lora_A     bf16 bits [E, r, I], lora_B bf16 bits [E, H, r], or None
             (adapter on the down projection)
  lora_gu_A  bf16 bits [E, r, H], lora_gu_B bf16 bits [E, 2I, r], or None
             (adapter on the gate_up projection, B's rows interleaved like
             the gate_up rows); both adapters share lora_scale

Flat routed rows are f = t * k + j for token t and slot j.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import mxfp4, mxfp8


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly.  A float64 array is
    taken as already decoded (finite-difference probes use this)."""
    a = np.asarray(bits)
    if a.dtype == np.float64:
        return a
    b = a.astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


@dataclass
class Layer:
    """One MoE layer's frozen parameters (numpy arrays, layouts above)."""
    router_w: np.ndarray
    router_b: np.ndarray | None
    gu_codes: np.ndarray
    gu_scales: np.ndarray
    gu_bias: np.ndarray | None
    dn_codes: np.ndarray
    dn_scales: np.ndarray
    dn_bias: np.ndarray | None
    k: int
    alpha: float = 1.702
    limit: float = 7.0
    lora_A: np.ndarray | None = None
    lora_B: np.ndarray | None = None
    lora_scale: float = 1.0
    lora_gu_A: np.ndarray | None = None
    lora_gu_B: np.ndarray | None = None
    #: float64 weights used instead of the dequantized codes ([E, 2I, H] and
    #: [E, H, I]); only for finite-difference probes of the weight gradients
    gu_weight: np.ndarray | None = None
    dn_weight: np.ndarray | None = None
    #: precision the logits are rounded to before the top-k decision;
    #: float64 only for finite-difference probes of the router path
    logit_dtype: type = np.float32

    @property
    def E(self):
        return self.gu_codes.shape[0]

    @property
    def H(self):
        return self.gu_codes.shape[2] * 2

    @property
    def I(self):
        return self.gu_codes.shape[1] // 2

    def gate_up(self, e):
        """Dequantized gate_up weight of expert e, float64 [2I, H]."""
        if self.gu_weight is not None:
            return self.gu_weight[e]
        return mxfp4.dequantize(self.gu_codes[e], self.gu_scales[e])

    def down(self, e):
        """Dequantized down weight of expert e, float64 [H, I]."""
        if self.dn_weight is not None:
            return self.dn_weight[e]
        return mxfp4.dequantize(self.dn_codes[e], self.dn_scales[e])

    def gu_b(self, e):
        return np.zeros(2 * self.I) if self.gu_bias is None else bf16_to_f64(self.gu_bias[e])

    def dn_b(self, e):
        return np.zeros(self.H) if self.dn_bias is None else bf16_to_f64(self.dn_bias[e])

    @property
    def has_lora(self):
        """An adapter on the down projection."""
        return self.lora_A is not None

    @property
    def has_lora_gu(self):
        """An adapter on the gate_up projection."""
        return self.lora_gu_A is not None


# ----------------------------------------------------------------- router

def router_logits(layer: Layer, x_bits) -> np.ndarray:
    """l[t, e] = sum_h x[t, h] * Wr[e, h] + b[e].

    The products of bf16 and fp32 values are exact in float64 and are summed
    in float64, then the logit is rounded once to float32: the routing
    decision is taken on those float32 values.  (Reading: the pages give no
    precision for the router; taking the decision on once-rounded logits
    makes it reproducible up to exact ties.)
    """
    x = bf16_to_f64(x_bits)
    l = x @ layer.router_w.astype(np.float64).T
    if layer.router_b is not None:
        l = l + layer.router_b.astype(np.float64)
    return l.astype(layer.logit_dtype)


def topk_softmax(logits: np.ndarray, k: int):
    """Top-k selection and softmax over the selected k ([P1] "What this
    does": top-k router; the softmax is over the k selected logits).

    Reading: experts are ordered by logit descending, ties to the lower
    expert index, and slot j holds the j-th in that order.
    Returns idx int32 [T, k] and weights float64 [T, k].
    """
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    order = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(logits, idx, axis=1).astype(np.float64)
    z = np.exp(sel - sel[:, :1])
    w = z / z.sum(axis=1, keepdims=True)
    return idx, w


def permutation(idx: np.ndarray, E: int):
    """Expert histogram, its exclusive prefix sum, and the token permutation.

    offsets[e] = number of routed rows with expert < e (offsets[E] = T*k);
    sorted_rows lists, expert by expert, the flat rows f = t*k + j routed to
    that expert, in ascending f (reading: a stable counting sort; the pages
    only say the grouped path sorted rows by expert).
    """
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    hist = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(hist)
    sorted_rows = np.argsort(flat, kind="stable")
    return offsets.astype(np.int32), sorted_rows.astype(np.int32)


# -------------------------------------------------------------- activation

def swiglu(g, u, alpha, limit):
    """Clamped SwiGLU of GPT-OSS: gate clamped above at limit, up clamped to
    [-limit, limit], a = g_c * sigmoid(alpha * g_c) * (u_c + 1).

    Reading: the pages call the activation the GptOssExperts GLU ([P1],
    [P3] notes on the fused GLU epilogue); alpha = 1.702 and limit = 7 come
    with the workloads; the one-sided gate clamp and the +1 on up are the
    published GPT-OSS activation.
    """
    gc = np.minimum(g, limit)
    uc = np.clip(u, -limit, limit)
    sig = 1.0 / (1.0 + np.exp(-alpha * gc))
    return gc * sig * (uc + 1.0)


def swiglu_backward(g, u, da, alpha, limit):
    """d a / d g and d a / d u times da.  A clamped input passes no gradient
    outside its range; at the bound itself it passes (like an autograd
    clamp; reading)."""
    gc = np.minimum(g, limit)
    uc = np.clip(u, -limit, limit)
    sig = 1.0 / (1.0 + np.exp(-alpha * gc))
    dgc = da * (uc + 1.0) * sig * (1.0 + alpha * gc * (1.0 - sig))
    duc = da * gc * sig
    dg = np.where(g <= limit, dgc, 0.0)
    du = np.where((u >= -limit) & (u <= limit), duc, 0.0)
    return dg, du


# ----------------------------------------------------------------- forward

@dataclass
class Routing:
    logits: np.ndarray       # float32 [T, E]
    idx: np.ndarray          # int32 [T, k]
    w: np.ndarray            # float64 [T, k]
    offsets: np.ndarray      # int32 [E + 1]
    sorted_rows: np.ndarray  # int32 [T * k]


def route(layer: Layer, x_bits) -> Routing:
    logits = router_logits(layer, x_bits)
    idx, w = topk_softmax(logits, layer.k)
    offsets, sorted_rows = permutation(idx, layer.E)
    return Routing(logits, idx, w, offsets, sorted_rows)


def _expert_rows(r: Routing, e, k, tokens_mask):
    rows = r.sorted_rows[r.offsets[e]:r.offsets[e + 1]].astype(np.int64)
    if tokens_mask is not None:
        rows = rows[tokens_mask[rows // k]]
    return rows


def _lora_v(layer, e, a):
    return a @ bf16_to_f64(layer.lora_A[e]).T            # [rows, r]


def _lora_vg(layer, e, xt):
    """The gate_up adapter's rank-space activations x A_gu^T, [rows, r]."""
    return xt @ bf16_to_f64(layer.lora_gu_A[e]).T


def _gate_up_pre(layer, e, xt, Wgu, xqt=None):
    """h = x Wgu^T + b (+ s (x A_gu^T) B_gu^T with the gate_up adapter).
    ``xqt``, when given, is the product's input under a block-scaled
    activation format (gate_up_input); the adapter still reads x."""
    h = (xt if xqt is None else xqt) @ Wgu.T + layer.gu_b(e)
    if layer.has_lora_gu:
        h = h + layer.lora_scale * _lora_vg(layer, e, xt) @ bf16_to_f64(layer.lora_gu_B[e]).T
    return h


def gate_up_input(x: np.ndarray, fmt: str) -> np.ndarray:
    """The activations the gate_up product consumes under an activation
    format ([P3] commit notes: activation_format "bf16" = weight-only, None =
    the weights' block-scaled format): "bf16" keeps x; "mxfp8" is one MXFP8
    quantization of each token row; "mxfp8x2" the hi + lo pair, x ~ deq(hi) +
    deq(lo) (oracle/mxfp8.py)."""
    if fmt == "bf16":
        return x
    if fmt == "mxfp8":
        return mxfp8.dequantize(*mxfp8.quantize(x))
    if fmt == "mxfp8x2":
        hc, hs, lc, ls = mxfp8.quantize_hi_lo(x)
        return mxfp8.dequantize(hc, hs) + mxfp8.dequantize(lc, ls)
    raise ValueError(f"unknown activation format {fmt!r}")


def forward(layer: Layer, x_bits, tokens=None, routing: Routing | None = None, experts=None,
            act_format: str = "bf16"):
    """Expert-block forward.  Returns (out float64 [T, H], routing, cache).

    out[t] = sum_j w[t, j] * y_(t, j), where for expert e = idx[t, j]
      h = x[t] @ Wgu[e].T + bgu[e]                (2I values)
          (+ s * (x[t] @ Agu_e.T) @ Bgu_e.T with the gate_up adapter)
      a = swiglu(h[0::2], h[1::2])                (stride-2 split, [P3])
      y = a @ Wd[e].T + bd[e] (+ s * (a @ A_e.T) @ B_e.T with LoRA)

    ``tokens`` (optional index array) restricts the expert loop to those
    tokens; the other rows of ``out`` stay zero.  ``experts`` (optional)
    restricts it to those experts: ``out`` then holds only their share.
    ``act_format`` quantizes the gate_up product's input (gate_up_input);
    the router, the adapters and the down product keep their inputs.
    Routing is always for all tokens (it is what the permutation is defined
    on).  ``cache`` maps each flat row f that was computed to (h, a, y, vg)
    for the backward and tests (vg = x A_gu^T, None without the gate_up
    adapter).
    """
    x = bf16_to_f64(x_bits)
    T, H = x.shape
    k = layer.k
    r = route(layer, x_bits) if routing is None else routing
    mask = None
    if tokens is not None:
        mask = np.zeros(T, dtype=bool)
        mask[np.asarray(tokens)] = True
    out = np.zeros((T, H))
    cache = {}
    xq = gate_up_input(x, act_format)
    for e in range(layer.E):
        if experts is not None and e not in experts:
            continue
        rows = _expert_rows(r, e, k, mask)
        if rows.size == 0:
            continue
        t = rows // k
        h = xq[t] @ layer.gate_up(e).T + layer.gu_b(e)
        if layer.has_lora_gu:
            h = h + layer.lora_scale * _lora_vg(layer, e, x[t]) @ bf16_to_f64(layer.lora_gu_B[e]).T
        a = swiglu(h[:, 0::2], h[:, 1::2], layer.alpha, layer.limit)
        y = a @ layer.down(e).T + layer.dn_b(e)
        if layer.has_lora:
            y = y + layer.lora_scale * _lora_v(layer, e, a) @ bf16_to_f64(layer.lora_B[e]).T
        vg = _lora_vg(layer, e, x[t]) if layer.has_lora_gu else None
        wr = r.w.reshape(-1)[rows]
        np.add.at(out, t, wr[:, None] * y)
        for i, f in enumerate(rows):
            cache[int(f)] = (h[i], a[i], y[i], None if vg is None else vg[i])
    return out, r, cache


# ---------------------------------------------------------------- backward

def backward_dx(layer: Layer, x_bits, dy_bits, tokens=None, routing: Routing | None = None,
                want_lora=True, experts=None, gu_grads: dict | None = None,
                base_grads: dict | None = None, act_format: str = "bf16"):
    """Gradient of L = sum(dY * out) with respect to x (and the LoRA
    adapters), base weights and biases frozen ([P1]: only the input and
    adapter gradients are needed for LoRA training).

    Per routed row f = (t, j) of expert e:
      dw_f  = dY[t] . y_f                      (gradient of its routing weight)
      g_y   = w_f * dY[t]
      da    = g_y @ Wd[e]   (+ LoRA: dv = s * g_y @ B_e; da += dv @ A_e)
      dg, du = swiglu_backward(h[0::2], h[1::2], da)
      dh    = interleave(dg, du)
      dx_f  = dh @ Wgu[e]   (+ gate_up adapter: dvg = s * dh @ Bgu_e; dx_f += dvg @ Agu_e)
    Router (softmax over the selected logits, reading: dX includes it):
      dl_j  = w_j * (dw_j - sum_i w_i dw_i)
      dX[t] = sum_j dx_(t, j) + sum_j dl_j * Wr[idx[t, j]]
    LoRA: dB_e = s * sum_f g_y^T v_f, dA_e = sum_f dv^T a_f.
    Gate_up adapter (filled into ``gu_grads`` as "dA_gu" [E, r, H] and
    "dB_gu" [E, 2I, r] when a dict is given): dB_gu_e = s * sum_f dh^T vg_f
    with vg = x A_gu^T, dA_gu_e = sum_f dvg^T x_t.
    Base weights and biases, as if they were trained (filled into
    ``base_grads`` when a dict is given; [P1] "Relation to the backward
    triton kernels": native MXFP4 training needs them): the gradients with
    respect to the dequantized weights,
      dW_gu_e = sum_f dh_f^T x_t [E, 2I, H],   db_gu_e = sum_f dh_f [E, 2I],
      dW_dn_e = sum_f g_y^T a_f  [E, H, I],    db_dn_e = sum_f g_y  [E, H].

    ``act_format`` names the forward's gate_up input format
    (gate_up_input).  The backward keeps the h that forward computed from
    the quantized input and treats the quantizer as the identity
    (straight-through): every product above that needs the gate_up input
    (dW_gu, the adapters) reads x, and dX is the exact gradient of the
    forward with the quantization error x_q - x held constant.

    ``tokens`` restricts dX to those tokens (then dA/dB cover only them).
    ``experts`` restricts the expert loop to those experts: dA/dB are then
    exact for them (zero elsewhere) and dX holds only their share, so the
    router term, which needs every slot of a token, is left out.
    Returns (dX float64 [T, H], dA [E, r, I] or None, dB [E, H, r] or None).
    """
    x = bf16_to_f64(x_bits)
    dY = bf16_to_f64(dy_bits)
    T, H = x.shape
    k = layer.k
    r = route(layer, x_bits) if routing is None else routing
    mask = None
    if tokens is not None:
        mask = np.zeros(T, dtype=bool)
        mask[np.asarray(tokens)] = True
    dX = np.zeros((T, H))
    dw = np.zeros(T * k)
    lora = layer.has_lora and want_lora
    dA = np.zeros(layer.lora_A.shape) if lora else None
    dB = np.zeros(layer.lora_B.shape) if lora else None
    lora_gu = layer.has_lora_gu and want_lora and gu_grads is not None
    dAg = np.zeros(layer.lora_gu_A.shape) if lora_gu else None
    dBg = np.zeros(layer.lora_gu_B.shape) if lora_gu else None
    xq = gate_up_input(x, act_format)
    base = base_grads is not None
    if base:
        E, I = layer.E, layer.I
        dWg, dbg = np.zeros((E, 2 * I, H)), np.zeros((E, 2 * I))
        dWd, dbd = np.zeros((E, H, I)), np.zeros((E, H))
    wflat = r.w.reshape(-1)
    for e in range(layer.E):
        if experts is not None and e not in experts:
            continue
        rows = _expert_rows(r, e, k, mask)
        if rows.size == 0:
            continue
        t = rows // k
        Wgu = layer.gate_up(e)
        Wd = layer.down(e)
        h = _gate_up_pre(layer, e, x[t], Wgu, xq[t])
        g, u = h[:, 0::2], h[:, 1::2]
        a = swiglu(g, u, layer.alpha, layer.limit)
        y = a @ Wd.T + layer.dn_b(e)
        if layer.has_lora:
            A = bf16_to_f64(layer.lora_A[e])
            B = bf16_to_f64(layer.lora_B[e])
            v = a @ A.T
            y = y + layer.lora_scale * v @ B.T
        dw[rows] = np.einsum("rh,rh->r", dY[t], y)
        gy = wflat[rows][:, None] * dY[t]
        da = gy @ Wd
        if base:
            dWd[e] += gy.T @ a
            dbd[e] += gy.sum(axis=0)
        if layer.has_lora:
            dv = layer.lora_scale * gy @ B
            da = da + dv @ A
            if lora:
                dB[e] += layer.lora_scale * gy.T @ v
                dA[e] += dv.T @ a
        dg, du = swiglu_backward(g, u, da, layer.alpha, layer.limit)
        dh = np.empty_like(h)
        dh[:, 0::2] = dg
        dh[:, 1::2] = du
        dxf = dh @ Wgu
        if base:
            dWg[e] += dh.T @ x[t]
            dbg[e] += dh.sum(axis=0)
        if layer.has_lora_gu:
            Ag = bf16_to_f64(layer.lora_gu_A[e])
            Bg = bf16_to_f64(layer.lora_gu_B[e])
            dvg = layer.lora_scale * dh @ Bg
            dxf = dxf + dvg @ Ag
            if lora_gu:
                dBg[e] += layer.lora_scale * dh.T @ (x[t] @ Ag.T)
                dAg[e] += dvg.T @ x[t]
        np.add.at(dX, t, dxf)
    if lora_gu:
        gu_grads["dA_gu"], gu_grads["dB_gu"] = dAg, dBg
    if base:
        base_grads.update(dW_gu=dWg, db_gu=dbg, dW_dn=dWd, db_dn=dbd)
    if experts is not None:
        return dX, dA, dB
    # router path through the softmax over the selected logits
    Wr = layer.router_w.astype(np.float64)
    dwt = dw.reshape(T, k)
    dl = r.w * (dwt - (r.w * dwt).sum(axis=1, keepdims=True))
    toks = np.arange(T) if mask is None else np.nonzero(mask)[0]
    for tt in toks:
        dX[tt] += dl[tt] @ Wr[r.idx[tt]]
    return dX, dA, dB
