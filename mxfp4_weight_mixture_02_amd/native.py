"""ctypes binding of libmxfp4_moe.so (include/mxfp4_moe.h).

Argument marshalling only: every step of the expert block runs in the HIP
library.  torch provides device memory and the current stream.  There is
no CPU fallback: if the library is missing or no GPU is present, the calls
raise.
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmxfp4_moe.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "mxfp4_moe.h")

MXFP4_OK = 0
WS_FORWARD, WS_FORWARD_SAVED, WS_BACKWARD, WS_BACKWARD_FULL = 0, 1, 2, 3
ERRORS = {-1: "EINVAL", -2: "EUNSUPPORTED", -3: "EWORKSPACE", -4: "EHIP"}


class Mxfp4Error(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed: {ERRORS.get(code, code)}: {msg}")
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64), ("I", ctypes.c_int64),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("swiglu_alpha", ctypes.c_float), ("swiglu_limit", ctypes.c_float),
                ("lora_rank", ctypes.c_int32), ("lora_scale", ctypes.c_float),
                ("lora_targets", ctypes.c_int32), ("activation_format", ctypes.c_int32)]

LORA_DOWN, LORA_GATE_UP = 1, 2
ACT_FORMATS = {"bf16": 0, "mxfp8": 1, "mxfp8x2": 2}


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("router_w", "router_b", "gu_codes", "gu_scales", "gu_bias",
                 "dn_codes", "dn_scales", "dn_bias", "lora_A", "lora_B", "lora_gu_A", "lora_gu_B")]


class Saved(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_idx", "topk_w", "expert_offsets", "sorted_rows", "h", "a", "lora_v", "lora_vg")]


class SavedSizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n, _ in Saved._fields_]


class Grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("dx", "dA", "dB", "dA_gu", "dB_gu", "dW_gu", "dW_dn", "db_gu", "db_dn")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mxfp4_weight_mixture_02_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.mxfp4_last_error.restype = ctypes.c_char_p
        L.mxfp4_last_error.argtypes = []
        L.mxfp4_moe_workspace_bytes.restype = ctypes.c_size_t
        L.mxfp4_moe_workspace_bytes.argtypes = [ctypes.POINTER(Dims), i32]
        L.mxfp4_moe_saved_bytes.restype = i32
        L.mxfp4_moe_saved_bytes.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(SavedSizes)]
        L.mxfp4_moe_forward.restype = i32
        L.mxfp4_moe_forward.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Weights), vp, vp,
                                        ctypes.POINTER(Saved), vp, ctypes.c_size_t, vp]
        L.mxfp4_moe_forward_noalloc.restype = i32
        L.mxfp4_moe_forward_noalloc.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Weights), vp,
                                                vp, ctypes.POINTER(Saved), vp]
        L.mxfp4_moe_backward_dx.restype = i32
        L.mxfp4_moe_backward_dx.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Weights),
                                            ctypes.POINTER(Saved), vp, vp, vp, vp, vp, vp, vp,
                                            vp, ctypes.c_size_t, vp]
        L.mxfp4_moe_backward.restype = i32
        L.mxfp4_moe_backward.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Weights),
                                         ctypes.POINTER(Saved), vp, vp, ctypes.POINTER(Grads), vp,
                                         ctypes.c_size_t, vp]
        L.mxfp8_quantize.restype = i32
        L.mxfp8_quantize.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp]
        L.mxfp4_quantize.restype = i32
        L.mxfp4_quantize.argtypes = [vp, i64, i64, vp, vp, vp]
        L.mxfp4_dequantize.restype = i32
        L.mxfp4_dequantize.argtypes = [vp, vp, i64, i64, i32, vp, vp]
        _lib = L
    return _lib


def header_symbols() -> list[str]:
    """Function names declared in include/mxfp4_moe.h."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(mxfp[48]_\w+)\s*\(", txt, re.M)))


def _check(fn, rc):
    if rc != MXFP4_OK:
        raise Mxfp4Error(fn, rc, lib().mxfp4_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, dtype, name):
    if t is None:
        return None
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor")
    return t


def _shape(t, shape, dtype, name, optional=False):
    """Refuse a tensor whose shape or dtype differs from what the C ABI will
    assume (it sees only pointers, so a mismatch would read or write out of
    bounds).  Runs before the device checks and on any device."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


# --------------------------------------------------------------- quantise

def mxfp4_quantize(w: torch.Tensor):
    """fp32 [..., K] -> (codes uint8 [..., K/2], scales uint8 [..., K/32])."""
    w = _dev(w, torch.float32, "w")
    K = w.shape[-1]
    rows = w.numel() // K
    codes = torch.empty(w.shape[:-1] + (K // 2,), dtype=torch.uint8, device=w.device)
    scales = torch.empty(w.shape[:-1] + (K // 32,), dtype=torch.uint8, device=w.device)
    _check("mxfp4_quantize", lib().mxfp4_quantize(_ptr(w), rows, K, _ptr(codes), _ptr(scales),
                                                  _stream()))
    return codes, scales


def mxfp4_dequantize(codes: torch.Tensor, scales: torch.Tensor, dtype=torch.float32):
    codes = _dev(codes, torch.uint8, "codes")
    scales = _dev(scales, torch.uint8, "scales")
    K = codes.shape[-1] * 2
    rows = codes.numel() // codes.shape[-1]
    out = torch.empty(codes.shape[:-1] + (K,), dtype=dtype, device=codes.device)
    code = {torch.float32: 0, torch.bfloat16: 1}[dtype]
    _check("mxfp4_dequantize", lib().mxfp4_dequantize(_ptr(codes), _ptr(scales), rows, K, code,
                                                      _ptr(out), _stream()))
    return out


# ------------------------------------------------------------- the block

@dataclass
class MoeLayer:
    """Device tensors of one layer (layouts as in include/mxfp4_moe.h)."""
    router_w: torch.Tensor            # fp32 [E, H]
    router_b: torch.Tensor | None     # fp32 [E]
    gu_codes: torch.Tensor            # uint8 [E, 2I, H/2]
    gu_scales: torch.Tensor           # uint8 [E, 2I, H/32]
    gu_bias: torch.Tensor | None      # bf16 [E, 2I]
    dn_codes: torch.Tensor            # uint8 [E, H, I/2]
    dn_scales: torch.Tensor           # uint8 [E, H, I/32]
    dn_bias: torch.Tensor | None      # bf16 [E, H]
    k: int
    alpha: float = 1.702
    limit: float = 7.0
    lora_A: torch.Tensor | None = None       # bf16 [E, r, I]   adapter on down
    lora_B: torch.Tensor | None = None       # bf16 [E, H, r]
    lora_scale: float = 1.0
    lora_gu_A: torch.Tensor | None = None    # bf16 [E, r, H]   adapter on gate_up
    lora_gu_B: torch.Tensor | None = None    # bf16 [E, 2I, r]
    act_format: str = "bf16"                 # gate_up input: bf16 | mxfp8 | mxfp8x2

    @property
    def E(self):
        return self.gu_codes.shape[0]

    @property
    def H(self):
        return self.gu_codes.shape[2] * 2

    @property
    def I(self):
        return self.gu_codes.shape[1] // 2

    @property
    def lora_rank(self):
        if self.lora_A is not None:
            return self.lora_A.shape[1]
        return 0 if self.lora_gu_A is None else self.lora_gu_A.shape[1]

    @property
    def lora_targets(self):
        return (LORA_DOWN if self.lora_A is not None else 0) | \
               (LORA_GATE_UP if self.lora_gu_A is not None else 0)

    def dims(self, T):
        if self.act_format not in ACT_FORMATS:
            raise ValueError(f"act_format must be one of {sorted(ACT_FORMATS)}")
        return Dims(T, self.H, self.I, self.E, self.k, self.alpha, self.limit, self.lora_rank,
                    self.lora_scale, self.lora_targets, ACT_FORMATS[self.act_format])

    def check_shapes(self):
        """Every parameter's shape and dtype against E, H, I (and the rank)."""
        if self.gu_codes.dim() != 3 or min(self.gu_codes.shape) < 1:
            raise ValueError(f"gu_codes must be [E, 2I, H/2], got {tuple(self.gu_codes.shape)}")
        E, H, I = self.E, self.H, self.I
        u8, bf = torch.uint8, torch.bfloat16
        _shape(self.router_w, (E, H), torch.float32, "router_w")
        _shape(self.router_b, (E,), torch.float32, "router_b", optional=True)
        _shape(self.gu_codes, (E, 2 * I, H // 2), u8, "gu_codes")
        _shape(self.gu_scales, (E, 2 * I, H // 32), u8, "gu_scales")
        _shape(self.gu_bias, (E, 2 * I), bf, "gu_bias", optional=True)
        _shape(self.dn_codes, (E, H, I // 2), u8, "dn_codes")
        _shape(self.dn_scales, (E, H, I // 32), u8, "dn_scales")
        _shape(self.dn_bias, (E, H), bf, "dn_bias", optional=True)
        if (self.lora_A is None) != (self.lora_B is None):
            raise ValueError("lora_A and lora_B go together")
        if self.lora_A is not None:
            if self.lora_A.dim() != 3:
                raise ValueError(f"lora_A must be [E, r, I], got {tuple(self.lora_A.shape)}")
            r = self.lora_A.shape[1]
            _shape(self.lora_A, (E, r, I), bf, "lora_A")
            _shape(self.lora_B, (E, H, r), bf, "lora_B")
        if (self.lora_gu_A is None) != (self.lora_gu_B is None):
            raise ValueError("lora_gu_A and lora_gu_B go together")
        if self.lora_gu_A is not None:
            if self.lora_gu_A.dim() != 3:
                raise ValueError(f"lora_gu_A must be [E, r, H], got {tuple(self.lora_gu_A.shape)}")
            r = self.lora_rank   # one rank for both adapters
            _shape(self.lora_gu_A, (E, r, H), bf, "lora_gu_A")
            _shape(self.lora_gu_B, (E, 2 * I, r), bf, "lora_gu_B")

    def weights(self):
        self.check_shapes()
        _dev(self.router_w, torch.float32, "router_w")
        _dev(self.router_b, torch.float32, "router_b")
        for n in ("gu_codes", "gu_scales", "dn_codes", "dn_scales"):
            _dev(getattr(self, n), torch.uint8, n)
        for n in ("gu_bias", "dn_bias", "lora_A", "lora_B", "lora_gu_A", "lora_gu_B"):
            _dev(getattr(self, n), torch.bfloat16, n)
        return Weights(*[_ptr(getattr(self, n)) for n, _ in Weights._fields_])


@dataclass
class SavedState:
    topk_idx: torch.Tensor       # int32 [T, k]
    topk_w: torch.Tensor         # fp32 [T, k]
    expert_offsets: torch.Tensor  # int32 [E + 1]
    sorted_rows: torch.Tensor    # int32 [T*k]
    h: torch.Tensor              # bf16 [T*k, 2I]
    a: torch.Tensor              # bf16 [T*k, I]
    lora_v: torch.Tensor | None = None    # fp32 [T*k, r] with the down adapter
    lora_vg: torch.Tensor | None = None   # fp32 [T*k, r] with the gate_up adapter

    @staticmethod
    def empty(layer: MoeLayer, T: int, device):
        """Caller-owned buffers of the sizes mxfp4_moe_saved_bytes gives."""
        R = T * layer.k
        r = layer.lora_rank
        nbytes = saved_bytes(layer, T)
        shapes = {"topk_idx": ((T, layer.k), torch.int32), "topk_w": ((T, layer.k), torch.float32),
                  "expert_offsets": ((layer.E + 1,), torch.int32), "sorted_rows": ((R,), torch.int32),
                  "h": ((R, 2 * layer.I), torch.bfloat16), "a": ((R, layer.I), torch.bfloat16),
                  "lora_v": ((R, r), torch.float32), "lora_vg": ((R, r), torch.float32)}
        bufs = {}
        for n, (shape, dt) in shapes.items():
            if nbytes[n] == 0:
                bufs[n] = None
                continue
            t = torch.empty(shape, dtype=dt, device=device)
            if t.numel() * t.element_size() != nbytes[n]:
                raise Mxfp4Error("mxfp4_moe_saved_bytes", -1, f"{n}: {nbytes[n]} bytes, shape {shape}")
            bufs[n] = t
        return SavedState(**bufs)

    def check_shapes(self, layer: MoeLayer, T: int):
        """Every buffer against the sizes a call with T tokens uses."""
        R = T * layer.k
        r = layer.lora_rank
        _shape(self.topk_idx, (T, layer.k), torch.int32, "saved.topk_idx")
        _shape(self.topk_w, (T, layer.k), torch.float32, "saved.topk_w")
        _shape(self.expert_offsets, (layer.E + 1,), torch.int32, "saved.expert_offsets")
        _shape(self.sorted_rows, (R,), torch.int32, "saved.sorted_rows")
        _shape(self.h, (R, 2 * layer.I), torch.bfloat16, "saved.h")
        _shape(self.a, (R, layer.I), torch.bfloat16, "saved.a")
        _shape(self.lora_v, (R, r), torch.float32, "saved.lora_v", optional=(layer.lora_A is None))
        _shape(self.lora_vg, (R, r), torch.float32, "saved.lora_vg",
               optional=(layer.lora_gu_A is None))

    def struct(self):
        for n, _ in Saved._fields_:
            t = getattr(self, n)
            _dev(t, t.dtype if t is not None else None, f"saved.{n}")
        return Saved(*[_ptr(getattr(self, n)) for n, _ in Saved._fields_])


class Workspace:
    """Grow-only device workspace, reused across calls on one stream."""

    def __init__(self):
        self.buf = None

    def get(self, nbytes, device):
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        return self.buf


_WS = Workspace()


def saved_bytes(layer: MoeLayer, T: int) -> dict:
    """Byte size of each saved-state buffer (mxfp4_moe_saved_bytes)."""
    d = layer.dims(T)
    z = SavedSizes()
    _check("mxfp4_moe_saved_bytes", lib().mxfp4_moe_saved_bytes(ctypes.byref(d), ctypes.byref(z)))
    return {n: getattr(z, n) for n, _ in SavedSizes._fields_}


def workspace_bytes(layer: MoeLayer, T: int, mode: int) -> int:
    d = layer.dims(T)
    n = lib().mxfp4_moe_workspace_bytes(ctypes.byref(d), mode)
    if n == 0:
        raise Mxfp4Error("mxfp4_moe_workspace_bytes", -1, lib().mxfp4_last_error().decode())
    return n


def mxfp4_moe_forward(layer: MoeLayer, x: torch.Tensor, saved: SavedState | bool | None = None,
                      out: torch.Tensor | None = None, workspace: Workspace | None = None):
    """Expert-block forward.  ``saved=True`` allocates and fills the state
    the backward needs.  Returns (out, saved)."""
    layer.check_shapes()
    if x.dim() != 2:
        raise ValueError(f"x must be [T, H], got {tuple(x.shape)}")
    T = x.shape[0]
    _shape(x, (T, layer.H), torch.bfloat16, "x")
    if out is not None:
        _shape(out, (T, layer.H), torch.bfloat16, "out")
    if saved is not None and saved is not True and saved is not False:
        saved.check_shapes(layer, T)
    x = _dev(x, torch.bfloat16, "x")
    if saved is True:
        saved = SavedState.empty(layer, T, x.device)
    if out is None:
        out = torch.empty_like(x)
    _dev(out, torch.bfloat16, "out")
    mode = WS_FORWARD_SAVED if saved else WS_FORWARD
    nbytes = workspace_bytes(layer, T, mode)
    ws = (workspace or _WS).get(nbytes, x.device)
    d = layer.dims(T)
    w = layer.weights()
    sv = saved.struct() if saved else None
    rc = lib().mxfp4_moe_forward(ctypes.byref(d), ctypes.byref(w), _ptr(x), _ptr(out),
                                 ctypes.byref(sv) if sv is not None else None,
                                 _ptr(ws), ws.numel(), _stream())
    _check("mxfp4_moe_forward", rc)
    return out, saved


def mxfp4_moe_forward_noalloc(layer: MoeLayer, x: torch.Tensor, out: torch.Tensor,
                              saved: SavedState | None = None):
    """The forward through mxfp4_moe_forward_noalloc: the library's static
    scratch instead of a workspace, so nothing is allocated (the caller
    passes ``out`` and, for a saved forward, the saved-state buffers).
    Returns out."""
    layer.check_shapes()
    if x.dim() != 2:
        raise ValueError(f"x must be [T, H], got {tuple(x.shape)}")
    T = x.shape[0]
    _shape(x, (T, layer.H), torch.bfloat16, "x")
    _shape(out, (T, layer.H), torch.bfloat16, "out")
    if saved is not None:
        saved.check_shapes(layer, T)
    _dev(x, torch.bfloat16, "x")
    _dev(out, torch.bfloat16, "out")
    d = layer.dims(T)
    w = layer.weights()
    sv = saved.struct() if saved is not None else None
    rc = lib().mxfp4_moe_forward_noalloc(ctypes.byref(d), ctypes.byref(w), _ptr(x), _ptr(out),
                                         ctypes.byref(sv) if sv is not None else None, _stream())
    _check("mxfp4_moe_forward_noalloc", rc)
    return out


def mxfp4_moe_backward_dx(layer: MoeLayer, saved: SavedState, dy: torch.Tensor,
                          dx: torch.Tensor | None = None, workspace: Workspace | None = None,
                          dA: torch.Tensor | None = None, dB: torch.Tensor | None = None,
                          x: torch.Tensor | None = None, dA_gu: torch.Tensor | None = None,
                          dB_gu: torch.Tensor | None = None):
    """dX (and the adapter gradients, overwritten) for the loss sum(dy * out).
    ``x`` (the forward's input) is needed only with the gate_up adapter.
    Returns (dx, dA, dB), plus (dA_gu, dB_gu) when the layer has a gate_up
    adapter."""
    layer.check_shapes()
    if dy.dim() != 2:
        raise ValueError(f"dy must be [T, H], got {tuple(dy.shape)}")
    T = dy.shape[0]
    _shape(dy, (T, layer.H), torch.bfloat16, "dy")
    if dx is not None:
        _shape(dx, (T, layer.H), torch.bfloat16, "dx")
    saved.check_shapes(layer, T)
    grads = {}
    for name, base, on in (("dA", layer.lora_A, True), ("dB", layer.lora_B, True),
                           ("dA_gu", layer.lora_gu_A, True), ("dB_gu", layer.lora_gu_B, True)):
        g = {"dA": dA, "dB": dB, "dA_gu": dA_gu, "dB_gu": dB_gu}[name]
        if base is None:
            grads[name] = None
            continue
        if g is not None:
            _shape(g, tuple(base.shape), torch.float32, name)
        grads[name] = g
    gu = layer.lora_gu_A is not None
    if gu:
        if x is None:
            raise ValueError("x (the forward's input) is required with the gate_up adapter")
        _shape(x, (T, layer.H), torch.bfloat16, "x")
    dy = _dev(dy, torch.bfloat16, "dy")
    if dx is None:
        dx = torch.empty_like(dy)
    _dev(dx, torch.bfloat16, "dx")
    if gu:
        _dev(x, torch.bfloat16, "x")
    for name, base in (("dA", layer.lora_A), ("dB", layer.lora_B), ("dA_gu", layer.lora_gu_A),
                       ("dB_gu", layer.lora_gu_B)):
        if base is None:
            continue
        if grads[name] is None:
            grads[name] = torch.empty(base.shape, dtype=torch.float32, device=dy.device)
        _dev(grads[name], torch.float32, name)
    nbytes = workspace_bytes(layer, T, WS_BACKWARD)
    ws = (workspace or _WS).get(nbytes, dy.device)
    d = layer.dims(T)
    w = layer.weights()
    sv = saved.struct()
    rc = lib().mxfp4_moe_backward_dx(ctypes.byref(d), ctypes.byref(w), ctypes.byref(sv),
                                     _ptr(x if gu else None), _ptr(dy), _ptr(dx),
                                     _ptr(grads["dA"]), _ptr(grads["dB"]), _ptr(grads["dA_gu"]),
                                     _ptr(grads["dB_gu"]), _ptr(ws), ws.numel(), _stream())
    _check("mxfp4_moe_backward_dx", rc)
    if gu:
        return dx, grads["dA"], grads["dB"], grads["dA_gu"], grads["dB_gu"]
    return dx, grads["dA"], grads["dB"]


def mxfp4_moe_backward(layer: MoeLayer, saved: SavedState, x: torch.Tensor, dy: torch.Tensor,
                       base: bool = True, workspace: Workspace | None = None) -> dict:
    """The full backward (mxfp4_moe_backward): dx, the adapter gradients the
    layer has, and with ``base`` the base-weight and bias gradients dW_gu
    [E, 2I, H], dW_dn [E, H, I], db_gu [E, 2I], db_dn [E, H] (fp32, with
    respect to the dequantized weights).  Returns them by name."""
    layer.check_shapes()
    if dy.dim() != 2:
        raise ValueError(f"dy must be [T, H], got {tuple(dy.shape)}")
    T = dy.shape[0]
    _shape(dy, (T, layer.H), torch.bfloat16, "dy")
    _shape(x, (T, layer.H), torch.bfloat16, "x")
    saved.check_shapes(layer, T)
    _dev(dy, torch.bfloat16, "dy")
    _dev(x, torch.bfloat16, "x")
    E, H, I = layer.E, layer.H, layer.I
    f32 = dict(dtype=torch.float32, device=dy.device)
    out = {"dx": torch.empty_like(dy)}
    for name, t in (("dA", layer.lora_A), ("dB", layer.lora_B), ("dA_gu", layer.lora_gu_A),
                    ("dB_gu", layer.lora_gu_B)):
        out[name] = torch.empty(t.shape, **f32) if t is not None else None
    if base:
        out.update(dW_gu=torch.empty((E, 2 * I, H), **f32), dW_dn=torch.empty((E, H, I), **f32),
                   db_gu=torch.empty((E, 2 * I), **f32), db_dn=torch.empty((E, H), **f32))
    g = Grads(*[_ptr(out.get(n)) for n, _ in Grads._fields_])
    nbytes = workspace_bytes(layer, T, WS_BACKWARD_FULL)
    ws = (workspace or _WS).get(nbytes, dy.device)
    d = layer.dims(T)
    w = layer.weights()
    sv = saved.struct()
    rc = lib().mxfp4_moe_backward(ctypes.byref(d), ctypes.byref(w), ctypes.byref(sv), _ptr(x),
                                  _ptr(dy), ctypes.byref(g), _ptr(ws), ws.numel(), _stream())
    _check("mxfp4_moe_backward", rc)
    return {k: v for k, v in out.items() if v is not None}


def mxfp8_quantize(x: torch.Tensor, lo: bool = False):
    """Row-wise MXFP8 of bf16 x [rows, K]: (codes uint8 [rows, K], scales
    uint8 [rows, K/32]) and with ``lo`` also the residual's pair."""
    if x.dim() != 2 or x.dtype != torch.bfloat16:
        raise ValueError("x must be a 2-D bf16 tensor")
    x = _dev(x.contiguous(), torch.bfloat16, "x")
    rows, K = x.shape
    u8 = dict(dtype=torch.uint8, device=x.device)
    c, s = torch.empty((rows, K), **u8), torch.empty((rows, K // 32), **u8)
    lc = torch.empty((rows, K), **u8) if lo else None
    ls = torch.empty((rows, K // 32), **u8) if lo else None
    _check("mxfp8_quantize", lib().mxfp8_quantize(_ptr(x), rows, K, _ptr(c), _ptr(s), _ptr(lc),
                                                  _ptr(ls), _stream()))
    return (c, s, lc, ls) if lo else (c, s)
