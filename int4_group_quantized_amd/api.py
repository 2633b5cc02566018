"""Python entry points of libqmoe (argument marshalling only).

Every function takes torch tensors that already live on a ROCm device, checks dtype /
shape / contiguity, passes raw device pointers to the C ABI of include/qmoe.h and enqueues
on the current stream of the tensor's device.  All arithmetic happens in the HIP kernels;
there is no CPU path.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from ._lib import LoraC, MoELayerC, PrerouterC, QWeightC, check, lib


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


# ------------------------------------------------------------------------------ data types

@dataclass
class QWeight:
    """Group-affine quantized matrix (or expert stack) on the device.

    packed int32 [n_experts*rows, cols*bits/32] (uint32 words), scales / biases fp16 (or
    bf16 bit patterns in int16 tensors when param_dtype is PARAM_BF16) [n_experts*rows,
    cols/group]."""

    packed: torch.Tensor
    scales: torch.Tensor
    biases: torch.Tensor
    bits: int
    rows: int
    cols: int
    n_experts: int = 1
    group: int = 64
    param_dtype: int = 0

    def check(self) -> None:
        """The tensors must hold exactly the shapes the fields describe (the C layer cannot
        see buffer sizes)."""
        if self.bits not in (4, 8) or self.group not in (32, 64) or self.cols % self.group:
            raise ValueError(f"unsupported format: bits {self.bits}, group {self.group}, cols {self.cols}")
        if self.rows <= 0 or self.n_experts <= 0:
            raise ValueError("rows and n_experts must be positive")
        pdt = torch.int16 if self.param_dtype == PARAM_BF16 else torch.float16
        R = self.n_experts * self.rows
        for name, t, dt, cols in (("packed", self.packed, torch.int32, self.cols * self.bits // 32),
                                  ("scales", self.scales, pdt, self.cols // self.group),
                                  ("biases", self.biases, pdt, self.cols // self.group)):
            _dev(t, dt, name)
            if tuple(t.shape) != (R, cols):
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(R, cols)}")

    def c(self) -> QWeightC:
        self.check()
        return QWeightC(self.packed.data_ptr(), self.scales.data_ptr(), self.biases.data_ptr(),
                        self.rows, self.cols, self.bits, self.group, self.n_experts,
                        self.param_dtype)

    @classmethod
    def from_arrays(cls, packed: np.ndarray, scales: np.ndarray, biases: np.ndarray, bits: int,
                    device="cuda", group: int = 64, param_dtype: int = 0) -> "QWeight":
        """From host arrays (uint32 words; fp16 scales and biases, or their bf16 bit patterns
        as uint16 with param_dtype PARAM_BF16), optionally stacked along a leading expert
        axis.  The words and parameters are used as given (no requantization)."""
        n_experts = packed.shape[0] if packed.ndim == 3 else 1
        rows, cols = scales.shape[-2], scales.shape[-1] * group
        p = torch.from_numpy(np.ascontiguousarray(packed).view(np.int32).reshape(n_experts * rows, -1))
        s = torch.from_numpy(np.ascontiguousarray(scales).view(np.int16 if param_dtype else np.float16)
                             .reshape(n_experts * rows, -1))
        b = torch.from_numpy(np.ascontiguousarray(biases).view(np.int16 if param_dtype else np.float16)
                             .reshape(n_experts * rows, -1))
        return cls(p.to(device), s.to(device), b.to(device), bits, rows, cols, n_experts, group,
                   param_dtype)

    def expert(self, e: int) -> "QWeight":
        r = self.rows
        return QWeight(self.packed[e * r:(e + 1) * r], self.scales[e * r:(e + 1) * r],
                       self.biases[e * r:(e + 1) * r], self.bits, self.rows, self.cols, 1,
                       self.group, self.param_dtype)


@dataclass
class Lora:
    """LoRA adapter set(s): A fp16 [n_adapters, rank, in_dim], B fp16 [n_adapters, out_dim,
    rank], scale = alpha / rank."""

    A: torch.Tensor
    B: torch.Tensor
    scale: float

    def c(self) -> LoraC:
        _dev(self.A, torch.float16, "lora A")
        _dev(self.B, torch.float16, "lora B")
        n, r, i = self.A.shape
        if self.B.dim() != 3 or self.B.shape[0] != n or self.B.shape[2] != r:
            raise ValueError(f"lora B has shape {tuple(self.B.shape)}, expected ({n}, out_dim, {r})")
        return LoraC(self.A.data_ptr(), self.B.data_ptr(), r, n, i, self.B.shape[1],
                     float(self.scale))


@dataclass
class MoELayer:
    hidden: int
    inter: int
    shared_inter: int
    n_experts: int
    top_k: int
    router: QWeight
    shared_gate: QWeight
    exp_gate: QWeight
    exp_up: QWeight
    exp_down: QWeight
    sh_gate: QWeight
    sh_up: QWeight
    sh_down: QWeight
    lora_gate: Optional[Lora] = None
    lora_up: Optional[Lora] = None
    lora_down: Optional[Lora] = None
    router_bias: Optional[torch.Tensor] = None
    add_residual: bool = False

    def c(self) -> MoELayerC:
        """The C struct of the layer.  The LoRA structs it points to are owned by the
        returned struct (ctypes keeps a pointer field's target alive with the struct)."""
        loras = []
        for l in (self.lora_gate, self.lora_up, self.lora_down):
            loras.append(ctypes.POINTER(LoraC)() if l is None else ctypes.pointer(l.c()))
        if self.router_bias is not None:
            _dev(self.router_bias, torch.float32, "router_bias")
            if self.router_bias.numel() != self.n_experts:
                raise ValueError(f"router_bias must hold {self.n_experts} values")
        return MoELayerC(self.hidden, self.inter, self.shared_inter, self.n_experts, self.top_k,
                         int(self.add_residual), self.router.c(), self.shared_gate.c(),
                         self.exp_gate.c(), self.exp_up.c(), self.exp_down.c(), self.sh_gate.c(),
                         self.sh_up.c(), self.sh_down.c(), loras[0], loras[1], loras[2],
                         _ptr(self.router_bias))


@dataclass
class SuperGroupWeight:
    p4: torch.Tensor       # int32 [rows/period, cols/8]
    p2: torch.Tensor       # int32 [rows - rows/period, cols/16]
    scales: torch.Tensor   # fp16 [rows]
    period: int
    rows: int
    cols: int


# ------------------------------------------------------------------------------ entry points

def quantize_affine(w: torch.Tensor, bits: int = 4, group: int = 64) -> QWeight:
    _dev(w, torch.float32, "w")
    rows, cols = w.shape
    packed = torch.empty((rows, cols * bits // 32), dtype=torch.int32, device=w.device)
    scales = torch.empty((rows, cols // group), dtype=torch.float16, device=w.device)
    biases = torch.empty_like(scales)
    check(lib.qmoe_quantize_affine(w.data_ptr(), rows, cols, bits, group, packed.data_ptr(),
                                   scales.data_ptr(), biases.data_ptr(), _stream(w)),
          "qmoe_quantize_affine")
    return QWeight(packed, scales, biases, bits, rows, cols, 1, group)


def unpack(qw: QWeight) -> torch.Tensor:
    rows = qw.rows * qw.n_experts
    q = torch.empty((rows, qw.cols), dtype=torch.uint8, device=qw.packed.device)
    check(lib.qmoe_unpack(qw.packed.data_ptr(), rows, qw.cols, qw.bits, q.data_ptr(),
                          _stream(q)), "qmoe_unpack")
    return q


def dequantize(qw: QWeight) -> torch.Tensor:
    out = torch.empty((qw.rows * qw.n_experts, qw.cols), dtype=torch.float32,
                      device=qw.packed.device)
    c = qw.c()
    check(lib.qmoe_dequantize(ctypes.byref(c), out.data_ptr(), _stream(out)), "qmoe_dequantize")
    return out


def qlinear_int4(x: torch.Tensor, qw: QWeight, lora: Optional[Lora] = None,
                 adapter_idx: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _dev(x, torch.float16, "x")
    m = x.shape[0]
    y = out if out is not None else torch.empty((m, qw.rows), dtype=torch.float16, device=x.device)
    _dev(y, torch.float16, "out")
    if adapter_idx is not None:
        _dev(adapter_idx, torch.int32, "adapter_idx")
    c = qw.c()
    lc = lora.c() if lora is not None else None
    check(lib.qlinear_int4(x.data_ptr(), m, ctypes.byref(c),
                           ctypes.byref(lc) if lc is not None else None, _ptr(adapter_idx),
                           y.data_ptr(), _stream(x)), "qlinear_int4")
    return y


def router_topk(logits: torch.Tensor, k: int, bias: Optional[torch.Tensor] = None):
    _dev(logits, torch.float32, "logits")
    t, e = logits.shape
    if bias is not None:
        _dev(bias, torch.float32, "bias")
    idx = torch.empty((t, k), dtype=torch.int32, device=logits.device)
    w = torch.empty((t, k), dtype=torch.float32, device=logits.device)
    check(lib.router_topk(logits.data_ptr(), t, e, k, _ptr(bias), idx.data_ptr(), w.data_ptr(),
                          _stream(logits)), "router_topk")
    return idx, w


def lora_apply(x: torch.Tensor, lora: Lora, y_acc: torch.Tensor,
               adapter_idx: Optional[torch.Tensor] = None) -> torch.Tensor:
    _dev(x, torch.float16, "x")
    _dev(y_acc, torch.float32, "y_acc")
    if adapter_idx is not None:
        _dev(adapter_idx, torch.int32, "adapter_idx")
    lc = lora.c()
    check(lib.lora_apply(x.data_ptr(), x.shape[0], ctypes.byref(lc), _ptr(adapter_idx),
                         y_acc.data_ptr(), _stream(x)), "lora_apply")
    return y_acc


def moe_workspace_bytes(layer: MoELayer, max_tokens: int) -> int:
    c = layer.c()
    n = lib.moe_switchglu_int4_workspace_bytes(ctypes.byref(c), max_tokens)
    if n == 0:
        raise ValueError("invalid layer description or token count")
    return n


def moe_workspace(layer: MoELayer, max_tokens: int, device="cuda") -> torch.Tensor:
    """A workspace tensor for up to max_tokens tokens (uint8, 256-byte aligned)."""
    return torch.empty(moe_workspace_bytes(layer, max_tokens), dtype=torch.uint8, device=device)


def _moe_io(layer: MoELayer, x: torch.Tensor, y: torch.Tensor,
            adapter_idx: Optional[torch.Tensor], idx_out: Optional[torch.Tensor],
            w_out: Optional[torch.Tensor], idx_name: str = "idx_out") -> int:
    """Check the per-call tensors of a layer call (the C layer cannot see buffer sizes) and
    return the token count."""
    _dev(x, torch.float16, "x")
    _dev(y, torch.float16, "y")
    if x.dim() != 2 or x.shape[1] != layer.hidden or tuple(y.shape) != tuple(x.shape):
        raise ValueError(f"x and y must be [t, {layer.hidden}], got {tuple(x.shape)} and {tuple(y.shape)}")
    t = x.shape[0]
    for name, v, dt, n in (("adapter_idx", adapter_idx, torch.int32, t),
                           (idx_name, idx_out, torch.int32, t * layer.top_k),
                           ("w_out", w_out, torch.float32, t * layer.top_k)):
        if v is not None:
            _dev(v, dt, name)
            if v.numel() != n:
                raise ValueError(f"{name} must hold {n} elements, got {v.numel()}")
            if v.device != x.device:
                raise ValueError(f"{name} is on {v.device}, x on {x.device}")
    return t


def moe_switchglu_int4(layer: MoELayer, x: torch.Tensor,
                       adapter_idx: Optional[torch.Tensor] = None,
                       ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                       return_routing: bool = False):
    _dev(x, torch.float16, "x")
    t = x.shape[0]
    if ws is None:
        ws = moe_workspace(layer, t, x.device)
    _dev(ws, torch.uint8, "ws")
    y = out if out is not None else torch.empty_like(x)
    idx = w = None
    if return_routing:
        idx = torch.empty((t, layer.top_k), dtype=torch.int32, device=x.device)
        w = torch.empty((t, layer.top_k), dtype=torch.float32, device=x.device)
    _moe_io(layer, x, y, adapter_idx, idx, w)
    c = layer.c()
    check(lib.moe_switchglu_int4(ctypes.byref(c), x.data_ptr(), t, _ptr(adapter_idx),
                                 y.data_ptr(), _ptr(idx), _ptr(w), ws.data_ptr(), ws.numel(),
                                 _stream(x)), "moe_switchglu_int4")
    return (y, idx, w) if return_routing else y


def moe_switchglu_int4_routed(layer: MoELayer, x: torch.Tensor, route: torch.Tensor,
                              adapter_idx: Optional[torch.Tensor] = None,
                              ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                              w_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The layer under a given routing route int32 [t, top_k] (e.g. the prerouter head's
    prediction); w_out (fp32 [t, top_k]) receives the routing weights when given."""
    y = out if out is not None else torch.empty_like(x)
    if route is None:
        raise ValueError("route is required")
    t = _moe_io(layer, x, y, adapter_idx, route, w_out, "route")
    if ws is None:
        ws = moe_workspace(layer, t, x.device)
    _dev(ws, torch.uint8, "ws")
    c = layer.c()
    check(lib.moe_switchglu_int4_routed(ctypes.byref(c), x.data_ptr(), t, _ptr(adapter_idx),
                                        route.data_ptr(), y.data_ptr(), _ptr(w_out), ws.data_ptr(),
                                        ws.numel(), _stream(x)), "moe_switchglu_int4_routed")
    return y


def moe_switchglu_int4_noalloc(layer: MoELayer, x: torch.Tensor,
                               adapter_idx: Optional[torch.Tensor] = None,
                               out: Optional[torch.Tensor] = None,
                               idx_out: Optional[torch.Tensor] = None,
                               w_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The layer with the library's fixed per-device scratch as its workspace (the entry
    point for callers that cannot allocate; overlapping calls on one device race)."""
    y = out if out is not None else torch.empty_like(x)
    t = _moe_io(layer, x, y, adapter_idx, idx_out, w_out)
    c = layer.c()
    check(lib.moe_switchglu_int4_noalloc(ctypes.byref(c), x.data_ptr(), t, _ptr(adapter_idx),
                                         y.data_ptr(), _ptr(idx_out), _ptr(w_out), _stream(x)),
          "moe_switchglu_int4_noalloc")
    return y


STAGE_ALL, STAGE_ROUTE, STAGE_GATE_UP, STAGE_DOWN = 0, 1, 2, 3
PARAM_F16, PARAM_BF16 = 0, 1


class MoECall:
    """A prepared moe_switchglu_int4 call: the C layer struct and every pointer are built
    once, so repeated launches (a decode loop, graph capture) cost one C call each."""

    def __init__(self, layer: MoELayer, x: torch.Tensor, y: torch.Tensor, ws: torch.Tensor,
                 adapter_idx: Optional[torch.Tensor] = None,
                 idx_out: Optional[torch.Tensor] = None, w_out: Optional[torch.Tensor] = None):
        self.t = _moe_io(layer, x, y, adapter_idx, idx_out, w_out)
        _dev(ws, torch.uint8, "ws")
        self.layer, self.x, self.y, self.ws = layer, x, y, ws
        self.adapter_idx, self.idx_out, self.w_out = adapter_idx, idx_out, w_out
        self.c = layer.c()

    def __call__(self, stage: int = STAGE_ALL, stream: Optional[int] = None) -> None:
        s = ctypes.c_void_p(stream if stream is not None
                            else torch.cuda.current_stream(self.x.device).cuda_stream)
        check(lib.moe_switchglu_int4_stage(ctypes.byref(self.c), stage, self.x.data_ptr(), self.t,
                                           _ptr(self.adapter_idx), self.y.data_ptr(),
                                           _ptr(self.idx_out), _ptr(self.w_out),
                                           self.ws.data_ptr(), self.ws.numel(), s),
              "moe_switchglu_int4_stage")


def quantize_supergroup(w: torch.Tensor, period: int = 4) -> SuperGroupWeight:
    _dev(w, torch.float32, "w")
    rows, cols = w.shape
    n4 = rows // period
    p4 = torch.empty((n4, cols // 8), dtype=torch.int32, device=w.device)
    p2 = torch.empty((rows - n4, cols // 16), dtype=torch.int32, device=w.device)
    scales = torch.empty(rows, dtype=torch.float16, device=w.device)
    check(lib.qmoe_quantize_supergroup(w.data_ptr(), rows, cols, period, p4.data_ptr(),
                                       p2.data_ptr() if p2.numel() else None, scales.data_ptr(),
                                       _stream(w)), "qmoe_quantize_supergroup")
    return SuperGroupWeight(p4, p2, scales, period, rows, cols)


def qlinear_supergroup(x: torch.Tensor, W: SuperGroupWeight,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _dev(x, torch.float16, "x")
    b = x.shape[0]
    y = out if out is not None else torch.empty((b, W.rows), dtype=torch.float16, device=x.device)
    _dev(y, torch.float16, "out")
    check(lib.qlinear_supergroup(x.data_ptr(), b, W.p4.data_ptr(),
                                 W.p2.data_ptr() if W.p2.numel() else None, W.scales.data_ptr(),
                                 W.rows, W.cols, W.period, y.data_ptr(), _stream(x)),
          "qlinear_supergroup")
    return y


def quantize_act8(x: torch.Tensor):
    """8-bit per-token activation codes and scales: (qx int8 [b, cols], sx fp16 [b])."""
    _dev(x, torch.float16, "x")
    b, cols = x.shape
    qx = torch.empty((b, cols), dtype=torch.int8, device=x.device)
    sx = torch.empty(b, dtype=torch.float16, device=x.device)
    check(lib.qmoe_quantize_act8(x.data_ptr(), b, cols, qx.data_ptr(), sx.data_ptr(), _stream(x)),
          "qmoe_quantize_act8")
    return qx, sx


def qlinear_supergroup_a8(x: torch.Tensor, W: SuperGroupWeight,
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The super-group GEMM with 8-bit activations and an integer dot product."""
    _dev(x, torch.float16, "x")
    b = x.shape[0]
    y = out if out is not None else torch.empty((b, W.rows), dtype=torch.float16, device=x.device)
    _dev(y, torch.float16, "out")
    check(lib.qlinear_supergroup_a8(x.data_ptr(), b, W.p4.data_ptr(),
                                    W.p2.data_ptr() if W.p2.numel() else None, W.scales.data_ptr(),
                                    W.rows, W.cols, W.period, y.data_ptr(), _stream(x)),
          "qlinear_supergroup_a8")
    return y


@dataclass
class PrerouterHead:
    """One layer's prerouter head on the device: fp16 weights [out, in] and biases;
    w_init [E, D + 2E], w1 [F, D + 2E], w2 [E, F]."""

    w_init: torch.Tensor
    b_init: torch.Tensor
    w1: torch.Tensor
    b1: torch.Tensor
    w2: torch.Tensor
    b2: torch.Tensor

    def c(self) -> PrerouterC:
        E, F = self.w_init.shape[0], self.w1.shape[0]
        D = self.w_init.shape[1] - 2 * E
        for name in ("w_init", "b_init", "w1", "b1", "w2", "b2"):
            _dev(getattr(self, name), torch.float16, name)
        return PrerouterC(self.w_init.data_ptr(), self.b_init.data_ptr(), self.w1.data_ptr(),
                          self.b1.data_ptr(), self.w2.data_ptr(), self.b2.data_ptr(), D, E, F)


def prerouter_forward(P: PrerouterHead, h: torch.Tensor, topk_now: torch.Tensor,
                      topk_prev: torch.Tensor, predict: bool = True):
    """(act fp16 [t, F], logits fp32 [t, E], pred_idx int32 [t, k] or None, pred_w fp32 or
    None) of the prerouter head for t tokens."""
    _dev(h, torch.float16, "h")
    _dev(topk_now, torch.int32, "topk_now")
    _dev(topk_prev, torch.int32, "topk_prev")
    t, k = topk_now.shape
    c = P.c()
    act = torch.empty((t, c.ffn), dtype=torch.float16, device=h.device)
    logits = torch.empty((t, c.n_experts), dtype=torch.float32, device=h.device)
    idx = torch.empty((t, k), dtype=torch.int32, device=h.device) if predict else None
    w = torch.empty((t, k), dtype=torch.float32, device=h.device) if predict else None
    check(lib.prerouter_forward(ctypes.byref(c), h.data_ptr(), t, k, topk_now.data_ptr(),
                                topk_prev.data_ptr(), act.data_ptr(), logits.data_ptr(), _ptr(idx),
                                _ptr(w), _stream(h)), "prerouter_forward")
    return act, logits, idx, w
