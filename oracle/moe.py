"""Quantized linear, LoRA, router, SwitchGLU experts, shared expert, MoE layer (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).  Everything is float64 on the exact
dequantized weights; fp16 outputs are rounded once at the end.

Sources
-------
* "Edge0-35B-A3B Preview model repository guide" (trdm.cn), "model spec" table and the
  shared-expert paragraph: 256 routed experts per layer, expert intermediate 512, a shared
  expert of intermediate 512 next to the 256-way switch MLP, gated by
  ``shared_expert_gate``; experts are stored as ``switch_mlp.gate_proj / up_proj /
  down_proj``.  The same page and the Recover-LoRA page (section 1) give K = 4 routed
  experts per token (the config file says 8; both values are used).
* "Edge0 project review" (blog.kxstl.cn), highlight 2 and the strengths list: the MoE spec
  names the routing family SOFTMAX_TOPK; the expert combine is ``_swiglu(up, gate)`` and
  swapping gate and up moves the relative L2 error from 0.2 % to 100 %; a missing expert
  contributes nothing.  Highlight 3: the LoRA adapter is a parallel delta on a read-only
  base, never merged; one base serves many adapter sets.
* "Recover-LoRA ..." (bjdmk.com.cn), section 2: frozen int4 base plus an unmerged LoRA
  added at inference; one read-only base serves many adapter sets.

Readings where the pages are silent: SiLU(z) = z / (1 + e^-z)
applied to the gate projection and multiplied by the up projection; the shared expert is
scaled by sigmoid of the 8-bit gate's logit; the LoRA delta is ``(alpha/r) * B (A v)`` on
each of the shared expert's three projections, with the projection's own input ``v``; the
router picks the K largest logits (ties to the lower expert index) and the routing weights
are the softmax renormalized over the selected K; the layer output is
``fp16(sum_k w_k o_k + gamma * o_shared)``; stacked layers add a residual
``x_{l+1} = fp16(x_l + y_l)``.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from .affine import QWeight, dequantize


# ----------------------------------------------------------------------------------------
# building blocks
# ----------------------------------------------------------------------------------------

@dataclass
class Lora:
    """Unmerged low-rank adapter(s) on one projection.

    A      fp16 [n_adapters, rank, in_dim]
    B      fp16 [n_adapters, out_dim, rank]
    scale  alpha / rank
    """

    A: np.ndarray
    B: np.ndarray
    scale: float


def to_f16(y: np.ndarray) -> np.ndarray:
    """Round to fp16 once, round-to-nearest-even."""
    return np.asarray(y, dtype=np.float64).astype(np.float16)


def linear(v: np.ndarray, qw: QWeight) -> np.ndarray:
    """``v @ W_hat^T`` in float64 for v [T, cols]; W_hat is the exact dequantized matrix."""
    return np.asarray(v, dtype=np.float64) @ dequantize(qw).T


def lora_delta(v: np.ndarray, lora: Lora, adapter_idx: Optional[np.ndarray]) -> np.ndarray:
    """``scale * B_a (A_a v_t)`` for each row t of v, with a = adapter_idx[t] (or 0)."""
    v = np.asarray(v, dtype=np.float64)
    T = v.shape[0]
    out_dim = lora.B.shape[1]
    d = np.zeros((T, out_dim), dtype=np.float64)
    for t in range(T):
        a = 0 if adapter_idx is None else int(adapter_idx[t])
        z = lora.A[a].astype(np.float64) @ v[t]            # [rank]
        d[t] = lora.scale * (lora.B[a].astype(np.float64) @ z)
    return d


def qlinear(x: np.ndarray, qw: QWeight, lora: Optional[Lora] = None,
            adapter_idx: Optional[np.ndarray] = None) -> np.ndarray:
    """Quantized linear ``x W_hat^T (+ LoRA delta)``, float64 before output rounding."""
    y = linear(x, qw)
    if lora is not None:
        y = y + lora_delta(x, lora, adapter_idx)
    return y


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


# ----------------------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------------------

def router_logits(x: np.ndarray, router: QWeight,
                  bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Router logits [T, E] = x W_router^T (+ a per-expert additive bias)."""
    ell = linear(x, router)
    if bias is not None:
        ell = ell + np.asarray(bias, dtype=np.float64)[None, :]
    return ell


def topk(logits: np.ndarray, k: int):
    """Top-K expert selection and renormalized softmax weights, per token.

    The selected set is the K largest logits, an exact tie going to the lower expert
    index.  Softmax is strictly increasing, so this is the top-K of the softmax
    probabilities; choosing on the logits keeps rounding of the probabilities from creating
    ties.  The weights are ``p_k / sum_{j in S} p_j`` for ``p = softmax(logits)``, written
    as ``exp(l_k - m) / sum_{j in S} exp(l_j - m)`` with ``m`` the largest selected logit.

    Returns ``(idx int32 [T, K] in selection order, w float64 [T, K])``.
    """
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("k must be in [1, E]")
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))
        sel = order[:k]
        m = logits[t, sel[0]]
        ex = np.array([np.exp(logits[t, e] - m) for e in sel])
        idx[t] = sel
        w[t] = ex / ex.sum()
    return idx, w


def topk_f32(logits32: np.ndarray, k: int, bias32: Optional[np.ndarray] = None):
    """Top-K on float32 logits plus an optional float32 per-expert bias, the sum rounded to
    float32 before any comparison (the precision in which the device takes the decision).
    Weights as in :func:`topk`."""
    ell = np.asarray(logits32, dtype=np.float32)
    if bias32 is not None:
        ell = ell + np.asarray(bias32, dtype=np.float32)[None, :]
    return topk(ell.astype(np.float64), k)


def topk_gap(logits: np.ndarray, k: int) -> np.ndarray:
    """Per token, the K-th largest logit minus the (K+1)-th (inf when K == E)."""
    s = -np.sort(-np.asarray(logits, dtype=np.float64), axis=1)
    if k >= s.shape[1]:
        return np.full(s.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


# ----------------------------------------------------------------------------------------
# experts and the layer
# ----------------------------------------------------------------------------------------

@dataclass
class MoELayer:
    """One MoE SwitchGLU layer in its stored (quantized) form.

    router       8-bit QWeight [E, hidden]
    shared_gate  8-bit QWeight [1, hidden]
    exp_gate/up  int4 expert stacks [E, inter, hidden]; exp_down [E, hidden, inter]
    sh_gate/up   int4 [shared_inter, hidden]; sh_down [hidden, shared_inter]
    lora_*       optional adapters on the shared expert's three projections
    router_bias  optional float32 [E] added to the logits
    """

    router: QWeight
    shared_gate: QWeight
    exp_gate: QWeight
    exp_up: QWeight
    exp_down: QWeight
    sh_gate: QWeight
    sh_up: QWeight
    sh_down: QWeight
    top_k: int
    lora_gate: Optional[Lora] = None
    lora_up: Optional[Lora] = None
    lora_down: Optional[Lora] = None
    router_bias: Optional[np.ndarray] = None

    @property
    def n_experts(self) -> int:
        return int(self.exp_gate.scales.shape[0])


def expert_mlp(x: np.ndarray, gate: QWeight, up: QWeight, down: QWeight) -> np.ndarray:
    """One routed expert: ``down( silu(gate(x)) * up(x) )``, float64."""
    g = linear(x, gate)
    u = linear(x, up)
    return linear(silu(g) * u, down)


def shared_expert(x: np.ndarray, L: MoELayer, adapter_idx: Optional[np.ndarray]) -> np.ndarray:
    """The shared expert with its LoRA deltas inside each projection (before gating)."""
    gs = qlinear(x, L.sh_gate, L.lora_gate, adapter_idx)
    us = qlinear(x, L.sh_up, L.lora_up, adapter_idx)
    hs = silu(gs) * us
    return qlinear(hs, L.sh_down, L.lora_down, adapter_idx)


def shared_gate_value(x: np.ndarray, L: MoELayer) -> np.ndarray:
    """gamma [T] = sigmoid of the 8-bit shared-expert gate's logit."""
    return sigmoid(linear(x, L.shared_gate)[:, 0])


def moe_layer(x: np.ndarray, L: MoELayer, adapter_idx: Optional[np.ndarray] = None,
              idx: Optional[np.ndarray] = None) -> dict:
    """Full layer forward.  Returns a dict with

    ``logits`` [T,E], ``idx`` [T,K], ``w`` [T,K], ``routed`` [T,H], ``shared`` [T,H],
    ``gamma`` [T], ``y64`` [T,H] (float64) and ``y`` (fp16).

    ``idx`` may be given to evaluate the layer under a stated selection (for instance an
    alternative top-K at a logit near-tie); the weights are then the renormalized softmax
    over that selection.
    """
    x = np.asarray(x)
    T = x.shape[0]
    logits = router_logits(x, L.router, L.router_bias)
    if idx is None:
        idx, w = topk(logits, L.top_k)
    else:
        idx = np.asarray(idx, dtype=np.int32)
        w = np.empty(idx.shape, dtype=np.float64)
        for t in range(T):
            sel = logits[t, idx[t]]
            ex = np.exp(sel - sel.max())
            w[t] = ex / ex.sum()
    xd = x.astype(np.float64)
    # one expert at a time, each applied to the tokens that picked it
    o = np.zeros(idx.shape + (x.shape[1],), dtype=np.float64)
    for e in np.unique(idx):
        rows, ks = np.nonzero(idx == e)
        o[rows, ks] = expert_mlp(xd[rows], L.exp_gate.expert(e), L.exp_up.expert(e),
                                 L.exp_down.expert(e))
    routed = np.zeros((T, x.shape[1]), dtype=np.float64)
    for k in range(idx.shape[1]):
        routed = routed + w[:, k:k + 1] * o[:, k]
    shared = shared_expert(xd, L, adapter_idx)
    gamma = shared_gate_value(xd, L)
    y64 = routed + gamma[:, None] * shared
    return dict(logits=logits, idx=idx, w=w, routed=routed, shared=shared, gamma=gamma,
                y64=y64, y=to_f16(y64))


def residual(x: np.ndarray, y: np.ndarray) -> np.ndarray:
    """``fp16(x + y)`` for fp16 x and y (the float64 sum is exact, one rounding)."""
    return to_f16(np.asarray(x, np.float64) + np.asarray(y, np.float64))


def moe_stack(x: np.ndarray, layers: Sequence[MoELayer],
              adapter_idx: Optional[np.ndarray] = None) -> list:
    """Layers chained with a residual: ``x_{l+1} = fp16(x_l + y_l)``.

    Returns the list of per-layer inputs ``[x_0, x_1, ..., x_L]`` (fp16).
    """
    xs = [np.asarray(x, dtype=np.float16)]
    for L in layers:
        y = moe_layer(xs[-1], L, adapter_idx)["y"]
        xs.append(residual(xs[-1], y))
    return xs
