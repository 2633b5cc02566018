"""Prerouter head forward (oracle; test infrastructure only).

Source: "Edge0 project review" (blog.kxstl.cn), highlight 1 (prerouter, the "double
shift"): layer N owns a small head whose input is layer N's MoE input h together with the
experts this token was actually routed to and those the previous token was routed to, each
as a one-hot vector over the E experts; the head predicts layer N + 1's routing as
``logits = linear_init(feats) + fc2(gelu_erf(fc1(feats)))`` with
``feats = concat([h, executed_topk_onehot, prev_token_topk_onehot])``; the GELU is the exact
erf form; weights and arithmetic are fp16 (the page's 35B model: 33 heads of hidden 512).

Readings where the page is silent or garbled:
* h has the layer's hidden size D (the MoE input); the comment's "512 + 2E" is read as the
  head width, which is F = 512 here; feats has D + 2E entries in the order above.
* linear_init, fc1 and fc2 are linear layers with biases (weights [out][in], fp16).
* A one-hot over the K routed experts has K ones (a multi-hot vector).
* fp16 module semantics: every layer's output is rounded to fp16 (accumulation in full
  precision here): z = fp16(fc1 f), a = fp16(gelu_erf(z)), y2 = fp16(fc2 a),
  y0 = fp16(linear_init f), logits = fp16(y0 + y2).
* The predicted routing is the top-K of the logits with the router's rule (lower index on
  ties), softmax over the K.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
from scipy.special import erf


@dataclass
class PrerouterHead:
    w_init: np.ndarray   # fp16 [E, D + 2E]
    b_init: np.ndarray   # fp16 [E]
    w1: np.ndarray       # fp16 [F, D + 2E]
    b1: np.ndarray       # fp16 [F]
    w2: np.ndarray       # fp16 [E, F]
    b2: np.ndarray       # fp16 [E]

    @property
    def n_experts(self) -> int:
        return int(self.w_init.shape[0])

    @property
    def hidden(self) -> int:
        return int(self.w_init.shape[1]) - 2 * self.n_experts


def gelu_erf(z: np.ndarray) -> np.ndarray:
    """0.5 z (1 + erf(z / sqrt(2))) in float64."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))


def features(h: np.ndarray, topk_now: np.ndarray, topk_prev: np.ndarray, E: int) -> np.ndarray:
    """feats [T, D + 2E] = [h, multi-hot(topk_now), multi-hot(topk_prev)] in float64."""
    h = np.asarray(h, dtype=np.float64)
    T, D = h.shape
    f = np.zeros((T, D + 2 * E), dtype=np.float64)
    f[:, :D] = h
    for t in range(T):
        f[t, D + np.asarray(topk_now[t])] = 1.0
        f[t, D + E + np.asarray(topk_prev[t])] = 1.0
    return f


def f16(v: np.ndarray) -> np.ndarray:
    return np.asarray(v, dtype=np.float64).astype(np.float16)


def forward(P: PrerouterHead, h: np.ndarray, topk_now: np.ndarray, topk_prev: np.ndarray):
    """Returns (a fp16 [T, F], logits fp16 [T, E]) with the fp16 rounding points of the
    module docstring."""
    f = features(h, topk_now, topk_prev, P.n_experts)
    z = f16(f @ P.w1.astype(np.float64).T + P.b1.astype(np.float64))
    a = f16(gelu_erf(z.astype(np.float64)))
    y2 = f16(a.astype(np.float64) @ P.w2.astype(np.float64).T + P.b2.astype(np.float64))
    y0 = f16(f @ P.w_init.astype(np.float64).T + P.b_init.astype(np.float64))
    logits = f16(y0.astype(np.float64) + y2.astype(np.float64))
    return a, logits
