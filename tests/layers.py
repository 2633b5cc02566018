"""Build MoE layers for the tests: oracle-side (numpy) and device-side (torch) views of the
same bytes.

Weights come from ``synth`` (seeded per tensor) and are quantized by the *oracle*, so
every expected value traces back to the oracle and the seeded generators only.  Experts
are quantized in a process pool.  ``only_experts`` restricts quantization to the experts a
test can reach; the others are filled with random packed words and random fp16
parameters drawn from ``synth`` (as if imported from a pre-quantized checkpoint), which
the oracle evaluates like any other expert.
"""
from __future__ import annotations

import concurrent.futures
import os
from dataclasses import dataclass
from typing import Iterable, Optional

import numpy as np

import synth
from oracle import affine, moe

R = synth.Role


@dataclass
class Shape:
    hidden: int = synth.HIDDEN
    inter: int = synth.INTER
    shared_inter: int = synth.SHARED_INTER
    n_experts: int = synth.N_EXPERTS
    top_k: int = 4
    rank: int = synth.LORA_RANK
    n_adapters: int = 1
    alpha: float = synth.LORA_ALPHA


def _quant(args):
    wl, layer, role, index, rows, cols, bits = args[:7]
    group, params = args[7:] if len(args) > 7 else (64, "f16")
    w = synth.normal_f32((rows, cols), synth.WEIGHT_SIGMA, wl, layer, role, index)
    q = affine.quantize(w, bits, group, params)
    return q.packed, q.scales, q.biases


def _filler(wl, layer, role, index, rows, cols):
    words = synth.random_words((rows, cols // 8), wl, layer, R.WORDS, index * 16 + int(role))
    s = synth.uniform_f16((rows, cols // 64), 0.004, 0.012, wl, layer, R.SCALES, index * 16 + int(role))
    b = (-7.5 * s.astype(np.float64)).astype(np.float16)
    return words, s, b


def _pool():
    n = min(8, os.cpu_count() or 1)
    return concurrent.futures.ProcessPoolExecutor(max_workers=n)


def quantize_many(jobs):
    jobs = list(jobs)
    if len(jobs) <= 2:
        return [_quant(j) for j in jobs]
    with _pool() as ex:
        return list(ex.map(_quant, jobs, chunksize=4))


def stack(parts, group=64, params="f16"):
    return affine.QWeight(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]),
                          np.stack([p[2] for p in parts]), 4, group, params)


def one(part, bits):
    return affine.QWeight(part[0], part[1], part[2], bits, 64)


def build_layer(wl: int, layer: int, S: Shape, with_lora: bool = True, skew: bool = False,
                only_experts: Optional[Iterable[int]] = None, expert_group: int = 64,
                expert_params: str = "f16") -> moe.MoELayer:
    """Oracle-side layer.  ``only_experts=None`` quantizes every expert.  The routed expert
    stacks may take group 32 and/or bf16 parameters (then every expert is quantized)."""
    std = expert_group == 64 and expert_params == "f16"
    assert std or only_experts is None, "filler experts are group 64, fp16"
    H, I, SI, E = S.hidden, S.inter, S.shared_inter, S.n_experts
    dense = [(wl, layer, R.ROUTER, 0, E, H, 8), (wl, layer, R.SHARED_GATE, 0, 1, H, 8),
             (wl, layer, R.SH_GATE, 0, SI, H, 4), (wl, layer, R.SH_UP, 0, SI, H, 4),
             (wl, layer, R.SH_DOWN, 0, H, SI, 4)]
    wanted = set(range(E)) if only_experts is None else set(int(e) for e in only_experts)
    ejobs = []
    for e in sorted(wanted):
        fmt = () if std else (expert_group, expert_params)
        ejobs += [(wl, layer, R.EXP_GATE, e, I, H, 4) + fmt, (wl, layer, R.EXP_UP, e, I, H, 4) + fmt,
                  (wl, layer, R.EXP_DOWN, e, H, I, 4) + fmt]
    res = quantize_many(dense + ejobs)
    router, sgate, shg, shu, shd = res[:5]
    got = {}
    for i, e in enumerate(sorted(wanted)):
        got[e] = res[5 + 3 * i:5 + 3 * i + 3]
    gates, ups, downs = [], [], []
    for e in range(E):
        if e in got:
            g, u, d = got[e]
        else:
            g = _filler(wl, layer, R.EXP_GATE, e, I, H)
            u = _filler(wl, layer, R.EXP_UP, e, I, H)
            d = _filler(wl, layer, R.EXP_DOWN, e, H, I)
        gates.append(g); ups.append(u); downs.append(d)
    loras = [None, None, None]
    if with_lora:
        specs = [(R.LORA_A_GATE, R.LORA_B_GATE, H, SI), (R.LORA_A_UP, R.LORA_B_UP, H, SI),
                 (R.LORA_A_DOWN, R.LORA_B_DOWN, SI, H)]
        for i, (ra, rb, din, dout) in enumerate(specs):
            A = synth.normal_f16((S.n_adapters, S.rank, din), synth.LORA_SIGMA, wl, layer, ra)
            B = synth.normal_f16((S.n_adapters, dout, S.rank), synth.LORA_SIGMA, wl, layer, rb)
            loras[i] = moe.Lora(A, B, S.alpha / S.rank)
    bias = None
    if skew:
        bias = np.zeros(E, np.float32)
        bias[:16] = 2.0
    ef = (expert_group, expert_params)
    return moe.MoELayer(router=one(router, 8), shared_gate=one(sgate, 8), exp_gate=stack(gates, *ef),
                        exp_up=stack(ups, *ef), exp_down=stack(downs, *ef), sh_gate=one(shg, 4),
                        sh_up=one(shu, 4), sh_down=one(shd, 4), top_k=S.top_k,
                        lora_gate=loras[0], lora_up=loras[1], lora_down=loras[2],
                        router_bias=bias)


def routed_experts(x: np.ndarray, wl: int, layer: int, S: Shape, skew: bool = False,
                   margin: int = 2) -> set:
    """Experts the oracle's router picks for x, plus the next ``margin`` per token (so a
    near-tie on the device still lands on a quantized expert)."""
    r = _quant((wl, layer, R.ROUTER, 0, S.n_experts, S.hidden, 8))
    ell = moe.router_logits(x, one(r, 8), None)
    if skew:
        b = np.zeros(S.n_experts)
        b[:16] = 2.0
        ell = ell + b
    order = np.argsort(-ell, axis=1, kind="stable")[:, :S.top_k + margin]
    return set(order.ravel().tolist())


def to_device(L: moe.MoELayer, S: Shape, device="cuda", add_residual=False):
    """Device-side view (int4_group_quantized_amd.MoELayer) of an oracle layer."""
    import torch
    import int4_group_quantized_amd as q

    def qw(w: affine.QWeight):
        return q.QWeight.from_arrays(w.packed, w.scales, w.biases, w.bits, device, group=w.group,
                                     param_dtype=q.PARAM_BF16 if w.param_dtype == "bf16" else 0)

    def lo(l):
        if l is None:
            return None
        return q.Lora(torch.from_numpy(l.A).to(device), torch.from_numpy(l.B).to(device), l.scale)

    bias = None if L.router_bias is None else torch.from_numpy(L.router_bias).to(device)
    return q.MoELayer(hidden=S.hidden, inter=S.inter, shared_inter=S.shared_inter,
                      n_experts=S.n_experts, top_k=L.top_k, router=qw(L.router),
                      shared_gate=qw(L.shared_gate), exp_gate=qw(L.exp_gate), exp_up=qw(L.exp_up),
                      exp_down=qw(L.exp_down), sh_gate=qw(L.sh_gate), sh_up=qw(L.sh_up),
                      sh_down=qw(L.sh_down), lora_gate=lo(L.lora_gate), lora_up=lo(L.lora_up),
                      lora_down=lo(L.lora_down), router_bias=bias, add_residual=add_residual)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# Tolerance for every floating-point output against the float64 oracle: max abs 2e-2 and
# relative L2 1e-3 (the bar stated for this layer).
MAX_ABS = 2e-2
MAX_REL_L2 = 1e-3


def assert_close(got, ref, max_abs=MAX_ABS, max_rel=MAX_REL_L2, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.max(np.abs(got - ref)) if got.size else 0.0
    rel = rel_l2(got, ref) if got.size else 0.0
    assert err <= max_abs and rel <= max_rel, f"{what}: max abs {err:.3g}, rel L2 {rel:.3g}"
    return err, rel
