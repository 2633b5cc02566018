"""Seeded synthetic inputs for the int4 group-quantized MoE layer.

This module draws random numbers and nothing else: it holds none of the method's
arithmetic (no quantization, no dequantization, no matmul, no routing).  Both the CPU
oracle's tests and the GPU path's tests/benchmarks take their inputs from here, so that
the two sides see the same bytes.

Every stream is keyed by ``SeedSequence([1234, workload, layer, role, index])``, so each
tensor (one expert's gate matrix, one layer's router, one token batch ...) can be drawn on
its own, in any order, and always comes out the same.

Shapes and distributions follow the model the pages describe (Edge0-35B-A3B model
repository guide, "model spec" table: hidden 2048, 256 experts, expert and shared-expert
intermediate 512, 40 layers) with Gaussian weights of standard deviation 0.02 and LoRA
factors of standard deviation 0.01; activations are standard normal rounded to fp16.
"""
from __future__ import annotations

import enum

import numpy as np

ROOT_SEED = 1234


class Role(enum.IntEnum):
    """Which tensor a random stream feeds (part of the seed key)."""

    X = 0
    ROUTER = 1
    SHARED_GATE = 2
    SH_GATE = 3
    SH_UP = 4
    SH_DOWN = 5
    EXP_GATE = 6
    EXP_UP = 7
    EXP_DOWN = 8
    LORA_A_GATE = 9
    LORA_B_GATE = 10
    LORA_A_UP = 11
    LORA_B_UP = 12
    LORA_A_DOWN = 13
    LORA_B_DOWN = 14
    DENSE = 15
    SUPERGROUP = 16
    WORDS = 17
    SCALES = 18
    BIASES = 19
    LOGITS = 20
    MISC = 21


class Workload(enum.IntEnum):
    """Workload ids used in the seed key (one per benchmark workload, plus tests)."""

    GEMV = 0        # single int4 linear, decode
    MOE_DECODE = 1  # one MoE layer, 1 token
    MOE_PREFILL = 2 # one MoE layer, 512 tokens
    MOE_STACK = 3   # 40 layers, 16 tokens, 4 adapters
    SUPERGROUP = 4  # mixed ternary / 4-bit
    TEST = 9        # small shapes used only by tests


def rng(workload: int, layer: int, role: int, index: int = 0) -> np.random.Generator:
    """The generator for one tensor."""
    return np.random.default_rng(
        np.random.SeedSequence([ROOT_SEED, int(workload), int(layer), int(role), int(index)]))


def normal_f32(shape, sigma: float, workload: int, layer: int, role: int,
               index: int = 0) -> np.ndarray:
    """fp32 weights drawn N(0, sigma) (sigma is the standard deviation)."""
    g = rng(workload, layer, role, index)
    return g.standard_normal(shape, dtype=np.float32) * np.float32(sigma)


def normal_f16(shape, sigma: float, workload: int, layer: int, role: int,
               index: int = 0) -> np.ndarray:
    """fp16 tensor: a float64 N(0, sigma) draw rounded once to fp16."""
    g = rng(workload, layer, role, index)
    return (g.standard_normal(shape) * sigma).astype(np.float16)


def activations(tokens: int, hidden: int, workload: int, layer: int = 0,
                index: int = 0) -> np.ndarray:
    """x fp16 [tokens x hidden] ~ N(0, 1)."""
    return normal_f16((tokens, hidden), 1.0, workload, layer, Role.X, index)


def random_words(shape, workload: int, layer: int, role: int, index: int = 0) -> np.ndarray:
    """Uniformly random uint32 words (packed integer codes taken as given)."""
    g = rng(workload, layer, role, index)
    return g.integers(0, 2**32, size=shape, dtype=np.uint64).astype(np.uint32)


def binomial_codes(shape, levels: int, workload: int, layer: int, role: int,
                   index: int = 0) -> np.ndarray:
    """Integer codes in [0, levels-1], bell-shaped (Binomial(levels-1, 1/2)), uint8."""
    g = rng(workload, layer, role, index)
    return g.binomial(levels - 1, 0.5, size=shape).astype(np.uint8)


def uniform_f16(shape, lo: float, hi: float, workload: int, layer: int, role: int,
                index: int = 0) -> np.ndarray:
    """fp16 values drawn uniformly from [lo, hi) (float64 draw rounded to fp16)."""
    g = rng(workload, layer, role, index)
    return g.uniform(lo, hi, size=shape).astype(np.float16)


def expert_choices(tokens: int, k: int, n_experts: int, workload: int, layer: int = 0,
                   index: int = 0) -> np.ndarray:
    """A routing drawn at random: for each token, k distinct experts of n_experts, int32
    [tokens x k] (stands in for a routing the caller supplies, e.g. a predicted one)."""
    g = rng(workload, layer, Role.MISC, 1000 + index)
    return np.stack([g.choice(n_experts, k, replace=False) for _ in range(tokens)]).astype(np.int32)


def adapter_index(tokens: int, tokens_per_adapter: int) -> np.ndarray:
    """Per-token adapter id: token t is served by adapter t // tokens_per_adapter."""
    return (np.arange(tokens, dtype=np.int32) // np.int32(tokens_per_adapter)).astype(np.int32)


# Model shapes of the pages' 35B-A3B MoE (see module docstring).
HIDDEN = 2048
N_EXPERTS = 256
INTER = 512
SHARED_INTER = 512
N_LAYERS = 40
GROUP = 64
LORA_RANK = 16
LORA_ALPHA = 32.0
WEIGHT_SIGMA = 0.02
LORA_SIGMA = 0.01
