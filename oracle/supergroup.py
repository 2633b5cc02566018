"""Mixed ternary / 4-bit super-group quantization and weight-only GEMM (oracle; test-only).

Source: "EDGERAZOR deep dive: how 1.58-bit quantization makes on-device models 15x faster"
(zhichai.net), section 2.1 "SQMP: structural mixed-precision quantization":
* a fraction rho of the weights is 4-bit, the rest 1.58-bit (ternary); super-group
  allocation splits the output channels into periodic blocks of floor(1/rho) consecutive
  channels, exactly one of which is 4-bit;
* ternary quantizer ``Q(w) = clip(round(w / s), -1, 1)`` with
  ``s = max(beta * mean(|w|), eps)``, beta = 2;
* 4-bit quantizer ``Q(w) = round(w / s)`` with ``s = max(max(|w|) / (2^(n-1) - 1), eps)``;
* the matmul factors into a 16-bit scale product times a low-precision integer dot
  product: ``Y = sum (s_W s_X) Q(W)^T Q(X)``; weight-only here, so ``s_X = 1`` and x stays
  fp16.

Readings where the pages are silent: per-channel scales (mean / max over the channel's inputs);
the *first* channel of every block is the 4-bit one; eps = 1e-5 for both quantizers; the
scale is stored as fp16 and the codes are taken against the stored scale, in float32, ties
to even; the ternary mean is summed in float64 and rounded once to float32 so that its value
does not depend on the summation order; codes are stored as ``q + 8`` in nibbles
(8 per uint32) for 4-bit channels and ``q + 1`` in 2-bit fields (16 per uint32) for ternary
channels, lowest field first; the two kinds of rows live in two separate arrays, in channel
order.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

EPS = np.float32(1e-5)
BETA = np.float32(2.0)


@dataclass
class SuperGroupWeight:
    """p4      uint32 [rows / period, cols / 8]        4-bit channels, nibble = q + 8
    p2      uint32 [rows - rows/period, cols / 16]  ternary channels, 2-bit code = q + 1
    scales  fp16 [rows]                             one per output channel
    """

    p4: np.ndarray
    p2: np.ndarray
    scales: np.ndarray
    period: int
    rows: int
    cols: int


def is_four_bit(n: int, period: int) -> bool:
    """Channel n is the 4-bit member of its block of ``period`` channels."""
    return n % period == 0


def quantize_channel(w: np.ndarray, four_bit: bool):
    """One output channel (float32 [cols]) -> (codes int8 [cols], fp16 scale)."""
    w = np.asarray(w, dtype=np.float32)
    if four_bit:
        s32 = np.maximum(np.max(np.abs(w)) / np.float32(7), EPS)          # 2^(4-1) - 1
        qmax = np.float32(7)
    else:
        mean = np.float32(np.sum(np.abs(w).astype(np.float64)) / w.size)
        s32 = np.maximum(BETA * mean, EPS)
        qmax = np.float32(1)
    s16 = np.float16(s32)
    q = np.clip(np.rint(w / np.float32(s16)), -qmax, qmax)
    return q.astype(np.int8), s16


def quantize(w: np.ndarray, period: int = 4):
    """Quantize a float32 [rows, cols] matrix.  Returns (SuperGroupWeight, codes int8)."""
    w = np.asarray(w, dtype=np.float32)
    rows, cols = w.shape
    if rows % period or cols % 16:
        raise ValueError("rows must be a multiple of the period and cols of 16")
    codes = np.empty((rows, cols), dtype=np.int8)
    scales = np.empty(rows, dtype=np.float16)
    for n in range(rows):
        codes[n], scales[n] = quantize_channel(w[n], is_four_bit(n, period))
    four = np.array([is_four_bit(n, period) for n in range(rows)])
    p4 = pack_fields((codes[four].astype(np.int16) + 8).astype(np.uint8), 4)
    p2 = pack_fields((codes[~four].astype(np.int16) + 1).astype(np.uint8), 2)
    return SuperGroupWeight(p4, p2, scales, period, rows, cols), codes


def pack_fields(u: np.ndarray, bits: int) -> np.ndarray:
    """uint8 [r, c] fields -> uint32 [r, c*bits/32], lowest field first."""
    per = 32 // bits
    r, c = u.shape
    f = u.reshape(r, c // per, per).astype(np.uint32)
    words = np.zeros((r, c // per), dtype=np.uint32)
    for j in range(per):
        words |= f[:, :, j] << np.uint32(bits * j)
    return words


def unpack_fields(words: np.ndarray, bits: int) -> np.ndarray:
    per = 32 // bits
    mask = np.uint32(2 ** bits - 1)
    r, nw = words.shape
    u = np.empty((r, nw, per), dtype=np.uint8)
    for j in range(per):
        u[:, :, j] = (words >> np.uint32(bits * j)) & mask
    return u.reshape(r, nw * per)


def codes_of(W: SuperGroupWeight) -> np.ndarray:
    """Signed codes int8 [rows, cols] recovered from the two packed arrays."""
    c4 = unpack_fields(W.p4, 4).astype(np.int16) - 8
    c2 = unpack_fields(W.p2, 2).astype(np.int16) - 1
    codes = np.empty((W.rows, W.cols), dtype=np.int8)
    i4 = i2 = 0
    for n in range(W.rows):
        if is_four_bit(n, W.period):
            codes[n] = c4[i4]
            i4 += 1
        else:
            codes[n] = c2[i2]
            i2 += 1
    return codes


def gemm(x: np.ndarray, W: SuperGroupWeight) -> np.ndarray:
    """``y[b, n] = s_n * sum_k q[n, k] x[b, k]`` in float64 (before fp16 rounding)."""
    q = codes_of(W).astype(np.float64)
    acc = np.asarray(x, dtype=np.float64) @ q.T          # the integer-code dot product
    return acc * W.scales.astype(np.float64)[None, :]   # scale applied once per channel


# ---- weight-activation integer path ---------------------------------------------------------
#
# Same section of the same page: in ``Y = sum (s_W s_X) Q(W)^T Q(X)`` the activations are
# quantized too, so that the sum over the inputs is a pure integer dot product and the scale
# product (s_W s_X) is applied once per output; the page's weight-activation results quantize
# activations to 8 bits (its table of 1.58-8-8 / 1.88-8-8 runs).  Readings where the page is
# silent: one activation scale per token (row of X), symmetric, with the page's 4-bit formula
# at n = 8: ``s_X = max(max|x| / (2^(8-1) - 1), eps)`` (in float32) stored as fp16;
# ``Q(x) = clip(rint(x / s_X), -127, 127)`` with the quotient taken in float32 against the
# stored scale, ties to even (the same reading as the weight quantizers above).  The integer
# dot is exact; the scale product and the final scaling are done in full precision here (the
# fp16 factors are exact in float64) and the result is rounded to fp16 once.

ACT_QMAX = np.float32(127)    # 2^(8-1) - 1


def quantize_activations(x: np.ndarray):
    """x fp16 [B, K] -> (codes int8 [B, K], scales fp16 [B]), one symmetric scale per token."""
    x = np.asarray(x, dtype=np.float16).astype(np.float32)
    amax = np.max(np.abs(x), axis=1)
    s16 = np.maximum(amax / ACT_QMAX, EPS).astype(np.float16)
    q = np.clip(np.rint(x / s16.astype(np.float32)[:, None]), -ACT_QMAX, ACT_QMAX)
    return q.astype(np.int8), s16


def gemm_a8(x: np.ndarray, W: SuperGroupWeight) -> np.ndarray:
    """``y[b, n] = s_W[n] s_X[b] sum_k Q(W)[n, k] Q(X)[b, k]`` in float64 (before fp16
    rounding); the sum over k in exact integer arithmetic."""
    qx, sx = quantize_activations(x)
    acc = qx.astype(np.int64) @ codes_of(W).astype(np.int64).T
    return acc.astype(np.float64) * sx.astype(np.float64)[:, None] * W.scales.astype(np.float64)[None, :]
