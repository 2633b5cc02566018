"""Group-wise affine quantization: quantize, pack, unpack, dequantize (oracle; test-only).

Sources
-------
* "Recover-LoRA: how Edge0 recovers the precision lost to 4-bit compression"
  (bjdmk.com.cn), section 1 "what 4-bit compresses away": the checkpoint's ``quantization``
  field is 4-bit, group_size 64, affine mode — every 64 consecutive elements share one
  scale and one offset; every linear layer is stored as three tensors ``weight``,
  ``scales``, ``biases`` (integer weights plus per-group float parameters, dequantized to
  float at inference).  The router gate and the shared-expert gate are overridden to
  8-bit.
* "Bit-exact MLX 4-bit port of d1a-e2b-it-qat-4bit" (gtnt.cn), section "4-bit group
  quantization": integers stored as packed words, one scale and one bias per group; the
  dequantized weight is the scale times the integer plus the bias (the operator between the
  two is lost in the page's text; the tensors are called *biases*, so the offset is added).

Readings where the pages are silent:
* The scale is ``(max - min) / (2^bits - 1)`` and the bias is the group minimum (min-max
  affine), both computed in float32 and stored as fp16 (round-to-nearest-even).
* The integer code uses the *stored* fp16 scale and bias:
  ``q = clip(rint((w - bias) / scale), 0, 2^bits - 1)`` in float32, ties to even.
* A group whose stored scale is 0 (all elements equal) gets ``q = 0``, so it dequantizes to
  its bias exactly.
* Word layout: row-major, groups consecutive along the input dimension; element ``8m+j`` of
  a row sits in bits ``[4j, 4j+4)`` of word ``m`` (least-significant nibble first); for
  8-bit, element ``4m+j`` is byte ``j`` of word ``m``.

The port page's own checkpoint ("Bit-exact MLX 4-bit port ...", section "4-bit group
quantization", its config's quantization rule) uses 32 weights per group and stores each
group's scale and bias as bf16; its weights come out of quantization-aware training as
integers plus those parameters, so they are taken as given (no requantization) and the
dequantized value is exactly scale * q + bias.  Here a weight's parameters are either fp16
(``param_dtype = "f16"``, float16 arrays) or bf16 (``"bf16"``, uint16 arrays holding the
bf16 bit patterns); the group is 64 or 32.  Rounding to bf16 is to nearest, ties to even,
like the fp16 rounding above.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class QWeight:
    """One quantized matrix (or a stack of per-expert matrices along a leading axis).

    packed  uint32 [..., rows, cols * bits / 32]
    scales  float16 [..., rows, cols / group]
    biases  float16 [..., rows, cols / group]
    """

    packed: np.ndarray
    scales: np.ndarray
    biases: np.ndarray
    bits: int
    group: int
    param_dtype: str = "f16"

    @property
    def rows(self) -> int:
        return int(self.scales.shape[-2])

    @property
    def cols(self) -> int:
        return int(self.scales.shape[-1]) * self.group

    def expert(self, e: int) -> "QWeight":
        """The e-th matrix of an expert stack."""
        return QWeight(self.packed[e], self.scales[e], self.biases[e], self.bits, self.group,
                       self.param_dtype)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even (finite input):
    the upper 16 bits of the float32 pattern after adding 0x7FFF plus the lowest kept bit."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def params_f32(qw: "QWeight"):
    """The stored scales and biases as float32 (exact for either parameter type)."""
    if qw.param_dtype == "bf16":
        return bf16_to_f32(qw.scales), bf16_to_f32(qw.biases)
    return qw.scales.astype(np.float32), qw.biases.astype(np.float32)


def quantize_codes(w: np.ndarray, bits: int, group: int, param_dtype: str = "f16"):
    """Min-max affine quantization of a float32 matrix, per row and per group.

    Returns ``(q uint8 [rows, cols], scales [rows, cols/group], biases [...])``, the
    parameters as fp16 values or bf16 bit patterns.  Every decision is taken in float32 on
    the stored parameters (module docstring).
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    if cols % group != 0:
        raise ValueError("cols must be a multiple of the group size")
    top = np.float32(2 ** bits - 1)
    v = w.reshape(rows, cols // group, group)
    lo = v.min(axis=2)                                # float32, exact
    hi = v.max(axis=2)
    scale32 = (hi - lo) / top                         # float32 subtract, float32 divide
    if param_dtype == "bf16":                         # stored parameters (RNE)
        scales, biases = bf16_bits(scale32), bf16_bits(lo)
        s, b = bf16_to_f32(scales)[:, :, None], bf16_to_f32(biases)[:, :, None]
    else:
        scales, biases = scale32.astype(np.float16), lo.astype(np.float16)
        s, b = scales.astype(np.float32)[:, :, None], biases.astype(np.float32)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint((v - b) / s)                      # float32, ties to even
    q = np.where(s == 0, np.float32(0), np.clip(r, np.float32(0), top))
    return q.astype(np.uint8).reshape(rows, cols), scales, biases


def pack(q: np.ndarray, bits: int) -> np.ndarray:
    """Pack integer codes (uint8 [rows, cols]) into uint32 words, lowest field first."""
    per = 32 // bits
    rows, cols = q.shape
    if cols % per != 0:
        raise ValueError("cols must fill whole words")
    fields = q.reshape(rows, cols // per, per).astype(np.uint32)
    words = np.zeros((rows, cols // per), dtype=np.uint32)
    for j in range(per):
        words |= fields[:, :, j] << np.uint32(bits * j)
    return words


def unpack(words: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of :func:`pack`: uint32 [rows, W] -> uint8 [rows, W * 32 / bits]."""
    per = 32 // bits
    mask = np.uint32(2 ** bits - 1)
    rows, nw = words.shape
    q = np.empty((rows, nw, per), dtype=np.uint8)
    for j in range(per):
        q[:, :, j] = (words >> np.uint32(bits * j)) & mask
    return q.reshape(rows, nw * per)


def quantize(w: np.ndarray, bits: int = 4, group: int = 64, param_dtype: str = "f16") -> QWeight:
    """Quantize a float32 matrix and pack it (the stored form of one linear layer)."""
    q, scales, biases = quantize_codes(w, bits, group, param_dtype)
    return QWeight(pack(q, bits), scales, biases, bits, group, param_dtype)


def dequantize(qw: QWeight) -> np.ndarray:
    """Dequantized weights ``scale * q + bias`` as float64 (exact: no rounding happens).

    fp16 parameters: every finite fp16 value is a multiple of 2^-24 below 2^16 in magnitude,
    and a code is below 2^8, so ``scale * q + bias`` is a multiple of 2^-24 below 2^25: at
    most 49 significant bits, which float64 (53) holds exactly.  bf16 parameters (8
    significant bits): ``scale * q`` has at most 16, and the sum is exact whenever the
    exponents of the scale and the bias differ by less than 37, which holds for any weights
    of one group (checked below rather than assumed).
    """
    q = unpack(qw.packed, qw.bits).astype(np.float64)
    s32, b32 = params_f32(qw)
    if qw.param_dtype == "bf16":
        both = (s32 != 0) & (b32 != 0)
        _, es = np.frexp(s32[both])
        _, eb = np.frexp(b32[both])
        if np.abs(eb - es).max(initial=0) >= 37:
            raise ValueError("bias and scale too far apart for an exact float64 dequantization")
    s = np.repeat(s32.astype(np.float64), qw.group, axis=1)
    b = np.repeat(b32.astype(np.float64), qw.group, axis=1)
    return s * q + b


def dequantize_f32(qw: QWeight) -> np.ndarray:
    """The dequantized weights rounded once to float32 (what an fp32 dequant stores)."""
    return dequantize(qw).astype(np.float32)
