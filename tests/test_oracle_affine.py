"""Pins for the oracle's affine quantizer, packing and dequantization (CPU only).

Each test checks the oracle against something other than itself: exact rational brute
force, an exhaustive enumeration, the pages' 0.0-error claim on grid-valued weights, the
pages' storage arithmetic, or a closed form.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import affine

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _groups(n_groups, seed, kind):
    g = np.random.default_rng(seed)
    if kind == "normal":
        return (g.standard_normal((n_groups, 64)) * 0.02).astype(np.float32)
    if kind == "outlier":
        v = (g.standard_normal((n_groups, 64)) * 0.02).astype(np.float32)
        v[:, 5] *= 40
        return v
    if kind == "uniform":
        return g.uniform(-3, 5, size=(n_groups, 64)).astype(np.float32)
    if kind == "tiny":
        return (g.standard_normal((n_groups, 64)) * 1e-6).astype(np.float32)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["normal", "outlier", "uniform", "tiny"])
@pytest.mark.parametrize("bits", [4, 8])
def test_codes_are_nearest_level_brute_force(kind, bits):
    """q is the grid level nearest to w (exact rationals), except at float32 near-ties."""
    w = _groups(60, 11 + bits, kind)
    q, s, b = affine.quantize_codes(w, bits, 64)
    top = 2 ** bits - 1
    near_ties = 0
    for r in range(w.shape[0]):
        S = Fraction(float(s[r, 0]))
        B = Fraction(float(b[r, 0]))
        assert S >= 0
        for i in range(64):
            W = Fraction(float(w[r, i]))
            if S == 0:
                assert q[r, i] == 0
                continue
            dist = [abs(W - (S * k + B)) for k in range(top + 1)]
            best = min(dist)
            cands = [k for k in range(top + 1) if dist[k] == best]
            if int(q[r, i]) in cands:
                continue
            # float32 rounding of (w - b) / s may pick the other neighbour only when the
            # exact quotient is within float32 error of a half-integer
            exact = (W - B) / S
            frac = exact - int(exact)
            assert abs(float(frac) - 0.5) < 1e-5, (r, i, float(exact), int(q[r, i]))
            near_ties += 1
    assert near_ties <= 2


@pytest.mark.parametrize("kind", ["normal", "outlier", "uniform"])
def test_error_within_half_scale(kind):
    """|w_hat - w| <= scale/2 for every element inside [bias, bias + 15 scale]; elements
    pushed outside the grid by the fp16 rounding of the parameters miss by at most that
    overshoot plus half a step."""
    w = _groups(2000, 5, kind)
    qw = affine.quantize(w, 4, 64)
    what = affine.dequantize(qw)
    s = qw.scales.astype(np.float64).repeat(64, axis=1)
    b = qw.biases.astype(np.float64).repeat(64, axis=1)
    w64 = w.astype(np.float64)
    over = np.maximum(0.0, np.maximum(b - w64, w64 - (b + 15 * s)))
    err = np.abs(what - w64)
    # the quotient is formed in float32: allow its relative rounding (2^-23) on top
    assert np.all(err <= s / 2 * (1 + 2.0 ** -20) + over)
    inside = over == 0
    assert np.mean(err[inside] <= s[inside] / 2 * (1 + 2.0 ** -20)) == 1.0


def test_on_grid_weights_round_trip_with_zero_error():
    """Weights that already lie on an int4 grid (each group using codes 0 and 15) are
    recovered bit-exactly — codes, scale and bias — and dequantize with error exactly 0.0,
    the claim of the bit-exact QAT port page."""
    g = np.random.default_rng(7)
    n = 4000
    q = g.integers(0, 16, size=(n, 64)).astype(np.uint8)
    q[:, 0] = 0
    q[:, 1] = 15
    g.shuffle(q, axis=1)
    s16 = np.abs(g.standard_normal(n) * 0.008 + 0.008).astype(np.float16)
    s16[s16 == 0] = np.float16(0.001)
    b16 = (-7.5 * s16.astype(np.float64) + g.standard_normal(n) * 0.002).astype(np.float16)
    exact = s16.astype(np.float64)[:, None] * q + b16.astype(np.float64)[:, None]
    w = exact.astype(np.float32)
    keep = np.all(w.astype(np.float64) == exact, axis=1)      # grid values exact in fp32
    assert keep.mean() > 0.99
    w, q, s16, b16 = w[keep], q[keep], s16[keep], b16[keep]
    qw = affine.quantize(w, 4, 64)
    assert np.array_equal(affine.unpack(qw.packed, 4), q)
    assert np.array_equal(qw.scales[:, 0].view(np.uint16), s16.view(np.uint16))
    assert np.array_equal(qw.biases[:, 0].view(np.uint16), b16.view(np.uint16))
    err = affine.dequantize(qw) - w.astype(np.float64)
    assert np.max(np.abs(err)) == 0.0


def test_degenerate_group_scale_zero():
    """All-equal group: scale 0, every code 0, dequantizes to the fp16-rounded value."""
    w = np.full((3, 128), 0.0123, dtype=np.float32)
    w[1, 64:] = -2.5
    w[2] = 0.0
    qw = affine.quantize(w, 4, 64)
    assert np.all(qw.scales == 0)
    assert np.all(affine.unpack(qw.packed, 4) == 0)
    assert np.array_equal(affine.dequantize(qw), w.astype(np.float16).astype(np.float64))


@pytest.mark.parametrize("bits", [4, 8])
def test_pack_exhaustive_positions_and_values(bits):
    per = 32 // bits
    top = 2 ** bits
    for pos in range(per):
        q = np.zeros((top, per), dtype=np.uint8)
        q[:, pos] = np.arange(top)
        words = affine.pack(q, bits)
        assert np.array_equal(words[:, 0], np.arange(top, dtype=np.uint64).astype(np.uint32)
                              << np.uint32(bits * pos))
        assert np.array_equal(affine.unpack(words, bits), q)


@pytest.mark.parametrize("bits", [4, 8])
def test_unpack_pack_identity_on_random_words(bits):
    words = synth.random_words((1000, 1000), synth.Workload.TEST, 0, synth.Role.WORDS)
    assert np.array_equal(affine.pack(affine.unpack(words, bits), bits), words)


def test_dequant_f32_is_single_rounding():
    """scale*q is exact in float32 (11-bit times 4-bit), so the float32 dequant equals
    one rounding of the exact value; spot-check against exact rationals."""
    w = _groups(50, 3, "uniform")
    qw = affine.quantize(w, 4, 64)
    d32 = affine.dequantize_f32(qw)
    q = affine.unpack(qw.packed, 4)
    for r in range(0, 50, 7):
        for i in range(0, 64, 5):
            ex = Fraction(float(qw.scales[r, 0])) * int(q[r, i]) + Fraction(float(qw.biases[r, 0]))
            assert Fraction(float(np.float32(float(ex)))) == Fraction(float(d32[r, i])) or \
                abs(Fraction(float(d32[r, i])) - ex) <= abs(ex) * Fraction(1, 2 ** 24)


def test_storage_arithmetic_matches_the_page():
    """The QAT-port page's storage count (a group of 32 weights: 16 bytes of int4 codes plus
    4 bytes of parameters), and the same count for the group-64 layout of the MoE model."""
    with open(os.path.join(GOLDEN, "storage_arithmetic.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        g = case["group"]
        w = np.random.default_rng(0).standard_normal((1, g)).astype(np.float32)
        qw = affine.quantize(w, 4, g)
        assert qw.packed.nbytes == case["code_bytes"]
        assert qw.scales.nbytes + qw.biases.nbytes == case["param_bytes"]
    m = gold["matrix_512x2048"]
    w = np.zeros((512, 2048), dtype=np.float32)
    qw = affine.quantize(w, 4, 64)
    assert qw.packed.nbytes + qw.scales.nbytes + qw.biases.nbytes == m["total_bytes"]


# ---- group 32 and bf16 parameters (the port page's own checkpoint format) --------------

def test_bf16_rounding_hand_values_and_library():
    """Round to nearest even, by hand: 1.0 -> 0x3F80; 1 + 2^-8 is halfway between 0x3F80 and
    0x3F81 -> even 0x3F80; 1 + 3 * 2^-8 halfway between 0x3F81 and 0x3F82 -> 0x3F82; just
    above the first tie -> 0x3F81; -2.5 -> 0xC020; and equal to torch's CPU conversion on a
    random sample that includes exact ties."""
    x = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, -2.5], np.float32)
    assert affine.bf16_bits(x).tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020]
    assert affine.bf16_to_f32(np.array([0x3F80, 0xC020], np.uint16)).tolist() == [1.0, -2.5]
    import torch
    g = np.random.default_rng(3)
    v = (g.standard_normal(20000) * 0.05).astype(np.float32)
    u = v.view(np.uint32).copy()
    u[::7] = (u[::7] & 0xFFFF0000) | 0x8000          # exact ties
    v = u.view(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(affine.bf16_bits(v), ref)


@pytest.mark.parametrize("param_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [4, 8])
def test_group32_codes_are_nearest_level_brute_force(bits, param_dtype):
    """Group 32, fp16 or bf16 parameters: each group has its own scale and bias, and every code
    is the grid level nearest to w (exact rationals), except at float32 near-ties."""
    g = np.random.default_rng(31 + bits)
    w = (g.standard_normal((20, 128)) * 0.02).astype(np.float32)
    q, s, b = affine.quantize_codes(w, bits, 32, param_dtype)
    assert s.shape == (20, 4)
    qw = affine.QWeight(affine.pack(q, bits), s, b, bits, 32, param_dtype)
    s32, b32 = affine.params_f32(qw)
    top = 2 ** bits - 1
    near = 0
    for r in range(20):
        for i in range(128):
            S, B = Fraction(float(s32[r, i // 32])), Fraction(float(b32[r, i // 32]))
            exact = (Fraction(float(w[r, i])) - B) / S       # nearest level: round the exact quotient
            if int(q[r, i]) != min(top, max(0, round(exact))):
                assert abs(float(exact - int(exact)) - 0.5) < 1e-5
                near += 1
    assert near <= 2
    # the stored parameters are the rounded min-max values of each 32-input group
    v = w.reshape(20, 4, 32)
    lo, hi = v.min(2), v.max(2)
    if param_dtype == "bf16":
        assert np.array_equal(b, affine.bf16_bits(lo))
        assert np.array_equal(s, affine.bf16_bits((hi - lo) / np.float32(top)))
    else:
        assert np.array_equal(b, lo.astype(np.float16))


def test_bf16_group32_on_grid_import_is_exact():
    """The port page's claim for QAT weights: integers plus bf16 parameters taken as given
    dequantize exactly to scale * q + bias (0.0 error), and quantizing those grid values
    again reproduces the same codes and parameters."""
    g = np.random.default_rng(8)
    n = 500
    q = g.integers(0, 16, size=(n, 32)).astype(np.uint8)
    q[:, 0], q[:, 1] = 0, 15
    s = affine.bf16_bits(np.abs(g.standard_normal(n) * 0.004 + 0.006).astype(np.float32))
    b = affine.bf16_bits((-7.5 * affine.bf16_to_f32(s) + g.standard_normal(n) * 0.001).astype(np.float32))
    exact = affine.bf16_to_f32(s).astype(np.float64)[:, None] * q + affine.bf16_to_f32(b).astype(np.float64)[:, None]
    w = exact.astype(np.float32)
    keep = np.all(w.astype(np.float64) == exact, axis=1)
    w, q, s, b = w[keep], q[keep], s[keep], b[keep]
    imported = affine.QWeight(affine.pack(q, 4), s[:, None], b[:, None], 4, 32, "bf16")
    assert np.max(np.abs(affine.dequantize(imported) - w.astype(np.float64))) == 0.0
    again = affine.quantize(w, 4, 32, "bf16")
    assert np.array_equal(affine.unpack(again.packed, 4), q)
    assert np.array_equal(again.scales[:, 0], s) and np.array_equal(again.biases[:, 0], b)
