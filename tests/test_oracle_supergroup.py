"""Pins for the oracle's mixed ternary / 4-bit super-group quantizer and GEMM (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import supergroup as sg

W = synth.Workload.TEST


def test_channel_allocation_one_four_bit_per_block():
    """rho = 1/4: in every block of 4 consecutive channels exactly one (the first) is 4-bit;
    period 1 is the all-4-bit limit (rho = 1)."""
    flags = [sg.is_four_bit(n, 4) for n in range(64)]
    for b in range(16):
        assert flags[4 * b:4 * b + 4] == [True, False, False, False]
    assert all(sg.is_four_bit(n, 1) for n in range(17))


def test_hand_example_scales_and_codes():
    """Worked by hand from the quantizer formulas of the EdgeRazor page (section 2.1):
    4-bit channel [0.7, -0.35, 0.05, 0, ...]: s = max|w|/7 = 0.1 -> fp16 0.0999755859375,
    codes rint(w/s) = [7, -4 (-3.5009 rounds to -4), 1 (0.50012 rounds to 1), 0 ...].
    Ternary channel with |w| summing to 1.6 over 16 inputs: mean 0.1, s = 0.2 ->
    fp16 0.199951171875; w = 0.1 -> 0.50012 -> 1; w = -0.09 -> -0.45 -> 0; 0.6 -> 3 -> 1."""
    w4 = np.zeros(16, np.float32)
    w4[:3] = [0.7, -0.35, 0.05]
    q4, s4 = sg.quantize_channel(w4, True)
    assert float(s4) == 0.0999755859375
    assert q4[:4].tolist() == [7, -4, 1, 0]
    wt = np.zeros(16, np.float32)
    wt[:4] = [0.1, -0.09, 0.6, -0.81]
    assert abs(np.abs(wt.astype(np.float64)).sum() - 1.6) < 1e-7
    qt, st = sg.quantize_channel(wt, False)
    assert float(st) == 0.199951171875
    assert qt[:4].tolist() == [1, 0, 1, -1]


def test_epsilon_floor():
    q, s = sg.quantize_channel(np.zeros(32, np.float32), False)
    assert float(s) == float(np.float16(1e-5)) and np.all(q == 0)
    q, s = sg.quantize_channel(np.full(32, 1e-7, np.float32), True)
    assert float(s) == float(np.float16(1e-5)) and np.all(q == 0)


@pytest.mark.parametrize("four_bit", [True, False])
def test_codes_are_nearest_clipped_level_brute_force(four_bit):
    qmax = 7 if four_bit else 1
    g = np.random.default_rng(9)
    for trial in range(40):
        w = (g.standard_normal(256) * 0.02).astype(np.float32)
        q, s = sg.quantize_channel(w, four_bit)
        S = Fraction(float(s))
        for i in range(256):
            Wv = Fraction(float(w[i]))
            dist = [abs(Wv - S * k) for k in range(-qmax, qmax + 1)]
            best = min(dist)
            cands = [k - qmax for k in range(2 * qmax + 1) if dist[k] == best]
            if int(q[i]) not in cands:
                frac = abs(Wv / S) - int(abs(Wv / S))
                assert abs(float(frac) - 0.5) < 1e-5


def test_pack_round_trip_and_layout():
    w = synth.normal_f32((64, 128), 0.02, W, 0, synth.Role.SUPERGROUP)
    Wq, codes = sg.quantize(w, 4)
    assert Wq.p4.shape == (16, 16) and Wq.p2.shape == (48, 8)
    assert np.array_equal(sg.codes_of(Wq), codes)
    # channel 0 is the first 4-bit row; channel 1 the first ternary row
    assert (int(Wq.p4[0, 0]) & 0xF) == int(codes[0, 0]) + 8
    assert (int(Wq.p2[0, 0]) & 0x3) == int(codes[1, 0]) + 1
    assert ((int(Wq.p2[0, 0]) >> 2) & 0x3) == int(codes[1, 1]) + 1
    assert (int(Wq.p2[1, 0]) & 0x3) == int(codes[2, 0]) + 1


def test_storage_of_the_benchmark_matrix():
    """3072 x 1024 at rho = 1/4: 768 x 128 nibble words + 2304 x 64 two-bit words +
    3072 fp16 scales = 989,184 bytes (about 2.19 bits per weight plus scales)."""
    w = np.zeros((3072, 1024), np.float32)
    Wq, _ = sg.quantize(w[:3072], 4)
    assert Wq.p4.nbytes + Wq.p2.nbytes + Wq.scales.nbytes == 989184


def test_gemm_factorization_equals_dequantized_matmul():
    """s * sum(q x) (scale applied once per channel) equals sum((s q) x) on the dequantized
    weights — the scale/integer decomposition of the EdgeRazor page."""
    w = synth.normal_f32((32, 256), 0.02, W, 1, synth.Role.SUPERGROUP)
    Wq, codes = sg.quantize(w, 4)
    x = synth.activations(5, 256, W)
    deq = codes.astype(np.float64) * Wq.scales.astype(np.float64)[:, None]
    np.testing.assert_allclose(sg.gemm(x, Wq), x.astype(np.float64) @ deq.T, rtol=1e-12, atol=1e-15)


def test_gemm_integer_case_exact():
    w = synth.normal_f32((16, 64), 0.02, W, 2, synth.Role.SUPERGROUP)
    Wq, codes = sg.quantize(w, 4)
    Wq.scales[:] = np.float16(1.0)
    x = np.random.default_rng(3).integers(-4, 5, size=(3, 64)).astype(np.float16)
    ref = x.astype(np.int64) @ codes.astype(np.int64).T
    assert np.array_equal(sg.gemm(x, Wq), ref.astype(np.float64))


# ---- weight-activation integer path (8-bit activations) -------------------------------------

def test_act8_on_grid_rows_are_exact():
    """Rows that are already on an 8-bit grid (x = k * 2^-5, max |k| = 127): the scale is
    max|x| / 127 = 2^-5 exactly and the codes are the integers k; the integer path then gives
    exactly the weight-only GEMM (its dequantized activations are x itself)."""
    g = np.random.default_rng(21)
    k = g.integers(-127, 128, size=(4, 128))
    k[:, 7] = [127, -127, 127, -127]
    x = (k * 2.0 ** -5).astype(np.float16)
    qx, sx = sg.quantize_activations(x)
    assert np.all(sx == np.float16(2.0 ** -5))
    assert np.array_equal(qx.astype(np.int64), k)
    w = synth.normal_f32((16, 128), 0.02, W, 3, synth.Role.SUPERGROUP)
    Wq, _ = sg.quantize(w, 4)
    assert np.array_equal(sg.gemm_a8(x, Wq), sg.gemm(x, Wq))


def test_act8_hand_example():
    """Worked by hand from the page's quantizer at n = 8.  fp16(2.54) = 2.5390625 is the
    row's largest magnitude; 2.5390625 / 127 = 0.0199926...; fp16 values in [2^-6, 2^-5) are
    spaced 2^-16, and 0.0199926 / 2^-16 = 1310.2, so s = 1310 * 2^-16 = 0.019989013671875.
    Codes: 2.5390625 / s = 127.02 -> 127; 1.0 / s = 50.03 -> 50; fp16(-0.03) =
    -1966 * 2^-16 = -0.029998779296875, / s = -1.5007 -> -2; fp16(0.01) = 1311 * 2^-17 =
    0.01000213623046875, / s = 0.5004 -> 1; zeros -> 0."""
    x = np.zeros((1, 16), np.float16)
    x[0, :4] = [2.54, 1.0, -0.03, 0.01]
    assert [float(v) for v in x[0, :4]] == [2.5390625, 1.0, -0.029998779296875, 0.01000213623046875]
    qx, sx = sg.quantize_activations(x)
    assert float(sx[0]) == 0.019989013671875
    assert qx[0, :4].tolist() == [127, 50, -2, 1] and np.all(qx[0, 4:] == 0)


def test_act8_codes_nearest_level_and_bounds():
    """Every code is the integer nearest to the exact quotient x / s (Fraction arithmetic,
    ties to even), clipped to -127..127, except where the float32 quotient sits within its
    rounding of a half-integer; the largest magnitude of a row maps to +-127; an all-zero row
    gets the epsilon scale and zero codes."""
    x = synth.activations(6, 256, W, 4)
    x[5] = 0
    qx, sx = sg.quantize_activations(x)
    assert float(sx[5]) == float(np.float16(1e-5)) and np.all(qx[5] == 0)
    for b in range(5):
        S = Fraction(float(sx[b]))
        i_max = int(np.argmax(np.abs(x[b].astype(np.float32))))
        assert abs(int(qx[b, i_max])) == 127
        for i in range(256):
            r = Fraction(float(x[b, i])) / S
            if int(qx[b, i]) != min(127, max(-127, round(r))):       # round(): ties to even
                frac = abs(r) - int(abs(r))
                assert abs(float(frac) - 0.5) < 2.0 ** -16


def test_act8_exact_ties_go_to_even():
    """Planted exact ties: with s = 2^-5 (each row holds 127 * 2^-5), x = (c + 1/2) 2^-5 is
    exactly halfway and must give the even neighbour: 0.5 -> 0, 1.5 -> 2, 2.5 -> 2, -0.5 -> 0,
    -1.5 -> -2, 126.5 -> 126, -126.5 -> -126; and 127.4 * 2^-5 (not a tie) -> 127."""
    halves = [0.5, 1.5, 2.5, -0.5, -1.5, 126.5, -126.5]
    x = np.zeros((1, 16), np.float16)
    x[0, 0] = 127 * 2.0 ** -5
    x[0, 1:1 + len(halves)] = [h * 2.0 ** -5 for h in halves]
    qx, sx = sg.quantize_activations(x)
    assert float(sx[0]) == 2.0 ** -5
    assert qx[0, 1:1 + len(halves)].tolist() == [0, 2, 2, 0, -2, 126, -126]


def test_gemm_a8_equals_dequantized_matmul():
    """The factorized form s_W s_X * (integer dot) equals the float64 matmul of the two
    dequantized operands (s_X[b] Q(X)[b, :]) . (s_W[n] Q(W)[n, :]): a transposed operand or a
    scale applied on the wrong axis fails here."""
    w = synth.normal_f32((32, 256), 0.02, W, 5, synth.Role.SUPERGROUP)
    Wq, codes = sg.quantize(w, 4)
    x = synth.activations(7, 256, W, 6)
    qx, sx = sg.quantize_activations(x)
    xd = qx.astype(np.float64) * sx.astype(np.float64)[:, None]
    wd = codes.astype(np.float64) * Wq.scales.astype(np.float64)[:, None]
    np.testing.assert_allclose(sg.gemm_a8(x, Wq), xd @ wd.T, rtol=1e-12, atol=1e-15)


def test_gemm_a8_integer_dot_brute_force():
    """The integer dot on a tiny case by explicit loops over the unpacked fields (Python
    integers), scales set to 1."""
    w = synth.normal_f32((8, 32), 0.02, W, 7, synth.Role.SUPERGROUP)
    Wq, _ = sg.quantize(w, 4)
    Wq.scales[:] = np.float16(1.0)
    x = synth.activations(2, 32, W, 8)
    qx, sx = sg.quantize_activations(x)
    c4 = sg.unpack_fields(Wq.p4, 4)
    c2 = sg.unpack_fields(Wq.p2, 2)
    y = sg.gemm_a8(x, Wq)
    for b in range(2):
        for n in range(8):
            row = c4[n // 4].astype(int) - 8 if n % 4 == 0 else c2[(n // 4) * 3 + n % 4 - 1].astype(int) - 1
            dot = sum(int(row[k]) * int(qx[b, k]) for k in range(32))
            assert y[b, n] == dot * float(sx[b])


def test_gemm_a8_within_the_activation_rounding_bound():
    """Against the weight-only GEMM on the same weights, the integer path differs only by the
    activation rounding: |y_a8 - y| <= sum_k |s_W q_W[n, k]| * s_X[b] / 2 (no clipping occurs:
    the largest |x| maps to 127 within rounding)."""
    w = synth.normal_f32((24, 512), 0.02, W, 9, synth.Role.SUPERGROUP)
    Wq, codes = sg.quantize(w, 4)
    x = synth.activations(5, 512, W, 10)
    qx, sx = sg.quantize_activations(x)
    bound = (np.abs(codes.astype(np.float64)) * Wq.scales.astype(np.float64)[:, None]).sum(1)[None, :] \
        * (sx.astype(np.float64)[:, None] / 2) * (1 + 1e-3)
    diff = np.abs(sg.gemm_a8(x, Wq) - sg.gemm(x, Wq))
    assert np.all(diff <= bound)
    assert diff.max() > 0
