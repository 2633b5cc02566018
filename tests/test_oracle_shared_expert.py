"""Pins for the oracle's shared expert and its sigmoid gate (CPU only).

The shared expert sits beside the 256-way switch MLP and is scaled by the 8-bit
``shared_expert_gate`` ("Edge0-35B-A3B Preview model repository guide", shared-expert
paragraph; "Recover-LoRA ..." section 1 keeps that gate at 8 bits); the recovery LoRA is a
parallel delta on each of its three projections, never merged ("Recover-LoRA ..." section
2; "Edge0 project review", highlight 3).  None of these tests calls the oracle's shared
expert code to make its expected value: each expected value is a hand-worked closed form,
or the same function written a different way (LoRA merged into the float64 weights, torch
modules), so that a gate/up swap inside the shared expert, a negated gate logit, a dropped
or misplaced LoRA delta all turn a test red.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import synth
from oracle import affine, moe

W = synth.Workload.TEST
R = synth.Role


def const_matrix(rows, cols, bias, bits=4):
    """Every code 0, scale 0, every group's bias `bias`: each row is the constant `bias`."""
    return affine.QWeight(np.zeros((rows, cols * bits // 32), np.uint32),
                          np.zeros((rows, cols // 64), np.float16),
                          np.full((rows, cols // 64), bias, np.float16), bits, 64)


def qmat(rows, cols, bits, role, index=0):
    return affine.quantize(synth.normal_f32((rows, cols), 0.02, W, 7, role, index), bits)


def hand_layer(gate_b=1 / 64, up_b=2 / 64, down_b=1 / 64, sg_b=1 / 64, loras=(None, None, None)):
    """H = SI = 64, one routed expert, every matrix constant: with x = ones(64) the shared
    gate and up projections are 64 * gate_b and 64 * up_b, and the shared down output is
    64 * down_b * h_s per output."""
    H = SI = 64
    z4 = const_matrix(H, H, 0.0)
    stack = lambda m: affine.QWeight(m.packed[None], m.scales[None], m.biases[None], 4, 64)
    return moe.MoELayer(router=const_matrix(1, H, 0.0, 8), shared_gate=const_matrix(1, H, sg_b, 8),
                        exp_gate=stack(z4), exp_up=stack(z4), exp_down=stack(z4),
                        sh_gate=const_matrix(SI, H, gate_b), sh_up=const_matrix(SI, H, up_b),
                        sh_down=const_matrix(H, SI, down_b), top_k=1,
                        lora_gate=loras[0], lora_up=loras[1], lora_down=loras[2])


def rank1(value_a, value_b, in_dim=64, out_dim=64, scale=2.0):
    """A rank-1 adapter with every A entry value_a and every B entry value_b (exact in fp16)."""
    return moe.Lora(np.full((1, 1, in_dim), value_a, np.float16),
                    np.full((1, out_dim, 1), value_b, np.float16), scale)


ONES = np.ones((1, 64), np.float16)


def test_hand_example_silu_on_gate_times_up():
    """gate = 1, up = 2 (x = ones, constant rows): h_s = silu(1) * 2 = 2 / (1 + e^-1) and the
    down rows (bias 1/64 over 64 inputs) return h_s itself.  A swap of gate and up would give
    silu(2) * 1 = 2 / (1 + e^-2) instead."""
    out = moe.shared_expert(ONES, hand_layer(), None)
    expect = 2.0 / (1.0 + math.exp(-1.0))          # 1.4621171572600098
    swapped = 2.0 / (1.0 + math.exp(-2.0))         # 1.7615941559557646
    np.testing.assert_allclose(out, np.full((1, 64), expect), rtol=1e-15)
    assert abs(expect - swapped) > 0.29


def test_hand_example_gate_sign():
    """Shared-gate row constant 1/64, x = ones: the logit is +1, so gamma = 1 / (1 + e^-1)
    > 1/2; with x = -ones the logit is -1 and gamma = 1 / (1 + e^1) < 1/2."""
    L = hand_layer()
    g_pos = moe.shared_gate_value(ONES, L)
    g_neg = moe.shared_gate_value(-ONES, L)
    assert g_pos[0] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15) and g_pos[0] > 0.5
    assert g_neg[0] == pytest.approx(1.0 / (1.0 + math.exp(1.0)), rel=1e-15) and g_neg[0] < 0.5


def test_hand_example_layer_adds_gamma_times_shared():
    """The routed expert is all zeros here, so y64 = gamma * shared = sigmoid(1) * silu(1) * 2."""
    out = moe.moe_layer(ONES, hand_layer())
    expect = (1.0 / (1.0 + math.exp(-1.0))) * 2.0 / (1.0 + math.exp(-1.0))
    np.testing.assert_allclose(out["y64"], np.full((1, 64), expect), rtol=1e-15)


def test_hand_example_each_lora_delta_on_its_own_projection():
    """Rank-1 adapters, scale 2, A entries 1/64 (so A x = 1 for x = ones):
    * on the gate only (B = 1/4): gate = 1 + 2 * 1/4 = 1.5, h_s = silu(1.5) * 2;
    * on the up only (B = 1/4):   up = 2 + 0.5 = 2.5,        h_s = silu(1) * 2.5;
    * on the down only (B = 1/2): its input is h_s (A h_s = h_s), so the delta is
      2 * 1/2 * h_s = h_s and the output doubles to 2 silu(1) * 2."""
    s = lambda z: z / (1.0 + math.exp(-z))
    gate_only = moe.shared_expert(ONES, hand_layer(loras=(rank1(1 / 64, 0.25), None, None)), None)
    up_only = moe.shared_expert(ONES, hand_layer(loras=(None, rank1(1 / 64, 0.25), None)), None)
    down_only = moe.shared_expert(ONES, hand_layer(loras=(None, None, rank1(1 / 64, 0.5))), None)
    np.testing.assert_allclose(gate_only, np.full((1, 64), s(1.5) * 2.0), rtol=1e-15)
    np.testing.assert_allclose(up_only, np.full((1, 64), s(1.0) * 2.5), rtol=1e-15)
    np.testing.assert_allclose(down_only, np.full((1, 64), 2.0 * s(1.0) * 2.0), rtol=1e-15)


def small_shared_layer(n_ad=3, rank=8, H=256, SI=128):
    L = lambda ra, rb, din, dout: moe.Lora(synth.normal_f16((n_ad, rank, din), 0.01, W, 7, ra),
                                           synth.normal_f16((n_ad, dout, rank), 0.01, W, 7, rb), 2.0)
    E = 2
    z = affine.QWeight(np.zeros((E, 64, H // 8), np.uint32), np.zeros((E, 64, H // 64), np.float16),
                       np.zeros((E, 64, H // 64), np.float16), 4, 64)
    zd = affine.QWeight(np.zeros((E, H, 8), np.uint32), np.zeros((E, H, 1), np.float16),
                        np.zeros((E, H, 1), np.float16), 4, 64)
    return moe.MoELayer(router=qmat(E, H, 8, R.ROUTER), shared_gate=qmat(1, H, 8, R.SHARED_GATE),
                        exp_gate=z, exp_up=z, exp_down=zd,
                        sh_gate=qmat(SI, H, 4, R.SH_GATE), sh_up=qmat(SI, H, 4, R.SH_UP),
                        sh_down=qmat(H, SI, 4, R.SH_DOWN), top_k=1,
                        lora_gate=L(R.LORA_A_GATE, R.LORA_B_GATE, H, SI),
                        lora_up=L(R.LORA_A_UP, R.LORA_B_UP, H, SI),
                        lora_down=L(R.LORA_A_DOWN, R.LORA_B_DOWN, SI, H))


def test_shared_expert_equals_torch_modules_with_merged_adapters():
    """Per token t with adapter a: the same function as three torch Linear modules whose
    float64 weights are the dequantized matrices with the adapter merged in,
    W' = W_hat + (alpha/r) B_a A_a, combined as down'(silu(gate'(x)) * up'(x))
    (torch's own silu)."""
    L = small_shared_layer()
    T = 9
    x = synth.activations(T, 256, W, 7)
    ad = (np.arange(T) % 3).astype(np.int32)
    got = moe.shared_expert(x, L, ad)

    def module(qw, lora, a):
        Wm = affine.dequantize(qw) + lora.scale * (lora.B[a].astype(np.float64) @ lora.A[a].astype(np.float64))
        m = torch.nn.Linear(Wm.shape[1], Wm.shape[0], bias=False, dtype=torch.float64)
        with torch.no_grad():
            m.weight.copy_(torch.from_numpy(Wm))
        return m

    for a in range(3):
        gate, up, down = (module(L.sh_gate, L.lora_gate, a), module(L.sh_up, L.lora_up, a),
                          module(L.sh_down, L.lora_down, a))
        rows = np.nonzero(ad == a)[0]
        xt = torch.from_numpy(x[rows].astype(np.float64))
        with torch.no_grad():
            ref = down(torch.nn.functional.silu(gate(xt)) * up(xt)).numpy()
        np.testing.assert_allclose(got[rows], ref, rtol=1e-11, atol=1e-14)


def test_shared_gate_is_sigmoid_of_positive_logit():
    """gamma = torch.sigmoid(x . w_sg) with w_sg the dequantized 8-bit row, and gamma > 1/2
    exactly where that dot product is positive (a negated logit flips every comparison)."""
    L = small_shared_layer()
    x = synth.activations(64, 256, W, 8)
    logit = x.astype(np.float64) @ affine.dequantize(L.shared_gate)[0]
    got = moe.shared_gate_value(x, L)
    np.testing.assert_allclose(got, torch.sigmoid(torch.from_numpy(logit)).numpy(), rtol=1e-14)
    np.testing.assert_allclose(got, scipy.special.expit(logit), rtol=1e-14)
    assert (logit > 0).any() and (logit < 0).any()
    assert np.array_equal(got > 0.5, logit > 0)


def test_only_down_adapter_adds_scaled_b_a_of_hidden():
    """Adapters with B = 0 on gate and up and a nonzero B on the down projection: the
    shared expert changes by exactly (alpha/r) B_d (A_d h_s) with h_s = silu(x Wg^T) * (x Wu^T)
    written out in torch from the dequantized matrices (not from x: the down adapter's input
    is the hidden activation)."""
    L = small_shared_layer(n_ad=1)
    zero = lambda l: moe.Lora(l.A, np.zeros_like(l.B), l.scale)
    Ld = moe.MoELayer(**{**L.__dict__, "lora_gate": zero(L.lora_gate), "lora_up": zero(L.lora_up)})
    Lbase = moe.MoELayer(**{**L.__dict__, "lora_gate": None, "lora_up": None, "lora_down": None})
    x = synth.activations(5, 256, W, 9)
    xt = torch.from_numpy(x.astype(np.float64))
    g = xt @ torch.from_numpy(affine.dequantize(L.sh_gate)).T
    u = xt @ torch.from_numpy(affine.dequantize(L.sh_up)).T
    hs = torch.nn.functional.silu(g) * u
    delta = 2.0 * (hs @ torch.from_numpy(L.lora_down.A[0].astype(np.float64)).T) \
        @ torch.from_numpy(L.lora_down.B[0].astype(np.float64)).T
    diff = moe.shared_expert(x, Ld, None) - moe.shared_expert(x, Lbase, None)
    np.testing.assert_allclose(diff, delta.numpy(), rtol=1e-9, atol=1e-15)
    assert np.max(np.abs(delta.numpy())) > 1e-6
