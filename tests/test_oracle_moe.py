"""Pins for the oracle's quantized linear, LoRA, router and MoE layer (CPU only).

The pages print no layer output, so the layer is pinned by closed forms, exact integer
arithmetic, textbook/library routines and invariants that any plausible slip (a dropped
term, a swapped operand, a wrong index) breaks.
"""
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

import synth
from oracle import affine, moe

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
W = synth.Workload.TEST


def qmat(rows, cols, bits=4, layer=0, role=synth.Role.DENSE, index=0, sigma=0.02):
    return affine.quantize(synth.normal_f32((rows, cols), sigma, W, layer, role, index), bits)


def stack(E, rows, cols, role, layer=0, bits=4):
    mats = [qmat(rows, cols, bits, layer, role, e) for e in range(E)]
    return affine.QWeight(np.stack([m.packed for m in mats]), np.stack([m.scales for m in mats]),
                          np.stack([m.biases for m in mats]), bits, 64)


def lora(n_ad, rank, in_dim, out_dim, roleA, roleB, layer=0, scale=2.0, zero_b=False):
    A = synth.normal_f16((n_ad, rank, in_dim), 0.01, W, layer, roleA)
    B = synth.normal_f16((n_ad, out_dim, rank), 0.01, W, layer, roleB)
    if zero_b:
        B = np.zeros_like(B)
    return moe.Lora(A, B, scale)


def small_layer(E=8, H=128, I=64, SI=64, K=2, layer=0, with_lora=True, n_ad=1):
    R = synth.Role
    return moe.MoELayer(
        router=qmat(E, H, 8, layer, R.ROUTER),
        shared_gate=qmat(1, H, 8, layer, R.SHARED_GATE),
        exp_gate=stack(E, I, H, R.EXP_GATE, layer), exp_up=stack(E, I, H, R.EXP_UP, layer),
        exp_down=stack(E, H, I, R.EXP_DOWN, layer),
        sh_gate=qmat(SI, H, 4, layer, R.SH_GATE), sh_up=qmat(SI, H, 4, layer, R.SH_UP),
        sh_down=qmat(H, SI, 4, layer, R.SH_DOWN), top_k=K,
        lora_gate=lora(n_ad, 4, H, SI, R.LORA_A_GATE, R.LORA_B_GATE, layer) if with_lora else None,
        lora_up=lora(n_ad, 4, H, SI, R.LORA_A_UP, R.LORA_B_UP, layer) if with_lora else None,
        lora_down=lora(n_ad, 4, SI, H, R.LORA_A_DOWN, R.LORA_B_DOWN, layer) if with_lora else None)


# --------------------------------------------------------------------------- qlinear

def test_qlinear_integer_special_case_is_exact_integer_matmul():
    """scale 1, bias 0, integer activations: the result is the integer matmul, exactly."""
    g = np.random.default_rng(1)
    N, K, T = 40, 256, 5
    q = g.integers(0, 16, size=(N, K)).astype(np.uint8)
    qw = affine.QWeight(affine.pack(q, 4), np.ones((N, K // 64), np.float16),
                        np.zeros((N, K // 64), np.float16), 4, 64)
    x = g.integers(-8, 9, size=(T, K)).astype(np.float16)
    ref = x.astype(np.int64) @ q.astype(np.int64).T
    assert np.array_equal(moe.qlinear(x, qw), ref.astype(np.float64))


def test_qlinear_zero_codes_closed_form():
    """All codes 0: y[t, n] = sum_g bias[n, g] * (sum of x over group g)."""
    g = np.random.default_rng(2)
    N, K = 16, 320
    biases = g.standard_normal((N, K // 64)).astype(np.float16)
    qw = affine.QWeight(np.zeros((N, K // 8), np.uint32), np.ones((N, K // 64), np.float16),
                        biases, 4, 64)
    x = g.standard_normal((3, K)).astype(np.float16)
    xs = x.astype(np.float64).reshape(3, K // 64, 64).sum(axis=2)
    ref = xs @ biases.astype(np.float64).T
    np.testing.assert_allclose(moe.qlinear(x, qw), ref, rtol=1e-13, atol=1e-13)


def test_qlinear_scale_multiplies_codes_not_bias():
    """Doubling every scale changes y by exactly sum_g scale*(sum q x): the bias part is
    untouched (catches a bias multiplied by the scale, or a zero-point subtraction)."""
    qw = qmat(24, 192, 4)
    x = synth.activations(3, 192, W)
    q = affine.unpack(qw.packed, 4).astype(np.float64)
    s = qw.scales.astype(np.float64).repeat(64, axis=1)
    qw2 = affine.QWeight(qw.packed, (qw.scales.astype(np.float32) * 2).astype(np.float16),
                         qw.biases, 4, 64)
    diff = moe.qlinear(x, qw2) - moe.qlinear(x, qw)
    np.testing.assert_allclose(diff, x.astype(np.float64) @ (s * q).T, rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------------- LoRA

def test_lora_zero_b_is_base():
    L = lora(1, 16, 128, 40, synth.Role.LORA_A_GATE, synth.Role.LORA_B_GATE, zero_b=True)
    qw = qmat(40, 128)
    x = synth.activations(4, 128, W)
    assert np.array_equal(moe.qlinear(x, qw, L), moe.qlinear(x, qw))


def test_lora_unmerged_equals_merged():
    """Unmerged delta == the same adapter merged into the float64 weights (the pages'
    'parallel delta, never merged' is a deployment choice, not a different function)."""
    L = lora(1, 16, 128, 40, synth.Role.LORA_A_GATE, synth.Role.LORA_B_GATE, scale=2.0)
    qw = qmat(40, 128)
    x = synth.activations(6, 128, W)
    merged = affine.dequantize(qw) + 2.0 * (L.B[0].astype(np.float64) @ L.A[0].astype(np.float64))
    ref = x.astype(np.float64) @ merged.T
    np.testing.assert_allclose(moe.qlinear(x, qw, L), ref, rtol=1e-12, atol=1e-13)


def test_lora_adapter_index_selects_per_token_and_commutes_with_permutation():
    n_ad = 4
    L = lora(n_ad, 16, 128, 40, synth.Role.LORA_A_UP, synth.Role.LORA_B_UP)
    qw = qmat(40, 128)
    x = synth.activations(16, 128, W)
    ad = synth.adapter_index(16, 4)
    y = moe.qlinear(x, qw, L, ad)
    for a in range(n_ad):
        single = moe.Lora(L.A[a:a + 1], L.B[a:a + 1], L.scale)
        rows = np.nonzero(ad == a)[0]
        np.testing.assert_allclose(y[rows], moe.qlinear(x[rows], qw, single), rtol=0, atol=0)
    perm = np.random.default_rng(3).permutation(16)
    np.testing.assert_array_equal(moe.qlinear(x[perm], qw, L, ad[perm]), y[perm])


# --------------------------------------------------------------------------- router

def test_topk_matches_stable_argsort():
    logits = np.random.default_rng(4).standard_normal((50, 256))
    idx, w = moe.topk(logits, 8)
    ref = np.argsort(-logits, axis=1, kind="stable")[:, :8]
    assert np.array_equal(idx, ref)


def test_topk_exact_ties_prefer_lower_index():
    logits = np.zeros((3, 16))
    logits[0, [3, 9, 12]] = 1.0
    logits[1, :] = 0.5
    logits[2, [15, 2]] = 2.0
    logits[2, [7, 5]] = 1.5
    idx, w = moe.topk(logits, 3)
    assert idx[0].tolist() == [3, 9, 12]
    assert idx[1].tolist() == [0, 1, 2]
    assert idx[2].tolist() == [2, 15, 5]
    np.testing.assert_allclose(w[1], [1 / 3] * 3, rtol=0, atol=1e-15)


def test_topk_full_k_is_softmax_and_weights_sum_to_one():
    logits = np.random.default_rng(5).standard_normal((20, 32)) * 3
    idx, w = moe.topk(logits, 32)
    full = scipy.special.softmax(logits, axis=1)
    np.testing.assert_allclose(np.take_along_axis(full, idx, 1), w, rtol=1e-13)
    idx4, w4 = moe.topk(logits, 4)
    np.testing.assert_allclose(w4.sum(axis=1), 1.0, rtol=0, atol=4e-16)
    p = np.take_along_axis(full, idx4, 1)
    np.testing.assert_allclose(w4, p / p.sum(axis=1, keepdims=True), rtol=1e-13)


def test_router_bias_shifts_selection():
    """A +2.0 bias on experts 0..15 (the skewed workload) moves most picks onto them."""
    L = small_layer(E=64, H=128, K=4)
    x = synth.activations(64, 128, W)
    bias = np.zeros(64, np.float32)
    bias[:16] = 2.0
    plain = moe.router_logits(x, L.router)
    skew = moe.router_logits(x, L.router, bias)
    np.testing.assert_allclose(skew - plain, np.broadcast_to(bias, plain.shape), atol=1e-15)
    idx, _ = moe.topk(skew, 4)
    assert np.mean(idx < 16) > 0.8


# --------------------------------------------------------------------------- layer

def test_silu_sigmoid_match_library():
    z = np.linspace(-30, 30, 1001)
    zt = torch.from_numpy(z)
    np.testing.assert_allclose(moe.silu(z), torch.nn.functional.silu(zt).numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(moe.sigmoid(z), torch.sigmoid(zt).numpy(), rtol=1e-14, atol=1e-300)


def test_single_expert_top1_is_dense_swiglu_plus_gated_shared():
    L = small_layer(E=1, K=1)
    x = synth.activations(5, 128, W)
    out = moe.moe_layer(x, L)
    dense = moe.expert_mlp(x, L.exp_gate.expert(0), L.exp_up.expert(0), L.exp_down.expert(0))
    assert np.all(out["idx"] == 0) and np.all(out["w"] == 1.0)
    np.testing.assert_allclose(out["routed"], dense, rtol=0, atol=0)
    np.testing.assert_allclose(out["y64"], dense + out["gamma"][:, None] * out["shared"], rtol=1e-15)


def test_identical_experts_make_routing_irrelevant():
    """All experts equal: the routed output is that expert's output for any selection,
    because the renormalized weights sum to one."""
    base = small_layer(E=8, K=3)
    one = lambda s: affine.QWeight(np.repeat(s.packed[:1], 8, 0), np.repeat(s.scales[:1], 8, 0),
                                   np.repeat(s.biases[:1], 8, 0), 4, 64)
    L = moe.MoELayer(base.router, base.shared_gate, one(base.exp_gate), one(base.exp_up),
                     one(base.exp_down), base.sh_gate, base.sh_up, base.sh_down, 3)
    x = synth.activations(7, 128, W)
    out = moe.moe_layer(x, L)
    dense = moe.expert_mlp(x, L.exp_gate.expert(0), L.exp_up.expert(0), L.exp_down.expert(0))
    np.testing.assert_allclose(out["routed"], dense, rtol=1e-12, atol=1e-14)


def test_unselected_experts_contribute_nothing():
    L = small_layer(E=8, K=2)
    x = synth.activations(3, 128, W)
    out = moe.moe_layer(x, L)
    unused = sorted(set(range(8)) - set(out["idx"].ravel().tolist()))
    assert unused
    e = unused[0]
    scales = L.exp_down.scales.copy()
    scales[e] = np.float16(100.0)
    L2 = moe.MoELayer(**{**L.__dict__, "exp_down": affine.QWeight(L.exp_down.packed, scales,
                                                                   L.exp_down.biases, 4, 64)})
    assert np.array_equal(moe.moe_layer(x, L2)["y64"], out["y64"])


def test_routed_sum_is_weighted_in_selection_order():
    """Each token's routed output is sum_k w_k * expert_{idx_k}(x): recomputed per pair."""
    L = small_layer(E=8, K=3)
    x = synth.activations(4, 128, W)
    out = moe.moe_layer(x, L)
    for t in range(4):
        acc = np.zeros(128)
        for k in range(3):
            e = out["idx"][t, k]
            acc += out["w"][t, k] * moe.expert_mlp(x[t:t + 1], L.exp_gate.expert(e),
                                                   L.exp_up.expert(e), L.exp_down.expert(e))[0]
        np.testing.assert_allclose(out["routed"][t], acc, rtol=1e-12, atol=1e-15)


def test_zero_shared_gate_weights_give_half():
    L = small_layer()
    z = affine.QWeight(np.zeros_like(L.shared_gate.packed), np.zeros_like(L.shared_gate.scales),
                       np.zeros_like(L.shared_gate.biases), 8, 64)
    L2 = moe.MoELayer(**{**L.__dict__, "shared_gate": z})
    out = moe.moe_layer(synth.activations(3, 128, W), L2)
    assert np.all(out["gamma"] == 0.5)


def test_gate_goes_through_silu_and_up_does_not():
    """Gate rows with every code 0 and every bias b make each gate output b * (sum of x);
    with x = 1 that is 128 * fp16(20/128) = 20 exactly, so h = silu(20) * up."""
    H, I = 128, 64
    x = np.ones((1, H), np.float16)
    gate = affine.QWeight(np.zeros((I, H // 8), np.uint32), np.zeros((I, H // 64), np.float16),
                          np.full((I, H // 64), 20.0 / H, np.float16), 4, 64)
    assert np.all(moe.linear(x, gate) == 20.0)
    up = qmat(I, H, 4, 0, synth.Role.EXP_UP)
    down = qmat(H, I, 4, 0, synth.Role.EXP_DOWN)
    gval = moe.linear(x, gate)[0, 0]
    h = (gval / (1 + np.exp(-gval))) * moe.linear(x, up)
    np.testing.assert_allclose(moe.expert_mlp(x, gate, up, down), moe.linear(h, down), rtol=1e-14)


def test_gate_up_swap_changes_output_by_about_100_percent():
    """The streaming-layer docs quoted by the Edge0 review: swapping gate and up moves the
    relative L2 error to ~100 %."""
    with open(os.path.join(GOLDEN, "pages_claims.json")) as f:
        claim = json.load(f)["swiglu_swap_rel_l2"]
    H, I = synth.HIDDEN, synth.INTER                     # the model's shapes
    gate = qmat(I, H, 4, 0, synth.Role.EXP_GATE)
    up = qmat(I, H, 4, 0, synth.Role.EXP_UP)
    down = qmat(H, I, 4, 0, synth.Role.EXP_DOWN)
    x = synth.activations(32, H, W)
    good = moe.expert_mlp(x, gate, up, down)
    bad = moe.expert_mlp(x, up, gate, down)
    rel = np.linalg.norm(bad - good) / np.linalg.norm(good)
    assert claim["low"] <= rel <= claim["high"], rel


def test_stack_residual_identity_when_layer_output_is_zero():
    """Zero down-projections and zero shared down: y = 0, so x_{l+1} = x_l."""
    L = small_layer(with_lora=False)
    zd = affine.QWeight(np.zeros_like(L.exp_down.packed), np.zeros_like(L.exp_down.scales),
                        np.zeros_like(L.exp_down.biases), 4, 64)
    zs = affine.QWeight(np.zeros_like(L.sh_down.packed), np.zeros_like(L.sh_down.scales),
                        np.zeros_like(L.sh_down.biases), 4, 64)
    L2 = moe.MoELayer(**{**L.__dict__, "exp_down": zd, "sh_down": zs})
    x = synth.activations(3, 128, W)
    xs = moe.moe_stack(x, [L2, L2])
    assert np.array_equal(xs[2], x)


def test_residual_rounds_once():
    a = np.array([[1.0, 2048.0, -0.5]], np.float16)
    b = np.array([[2.0 ** -11, 1.0, 0.25]], np.float16)
    # 1 + 2^-11 is a tie -> even (1.0); 2048 + 1 is a tie -> even (2048); exact otherwise
    assert moe.residual(a, b).tolist() == [[1.0, 2048.0, -0.25]]


def test_given_selection_equal_to_topk_reproduces_topk_weights():
    """moe_layer(idx=...) with the router's own top-K as the given selection reproduces
    topk's indices, weights and output exactly; another given set gets the full softmax
    (scipy) restricted to that set and renormalized."""
    L = small_layer(E=8, K=3)
    x = synth.activations(6, 128, W)
    own = moe.moe_layer(x, L)
    given = moe.moe_layer(x, L, idx=own["idx"])
    assert np.array_equal(given["idx"], own["idx"])
    assert np.array_equal(given["w"], own["w"])
    assert np.array_equal(given["y64"], own["y64"])
    alt = np.array([[7, 0, 3]] * 6, np.int32)
    out = moe.moe_layer(x, L, idx=alt)
    p = scipy.special.softmax(out["logits"], axis=1)[:, [7, 0, 3]]
    np.testing.assert_allclose(out["w"], p / p.sum(axis=1, keepdims=True), rtol=1e-13)
    for t in range(6):
        acc = sum(out["w"][t, k] * moe.expert_mlp(x[t:t + 1], L.exp_gate.expert(e), L.exp_up.expert(e),
                                                   L.exp_down.expert(e))[0] for k, e in enumerate([7, 0, 3]))
        np.testing.assert_allclose(out["routed"][t], acc, rtol=1e-12, atol=1e-15)
