"""GPU parity of the layer under a given routing (moe_switchglu_int4_routed) against the
oracle's layer evaluated under the same selection (oracle.moe.moe_layer(idx=...)): the
routing the prerouter head predicts is the route itself ("Edge0 project review",
highlight 1).  The routing weights are the softmax of the router logits over the given set.
Decode sizes (fewer than 32 pairs) run the two-launch path, larger ones the token-sorted one.
"""
import numpy as np
import pytest
import torch

import synth
from layers import Shape, assert_close, build_layer, to_device
from oracle import moe

pytestmark = pytest.mark.gpu
DEV = "cuda"
W = synth.Workload.TEST


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.fixture(scope="module")
def q():
    import int4_group_quantized_amd as q
    assert torch.cuda.is_available()
    return q


def run_routed(q, Ld, x, route, ad=None):
    t, k = route.shape
    w = torch.full((t, k), float("nan"), dtype=torch.float32, device=DEV)
    y = q.moe_switchglu_int4_routed(Ld, dev(x), dev(route), None if ad is None else dev(ad), w_out=w)
    torch.cuda.synchronize()
    return y.cpu().numpy(), w.cpu().numpy()


def check(Lc, x, route, ad, y, w, residual=False):
    ref = moe.moe_layer(x, Lc, ad, idx=route)
    np.testing.assert_allclose(w, ref["w"], rtol=0, atol=1e-5)
    yref = ref["y64"]
    if residual:
        yref = x.astype(np.float64) + moe.to_f16(yref).astype(np.float64)
    return assert_close(y, yref, what="routed layer")


FULL = Shape(top_k=4, n_adapters=4)


@pytest.mark.parametrize("T,K,n_ad,skew", [(1, 4, 1, False), (3, 8, 4, False), (7, 4, 2, True)])
def test_routed_decode_full_shape(q, T, K, n_ad, skew):
    """Hidden 2048, 256 experts, inter 512, LoRA r16 on the shared expert: the two-launch
    decode path (T * K < 32 pairs)."""
    print(f"routed decode T={T} K={K}", flush=True)
    S = Shape(top_k=K, n_adapters=n_ad)
    route = synth.expert_choices(T, K, S.n_experts, W, 30 + T, 0)
    Lc = build_layer(W, 30 + T, S, skew=skew, only_experts=set(route.ravel().tolist()))
    x = synth.activations(T, S.hidden, W, 30 + T)
    ad = (np.arange(T) % n_ad).astype(np.int32)
    y, w = run_routed(q, to_device(Lc, S, DEV), x, route, ad)
    err, rel = check(Lc, x, route, ad, y, w)
    print(f"  max abs {err:.2e} rel L2 {rel:.2e}", flush=True)


@pytest.mark.parametrize("T", [8, 40])
def test_routed_prefill_path(q, T):
    """Token-sorted path (at least 32 pairs) with a given routing, ragged expert count."""
    print(f"routed prefill T={T}", flush=True)
    S = Shape(hidden=1024, inter=512, shared_inter=512, n_experts=37, top_k=4, rank=16, n_adapters=3)
    route = synth.expert_choices(T, S.top_k, S.n_experts, W, 40, T)
    Lc = build_layer(W, 40, S, skew=False)
    x = synth.activations(T, S.hidden, W, 40, T)
    ad = (np.arange(T) % 3).astype(np.int32)
    y, w = run_routed(q, to_device(Lc, S, DEV), x, route, ad)
    check(Lc, x, route, ad, y, w)


SMALL = Shape(hidden=512, inter=512, shared_inter=512, n_experts=16, top_k=4, rank=8, n_adapters=2)


def test_routed_small_residual_no_lora_and_repeated_expert(q):
    """Without adapters, with the residual, and a token whose routing names one expert twice
    (it counts twice in the weights and the sum)."""
    Lc = build_layer(W, 41, SMALL, with_lora=False)
    route = synth.expert_choices(5, 4, 16, W, 41, 0)
    route[2] = [9, 9, 3, 15]
    x = synth.activations(5, SMALL.hidden, W, 41)
    Ld = to_device(Lc, SMALL, DEV, add_residual=True)
    y, w = run_routed(q, Ld, x, route)
    check(Lc, x, route, None, y, w, residual=True)


def test_routed_out_of_range_entries_are_clamped(q):
    """Entries outside [0, E) read the first or last expert, never memory outside the stack:
    bit-identical to the clamped routing (decode and token-sorted paths)."""
    Lc = build_layer(W, 42, SMALL)
    Ld = to_device(Lc, SMALL, DEV)
    for T in (2, 12):
        route = synth.expert_choices(T, 4, 16, W, 42, T)
        bad = route.copy()
        bad[0, 0], bad[-1, 3] = -5, 1000
        good = np.clip(bad, 0, 15)
        x = synth.activations(T, SMALL.hidden, W, 42, T)
        yb, wb = run_routed(q, Ld, x, bad)
        yg, wg = run_routed(q, Ld, x, good)
        assert np.array_equal(yb, yg) and np.array_equal(wb, wg)


def test_routed_with_own_topk_matches_router_path(q):
    """Given the router's own top-K, the routed call reproduces the top-K call's routing
    weights and output (within the layer tolerance; the weights' sums are taken in another
    order)."""
    Lc = build_layer(W, 43, SMALL)
    Ld = to_device(Lc, SMALL, DEV)
    for T in (1, 6, 20):
        x = synth.activations(T, SMALL.hidden, W, 43, T)
        y0, idx, w0 = q.moe_switchglu_int4(Ld, dev(x), return_routing=True)
        torch.cuda.synchronize()
        y1, w1 = run_routed(q, Ld, x, idx.cpu().numpy())
        np.testing.assert_allclose(w1, w0.cpu().numpy(), rtol=0, atol=2e-7)
        assert_close(y1, y0.cpu().numpy().astype(np.float64), max_abs=2e-3, max_rel=2e-4,
                     what="routed vs router path")


def test_routed_is_deterministic(q):
    Lc = build_layer(W, 44, SMALL)
    Ld = to_device(Lc, SMALL, DEV)
    for T in (3, 30):
        route = synth.expert_choices(T, 4, 16, W, 44, T)
        x = synth.activations(T, SMALL.hidden, W, 44, T)
        a = run_routed(q, Ld, x, route)
        b = run_routed(q, Ld, x, route)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
