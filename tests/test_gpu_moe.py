"""GPU parity of the MoE SwitchGLU layer (moe_switchglu_int4) against the oracle.

Routing indices must equal the oracle's; the only accepted difference is a token whose
oracle logits have the K-th and (K+1)-th expert within TAU of each other (the device sums
the router in float32, the oracle in float64), and then the device must have picked the
oracle's own alternative and match the oracle's output under that alternative.
"""
import numpy as np
import pytest
import torch

import synth
from layers import Shape, assert_close, build_layer, routed_experts, to_device
from oracle import moe

pytestmark = pytest.mark.gpu
TAU = 1e-4
DEV = "cuda"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.fixture(scope="module")
def q():
    import int4_group_quantized_amd as q
    assert torch.cuda.is_available()
    return q


def run_device(q, Lc, S, x, ad=None, residual=False):
    Ld = to_device(Lc, S, DEV, add_residual=residual)
    y, idx, w = q.moe_switchglu_int4(Ld, dev(x), None if ad is None else dev(ad), return_routing=True)
    torch.cuda.synchronize()
    return y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def check_layer(Lc, x, ad, y, idx, w, residual=False, tau=TAU):
    """Compare one layer's device outputs with the oracle; returns (max abs, rel L2, #alt)."""
    ref = moe.moe_layer(x, Lc, ad)
    ridx = ref["idx"]
    K = ridx.shape[1]
    yref = ref["y64"].copy()
    n_alt = 0
    for t in range(x.shape[0]):
        if np.array_equal(idx[t], ridx[t]):
            np.testing.assert_allclose(w[t], ref["w"][t], rtol=0, atol=1e-5)
            continue
        order = np.argsort(-ref["logits"][t], kind="stable")
        ell = ref["logits"][t][order]
        if set(idx[t].tolist()) == set(ridx[t].tolist()):
            # same set, different order: only among near-equal selected logits
            assert np.min(np.diff(ell[:K]) * -1) < tau, (t, idx[t], ridx[t])
            continue
        gap = ell[K - 1] - ell[K]
        assert gap < tau, f"token {t}: device picked {idx[t]}, oracle {ridx[t]}, gap {gap}"
        alt = order[:K].copy()
        alt[K - 1] = order[K]
        assert set(idx[t].tolist()) == set(alt.tolist())
        yref[t] = moe.moe_layer(x[t:t + 1], Lc, None if ad is None else ad[t:t + 1],
                                idx=alt[None, :])["y64"][0]
        n_alt += 1
    if residual:
        yref = x.astype(np.float64) + moe.to_f16(yref).astype(np.float64)
    err, rel = assert_close(y, yref, what="moe layer")
    return err, rel, n_alt


SMALL = Shape(hidden=512, inter=512, shared_inter=512, n_experts=8, top_k=2, rank=8, n_adapters=2)


@pytest.mark.parametrize("T", [1, 5, 37])
def test_small_layer(q, T):
    print(f"small layer T={T}", flush=True)
    Lc = build_layer(synth.Workload.TEST, 10, SMALL)
    x = synth.activations(T, SMALL.hidden, synth.Workload.TEST, 10, T)
    ad = (np.arange(T) % 2).astype(np.int32)
    y, idx, w = run_device(q, Lc, SMALL, x, ad)
    check_layer(Lc, x, ad, y, idx, w)


def test_small_layer_without_lora_and_with_residual(q):
    Lc = build_layer(synth.Workload.TEST, 11, SMALL, with_lora=False)
    x = synth.activations(9, SMALL.hidden, synth.Workload.TEST, 11)
    y, idx, w = run_device(q, Lc, SMALL, x, None, residual=True)
    check_layer(Lc, x, None, y, idx, w, residual=True)


def test_wider_shapes_many_tiles(q):
    S = Shape(hidden=1024, inter=1536, shared_inter=512, n_experts=64, top_k=6, rank=16, n_adapters=3)
    Lc = build_layer(synth.Workload.TEST, 12, S)
    x = synth.activations(19, S.hidden, synth.Workload.TEST, 12)
    ad = (np.arange(19) % 3).astype(np.int32)
    y, idx, w = run_device(q, Lc, S, x, ad)
    check_layer(Lc, x, ad, y, idx, w)


@pytest.mark.parametrize("T", [33, 150])
def test_prefill_ragged_shapes(q, T):
    """Token-sorted path with ragged sizes: 37 experts (router rows and the logits stride
    are not a multiple of 64), top-3, hidden 1024, a wider shared expert, 3 adapters."""
    S = Shape(hidden=1024, inter=512, shared_inter=1024, n_experts=37, top_k=3, rank=16, n_adapters=3)
    Lc = build_layer(synth.Workload.TEST, 14, S)
    x = synth.activations(T, S.hidden, synth.Workload.TEST, 14, T)
    ad = (np.arange(T) % 3).astype(np.int32)
    y, idx, w = run_device(q, Lc, S, x, ad)
    err, rel, n_alt = check_layer(Lc, x, ad, y, idx, w)
    print(f"ragged T={T}: max abs {err:.2e} rel L2 {rel:.2e} alternatives {n_alt}", flush=True)


def test_prefill_wide_inter_many_items(q):
    """An expert with more than 64 tokens (several work items) and a 1536-wide inter."""
    S = Shape(hidden=1024, inter=1536, shared_inter=512, n_experts=4, top_k=2, rank=16, n_adapters=2)
    Lc = build_layer(synth.Workload.TEST, 15, S)
    x = synth.activations(200, S.hidden, synth.Workload.TEST, 15)
    ad = (np.arange(200) % 2).astype(np.int32)
    y, idx, w = run_device(q, Lc, S, x, ad)
    assert np.bincount(idx.ravel(), minlength=4).max() > 64
    check_layer(Lc, x, ad, y, idx, w)


# Few pairs (at most 256, at most 256 experts): the grouped GEMM blocks form their work items
# themselves.  37 experts (grid items past the last item), 256 pairs (the limit) over 64
# experts, and experts split over two 64-pair items.
@pytest.mark.parametrize("T,S,seed", [
    (16, Shape(hidden=1024, inter=512, shared_inter=512, n_experts=37, top_k=4, rank=16, n_adapters=2), 20),
    (32, Shape(hidden=512, inter=512, shared_inter=512, n_experts=64, top_k=8, rank=8, n_adapters=2), 21),
    (128, Shape(hidden=512, inter=512, shared_inter=512, n_experts=4, top_k=2, rank=8, n_adapters=2), 20),
], ids=["37-experts", "256-pairs", "two-items"])
def test_prefill_items_formed_in_block(q, T, S, seed):
    print(f"items in block T={T} E={S.n_experts} K={S.top_k}", flush=True)
    assert T * S.top_k <= 256
    Lc = build_layer(synth.Workload.TEST, seed, S)
    x = synth.activations(T, S.hidden, synth.Workload.TEST, seed)
    ad = (np.arange(T) % 2).astype(np.int32)
    y, idx, w = run_device(q, Lc, S, x, ad)
    if T == 128:
        assert np.bincount(idx.ravel(), minlength=S.n_experts).max() > 64
    check_layer(Lc, x, ad, y, idx, w)


@pytest.mark.parametrize("T", [64, 100, 200])
def test_prefill_inter_1024(q, T):
    """Routed and shared inner size 1024: 16-pair work items at 64 and 100 tokens (the down
    GEMMs with activations resident over all 1024 inputs), 32-pair items at 200 tokens."""
    S = Shape(hidden=1024, inter=1024, shared_inter=1024, n_experts=64, top_k=4, rank=16, n_adapters=2)
    Lc = build_layer(synth.Workload.TEST, 17, S)
    x = synth.activations(T, S.hidden, synth.Workload.TEST, 17, T)
    ad = (np.arange(T) % 2).astype(np.int32)
    y, idx, w = run_device(q, Lc, S, x, ad)
    err, rel, n_alt = check_layer(Lc, x, ad, y, idx, w)
    print(f"inter 1024 T={T}: max abs {err:.2e} rel L2 {rel:.2e} alternatives {n_alt}", flush=True)


WIDE_64 = Shape(hidden=2048, inter=512, shared_inter=512, n_experts=16, top_k=2, rank=16, n_adapters=2)
DEEP_64 = Shape(hidden=512, inter=2048, shared_inter=2048, n_experts=8, top_k=2, rank=16, n_adapters=2)


@pytest.mark.parametrize("T,S", [(256, SMALL), (300, WIDE_64), (2048, WIDE_64), (300, DEEP_64)],
                         ids=["256-small", "300-wide", "2048-wide", "300-deep"])
def test_prefill_64_pair_items(q, T, S):
    """Many pairs per expert (above 32 on average): 64-pair work items, four token tiles per
    GEMM block, including the short last items of an expert; hidden 512 (short steps),
    hidden 2048 (the full step count; at 2048 tokens the x side runs unsplit), and inner
    size 2048 (the down GEMMs over 2048 inputs)."""
    assert T * S.top_k > 32 * S.n_experts
    Lc = build_layer(synth.Workload.TEST, 18, S)
    x = synth.activations(T, S.hidden, synth.Workload.TEST, 18, T)
    ad = (np.arange(T) % 2).astype(np.int32)
    y, idx, w = run_device(q, Lc, S, x, ad)
    err, rel, n_alt = check_layer(Lc, x, ad, y, idx, w)
    print(f"64-pair items T={T}: max abs {err:.2e} rel L2 {rel:.2e} alternatives {n_alt}", flush=True)


SORT_16 = Shape(hidden=512, inter=512, shared_inter=512, n_experts=16, top_k=4, rank=8, n_adapters=2)


@pytest.mark.parametrize("T,S,n_check", [(1500, SMALL, None), (16500, SORT_16, 300)],
                         ids=["3000-pairs", "66000-pairs"])
def test_prefill_multi_block_sort(q, T, S, n_check):
    """More than 2048 (token, expert) pairs: the expert sort runs as per-segment counts and a
    placement pass over segments of 1024-pair chunks; 3000 pairs end in a ragged chunk,
    66000 pairs make each block place two chunks.  The layer is per token, so at 16500 tokens
    the oracle checks a seeded sample of the device's rows (first and last tokens included)."""
    Lc = build_layer(synth.Workload.TEST, 19, S)
    x = synth.activations(T, S.hidden, synth.Workload.TEST, 19, T)
    ad = (np.arange(T) % 2).astype(np.int32)
    y, idx, w = run_device(q, Lc, S, x, ad)
    rows = np.arange(T)
    if n_check is not None:
        rng = np.random.default_rng(T)
        rows = np.unique(np.concatenate([[0, T - 1], rng.choice(T, n_check, replace=False)]))
    err, rel, n_alt = check_layer(Lc, x[rows], ad[rows], y[rows], idx[rows], w[rows])
    print(f"multi-block sort T={T}: max abs {err:.2e} rel L2 {rel:.2e} alternatives {n_alt} "
          f"({len(rows)} rows)", flush=True)


def test_decode_one_token_full_shape(q):
    """The single-token decode workload: hidden 2048, 256 experts, top-4, shared expert with
    8-bit gate, LoRA rank 16 alpha 32 on the shared projections."""
    S = Shape(top_k=4)
    wl = synth.Workload.MOE_DECODE
    for layer in range(2):
        for i in range(4):
            x = synth.activations(1, S.hidden, wl, layer, i)
            Lc = build_layer(wl, layer, S, only_experts=routed_experts(x, wl, layer, S))
            y, idx, w = run_device(q, Lc, S, x)
            err, rel, _ = check_layer(Lc, x, None, y, idx, w)
            print(f"decode layer {layer} token {i}: max abs {err:.2e} rel L2 {rel:.2e}", flush=True)


def test_decode_seven_tokens_full_shape_with_adapters(q):
    """Seven tokens in one decode call (28 routed pairs, the largest batch of the decode
    path at top-4) at the full shape, four LoRA adapter sets chosen per token."""
    S = Shape(top_k=4, n_adapters=4)
    wl = synth.Workload.MOE_DECODE
    x = synth.activations(7, S.hidden, wl, 2, 0)
    Lc = build_layer(wl, 2, S, only_experts=routed_experts(x, wl, 2, S))
    ad = np.array([0, 1, 2, 3, 3, 1, 0], np.int32)
    y, idx, w = run_device(q, Lc, S, x, ad)
    err, rel, n_alt = check_layer(Lc, x, ad, y, idx, w)
    print(f"decode 7 tokens: max abs {err:.2e} rel L2 {rel:.2e} alternatives {n_alt}", flush=True)


@pytest.fixture(scope="module")
def prefill_layer():
    return build_layer(synth.Workload.MOE_PREFILL, 0, Shape(top_k=4))


@pytest.mark.parametrize("skew", [False, True])
def test_prefill_512_tokens(q, prefill_layer, skew):
    S = Shape(top_k=4)
    Lc = prefill_layer
    if skew:
        bias = np.zeros(256, np.float32)
        bias[:16] = 2.0
        Lc = moe.MoELayer(**{**Lc.__dict__, "router_bias": bias})
    x = synth.activations(512, S.hidden, synth.Workload.MOE_PREFILL, 0, int(skew))
    y, idx, w = run_device(q, Lc, S, x)
    err, rel, n_alt = check_layer(Lc, x, None, y, idx, w)
    print(f"prefill skew={skew}: max abs {err:.2e} rel L2 {rel:.2e} alternatives {n_alt}", flush=True)
    if skew:
        assert np.mean(idx < 16) > 0.5


@pytest.mark.parametrize("T", [2048, 8192])
def test_prefill_sweep_sizes_sampled(q, prefill_layer, T):
    """The prefill sweep's token counts at the full layer shape (hidden 2048, 256 experts,
    top-4, shared expert, LoRA): at 2048 tokens the x side runs unsplit and 32-pair items,
    at 8192 tokens 64-pair items (four-tile fp16-weight GEMMs, the resident down with four
    tiles), the two-pass sort and the many-token per-token and combine kernels.  The layer
    is per token, so the oracle checks a seeded sample of the device's rows (first and last
    tokens included)."""
    S = Shape(top_k=4)
    x = synth.activations(T, S.hidden, synth.Workload.MOE_PREFILL, 0, 10 + T)
    y, idx, w = run_device(q, prefill_layer, S, x)
    rng = np.random.default_rng(T + 1)
    rows = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 150, replace=False)]))
    err, rel, n_alt = check_layer(prefill_layer, x[rows], None, y[rows], idx[rows], w[rows])
    print(f"prefill sweep T={T}: max abs {err:.2e} rel L2 {rel:.2e} alternatives {n_alt} "
          f"({len(rows)} rows)", flush=True)


def test_multi_tenant_stack_teacher_forced(q):
    """Three stacked layers of the multi-tenant workload (16 tokens, top-8, 4 adapter sets,
    adapter = token // 4), each compared with the oracle on the oracle's own input."""
    S = Shape(top_k=8, n_adapters=4)
    wl = synth.Workload.MOE_STACK
    x = synth.activations(16, S.hidden, wl, 0)
    ad = synth.adapter_index(16, 4)
    for layer in range(3):
        Lc = build_layer(wl, layer, S, only_experts=routed_experts(x, wl, layer, S))
        y, idx, w = run_device(q, Lc, S, x, ad, residual=True)
        check_layer(Lc, x, ad, y, idx, w, residual=True)
        x = moe.residual(x, moe.moe_layer(x, Lc, ad)["y"])


def test_decode_path_top8_adapters(q):
    """Few tokens at top-8 (under the token-sorted path's threshold): the decode kernels'
    eight-expert case with per-token adapters."""
    S = Shape(top_k=8, n_adapters=4)
    wl = synth.Workload.MOE_STACK
    x = synth.activations(3, S.hidden, wl, 5)
    ad = np.array([3, 0, 2], np.int32)
    Lc = build_layer(wl, 5, S, only_experts=routed_experts(x, wl, 5, S))
    y, idx, w = run_device(q, Lc, S, x, ad, residual=True)
    check_layer(Lc, x, ad, y, idx, w, residual=True)


@pytest.mark.parametrize("T", [23, 100])
def test_deterministic(q, T):
    Lc = build_layer(synth.Workload.TEST, 13, SMALL)
    Ld = to_device(Lc, SMALL, DEV)
    x = dev(synth.activations(T, SMALL.hidden, synth.Workload.TEST, 13))
    ws = q.moe_workspace(Ld, T, DEV)
    a = q.moe_switchglu_int4(Ld, x, ws=ws).clone()
    b = q.moe_switchglu_int4(Ld, x, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("T", [5, 100])
def test_stages_in_order_equal_the_whole_layer(q, T):
    """moe_switchglu_int4_stage: ROUTE, GATE_UP, DOWN in order give the bits of one call."""
    Lc = build_layer(synth.Workload.TEST, 16, SMALL)
    Ld = to_device(Lc, SMALL, DEV)
    x = dev(synth.activations(T, SMALL.hidden, synth.Workload.TEST, 16))
    ad = dev((np.arange(T) % 2).astype(np.int32))
    ws = q.moe_workspace(Ld, T, DEV)
    whole = q.moe_switchglu_int4(Ld, x, ad, ws=ws).clone()
    y = torch.empty_like(x)
    call = q.MoECall(Ld, x, y, ws, adapter_idx=ad)
    for st in (q.STAGE_ROUTE, q.STAGE_GATE_UP, q.STAGE_DOWN):
        call(st)
    call(q.STAGE_DOWN)   # a stage re-run alone repeats its work on the same inputs
    torch.cuda.synchronize()
    assert torch.equal(whole.view(torch.int16), y.view(torch.int16))


def plant_groups(L, seed):
    """Every matrix of the layer (router, gate, experts, shared expert) with planted special
    groups: about one group in eight with scale 0 (the degenerate case: each weight equals
    the group's bias whatever its code), one in eight with every code at the top level (15,
    or 255 at 8 bits) and one in eight with every code 0, as an imported checkpoint may hold
    them."""
    from oracle import affine
    rng = np.random.default_rng(seed)

    def plant(qw):
        packed, scales, biases = qw.packed.copy(), qw.scales.copy(), qw.biases.copy()
        G = scales.shape[-1]
        wpg = 64 * qw.bits // 32                       # words per group
        sel = rng.integers(0, 8, size=scales.shape)
        scales[sel == 0] = np.float16(0.0)
        words = packed.reshape(scales.shape + (wpg,))
        words[sel == 1] = np.uint32(0xFFFFFFFF)
        words[sel == 2] = np.uint32(0)
        return affine.QWeight(words.reshape(packed.shape), scales, biases, qw.bits, qw.group)

    fields = {k: plant(getattr(L, k)) for k in ("router", "shared_gate", "exp_gate", "exp_up", "exp_down",
                                                 "sh_gate", "sh_up", "sh_down")}
    return moe.MoELayer(**{**L.__dict__, **fields})


@pytest.mark.parametrize("T", [2, 7, 64, 300])
def test_layer_with_degenerate_and_extreme_groups(q, T):
    """Layer parity with planted scale-0 groups and groups of all-15 / all-0 codes in every
    matrix, on the decode path (2, 7 tokens) and the token-sorted path (64: 16-pair items;
    300: 64-pair items with fp16 weights)."""
    S = Shape(hidden=1024, inter=512, shared_inter=512, n_experts=16, top_k=4, rank=16, n_adapters=2)
    Lc = plant_groups(build_layer(synth.Workload.TEST, 21, S), 21 + T)
    x = synth.activations(T, S.hidden, synth.Workload.TEST, 21, T)
    ad = (np.arange(T) % 2).astype(np.int32)
    y, idx, w = run_device(q, Lc, S, x, ad)
    err, rel, n_alt = check_layer(Lc, x, ad, y, idx, w)
    print(f"planted groups T={T}: max abs {err:.2e} rel L2 {rel:.2e} alternatives {n_alt}", flush=True)


@pytest.mark.parametrize("S,T", [
    # rank 24: the down launch takes A_d . h_s itself
    (Shape(hidden=1024, inter=512, shared_inter=512, n_experts=16, top_k=4, rank=24, n_adapters=3), 3),
    # inter 2048: 32 shares of 64 rows per token, rank 8 (half of the 16 share slots)
    (Shape(hidden=512, inter=2048, shared_inter=2048, n_experts=8, top_k=2, rank=8, n_adapters=2), 5),
    # one token, rank 16, three adapters: the gate/up launch's per-row-block shares of z_down
    (Shape(hidden=2048, inter=512, shared_inter=512, n_experts=64, top_k=4, rank=16, n_adapters=3), 1),
    # inter 2048, top-4: the routed rows take two passes, activations staged through LDS
    (Shape(hidden=512, inter=2048, shared_inter=2048, n_experts=8, top_k=4, rank=16, n_adapters=2), 3),
])
def test_decode_path_down_lora(q, S, T):
    """Decode path (fewer than 32 routed pairs): the down LoRA's z_down = A_d h_s either summed
    from the gate/up launch's per-64-row shares (ranks up to 16) or taken by the down blocks
    themselves (larger ranks), against the oracle; the adapter changes from token to token."""
    Lc = build_layer(synth.Workload.TEST, 49, S)
    x = synth.activations(T, S.hidden, synth.Workload.TEST, 49, T)
    ad = ((np.arange(T) + 1) % S.n_adapters).astype(np.int32)
    y, idx, w = run_device(q, Lc, S, x, ad)
    err, rel, n_alt = check_layer(Lc, x, ad, y, idx, w)
    print(f"decode down LoRA rank {S.rank} inter {S.inter} T={T}: max abs {err:.2e} rel L2 {rel:.2e}", flush=True)


WIDE_H = Shape(hidden=4096, inter=512, shared_inter=512, n_experts=16, top_k=4, rank=16, n_adapters=2)


@pytest.mark.parametrize("T", [3, 40, 300])
def test_largest_hidden(q, T):
    """Hidden 4096, the largest the layer accepts: two 32-input chunks per lane in the decode
    GEMVs (3 tokens), eight split-K partials per value in the per-token kernels (40 tokens: the
    eight-wave form and the feature-sliced down; 300 tokens: the four-wave form, sorted items)."""
    Lc = build_layer(synth.Workload.TEST, 50, WIDE_H)
    x = synth.activations(T, WIDE_H.hidden, synth.Workload.TEST, 50, T)
    ad = (np.arange(T) % 2).astype(np.int32)
    y, idx, w = run_device(q, Lc, WIDE_H, x, ad)
    err, rel, n_alt = check_layer(Lc, x, ad, y, idx, w)
    print(f"hidden 4096 T={T}: max abs {err:.2e} rel L2 {rel:.2e} alternatives {n_alt}", flush=True)


@pytest.mark.parametrize("E,K,T", [
    (260, 4, 5),      # decode path, 8 logits per lane, expert count not a multiple of 64
    (1024, 8, 3),     # decode path at the most experts the layer accepts (16 logits per lane)
    (260, 16, 4),     # token-sorted path (past 256 experts: the sort launch), top-16
    (1024, 32, 9),    # the largest expert count and top-K the layer accepts
])
def test_many_experts_and_large_top_k(q, E, K, T):
    """Expert counts past 256 and top-K past 8 on both paths, against the oracle (indices
    equal up to near-ties, weights and outputs within the tolerance)."""
    S = Shape(hidden=512, inter=512, shared_inter=512, n_experts=E, top_k=K, rank=8, n_adapters=2)
    Lc = build_layer(synth.Workload.TEST, 51, S)
    x = synth.activations(T, S.hidden, synth.Workload.TEST, 51, T)
    ad = (np.arange(T) % 2).astype(np.int32)
    y, idx, w = run_device(q, Lc, S, x, ad)
    err, rel, n_alt = check_layer(Lc, x, ad, y, idx, w)
    print(f"E={E} K={K} T={T}: max abs {err:.2e} rel L2 {rel:.2e} alternatives {n_alt}", flush=True)


DEEPEST = Shape(hidden=512, inter=4096, shared_inter=2048, n_experts=8, top_k=2, rank=16, n_adapters=2)


@pytest.mark.parametrize("T", [5, 70])
def test_largest_inter(q, T):
    """Routed inner size 4096 (the largest the layer accepts) with a shared expert of 2048: the
    token-sorted path at any token count (the decode path needs equal inner sizes of at most
    2048), down GEMMs over 4096 inputs, the per-token kernel's h_s loop over 2048 outputs."""
    Lc = build_layer(synth.Workload.TEST, 52, DEEPEST)
    x = synth.activations(T, DEEPEST.hidden, synth.Workload.TEST, 52, T)
    ad = (np.arange(T) % 2).astype(np.int32)
    y, idx, w = run_device(q, Lc, DEEPEST, x, ad)
    err, rel, n_alt = check_layer(Lc, x, ad, y, idx, w)
    print(f"inter 4096 T={T}: max abs {err:.2e} rel L2 {rel:.2e} alternatives {n_alt}", flush=True)


MANY_R = Shape(hidden=1536, inter=512, shared_inter=512, n_experts=16, top_k=6, rank=24, n_adapters=3)


def test_many_tokens_combine_with_residual_adapters_and_wide_rank(q):
    """The many-token combine (from 1024 tokens): residual stacking, three adapters changing
    every few tokens (its LoRA-B rows reloaded when the adapter changes), LoRA rank 24 (a
    third chunk of 8 ranks past the 16 kept in registers), top-6 (experts past the fourth),
    and hidden 1536 (a 1024-feature block whose second half is past the features)."""
    T = 1100
    Lc = build_layer(synth.Workload.TEST, 47, MANY_R)
    x = synth.activations(T, MANY_R.hidden, synth.Workload.TEST, 47, T)
    ad = ((np.arange(T) // 5) % 3).astype(np.int32)
    y, idx, w = run_device(q, Lc, MANY_R, x, ad, residual=True)
    err, rel, n_alt = check_layer(Lc, x, ad, y, idx, w, residual=True)
    print(f"many-token combine: max abs {err:.2e} rel L2 {rel:.2e} alternatives {n_alt}", flush=True)


@pytest.mark.parametrize("K", [1, 2])
def test_layer_exact_router_tie_goes_to_lower_expert(q, K):
    """Router rows 3 and 5 identical (same words, scales and biases) and both favoured by the
    router bias: every token's logits tie exactly between them.  With top-1 the tie sits at
    the selection boundary and expert 3 must win; with top-2 both are selected, 3 first.
    Exact index equality is required here (no near-tie allowance)."""
    S = Shape(hidden=512, inter=512, shared_inter=512, n_experts=8, top_k=K, rank=8, n_adapters=1)
    Lc = build_layer(synth.Workload.TEST, 48, S)
    for arr in (Lc.router.packed, Lc.router.scales, Lc.router.biases):
        arr[5] = arr[3]
    bias = np.zeros(S.n_experts, np.float32)
    bias[[3, 5]] = 4.0
    Lc.router_bias = bias
    T = 24
    x = synth.activations(T, S.hidden, synth.Workload.TEST, 48, T)
    y, idx, w = run_device(q, Lc, S, x)
    ref = moe.moe_layer(x, Lc, None)
    expect = np.array([[3] if K == 1 else [3, 5]] * T, np.int32)
    assert np.array_equal(ref["idx"], expect)
    assert np.array_equal(idx, expect)
    if K == 2:
        np.testing.assert_allclose(w, 0.5, rtol=0, atol=1e-7)
    from layers import assert_close
    assert_close(y, ref["y64"], what="tied router")
