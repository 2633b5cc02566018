"""GPU parity of the MoE layer whose routed expert stacks are in the bit-exact port page's
checkpoint format ("Bit-exact MLX 4-bit port of d1a-e2b-it-qat-4bit", "4-bit group
quantization": 32 weights per group, scale and bias stored as bf16), and in the two mixed
formats (group 32 with fp16 parameters, group 64 with bf16 parameters), against the oracle.

Such a layer runs the token-sorted path at every token count (one token included), with the
routed experts' parameters staged per block (bf16 converted to fp16, exact for these
weights' parameters, which lie inside fp16's normal range).
"""
import numpy as np
import pytest
import torch

import synth
from layers import Shape, build_layer, to_device
from oracle import moe
from test_gpu_moe import check_layer, dev

pytestmark = pytest.mark.gpu

FMT = Shape(hidden=1024, inter=512, shared_inter=512, n_experts=16, top_k=4, rank=8, n_adapters=2)
FMT_WIDE = Shape(hidden=2048, inter=1024, shared_inter=512, n_experts=8, top_k=2, rank=16, n_adapters=1)


@pytest.fixture(scope="module")
def q():
    import int4_group_quantized_amd as q
    assert torch.cuda.is_available()
    return q


def run(q, Lc, S, x, ad):
    Ld = to_device(Lc, S, "cuda")
    y, idx, w = q.moe_switchglu_int4(Ld, dev(x), dev(ad), return_routing=True)
    torch.cuda.synchronize()
    return y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("group,params", [(32, "bf16"), (32, "f16"), (64, "bf16")],
                         ids=["g32-bf16", "g32-f16", "g64-bf16"])
@pytest.mark.parametrize("T", [1, 5, 40, 300])
def test_layer_expert_formats(q, group, params, T):
    """One token (where standard stacks take the decode path), a few, 16-pair items and
    64-pair items (300 tokens x top-4 over 16 experts)."""
    S = FMT
    Lc = build_layer(synth.Workload.TEST, 40 + group, S, expert_group=group, expert_params=params)
    assert Lc.exp_gate.group == group and Lc.exp_gate.param_dtype == params
    x = synth.activations(T, S.hidden, synth.Workload.TEST, 40 + group, T)
    ad = (np.arange(T) % S.n_adapters).astype(np.int32)
    y, idx, w = run(q, Lc, S, x, ad)
    err, rel, n_alt = check_layer(Lc, x, ad, y, idx, w)
    print(f"experts g{group} {params} T={T}: max abs {err:.2e} rel L2 {rel:.2e} alternatives {n_alt}", flush=True)


@pytest.mark.parametrize("T", [3, 200])
def test_layer_port_format_wide(q, T):
    """The port format at hidden 2048 and inter 1024 (16- and 8-step reductions)."""
    S = FMT_WIDE
    Lc = build_layer(synth.Workload.TEST, 45, S, expert_group=32, expert_params="bf16")
    x = synth.activations(T, S.hidden, synth.Workload.TEST, 45, T)
    ad = np.zeros(T, np.int32)
    y, idx, w = run(q, Lc, S, x, ad)
    err, rel, n_alt = check_layer(Lc, x, ad, y, idx, w)
    print(f"port format wide T={T}: max abs {err:.2e} rel L2 {rel:.2e} alternatives {n_alt}", flush=True)


def test_port_format_routed_and_deterministic(q):
    """A given routing on such a layer (the prerouter's prediction as the route) matches the
    oracle under that routing, and repeated calls are bit-identical."""
    S = FMT
    Lc = build_layer(synth.Workload.TEST, 46, S, expert_group=32, expert_params="bf16")
    T = 24
    x = synth.activations(T, S.hidden, synth.Workload.TEST, 46, T)
    ad = (np.arange(T) % S.n_adapters).astype(np.int32)
    rng = np.random.default_rng(7)
    route = np.stack([rng.choice(S.n_experts, S.top_k, replace=False) for _ in range(T)]).astype(np.int32)
    Ld = to_device(Lc, S, "cuda")
    ys = [q.moe_switchglu_int4_routed(Ld, dev(x), dev(route), dev(ad)) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1])
    ref = moe.moe_layer(x, Lc, ad, idx=route)
    from layers import assert_close
    assert_close(ys[0].cpu().numpy().astype(np.float64), ref["y64"], what="routed port format")
