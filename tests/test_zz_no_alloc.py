"""The allocation-free layer call (moe_switchglu_int4_noalloc) against the workspace call
(moe_switchglu_int4), through the C ABI: bit-identical outputs and routing on consecutive
calls that share the library's scratch, a smaller call after a larger one and a larger one
after it, on the token-sorted and the decode launch sequences."""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def layer():
    import synth
    from layers import Shape, build_layer, to_device
    S = Shape(hidden=1024, inter=512, shared_inter=512, n_experts=32, top_k=4, rank=16, n_adapters=2)
    Lc = build_layer(synth.Workload.TEST, 77, S)
    return S, Lc, to_device(Lc, S, "cuda")


def run_both(q, S, Ld, t, seed):
    import synth
    x = torch.from_numpy(synth.activations(t, S.hidden, synth.Workload.TEST, 77, seed)).cuda()
    ad = torch.from_numpy((np.arange(t) % 2).astype(np.int32)).cuda()
    ref_y, ref_i, ref_w = q.moe_switchglu_int4(Ld, x, ad, return_routing=True)
    y = torch.full_like(x, float("nan"))
    idx = torch.full((t, S.top_k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((t, S.top_k), float("nan"), dtype=torch.float32, device="cuda")
    c = Ld.c()
    st = q.lib.moe_switchglu_int4_noalloc(ctypes.byref(c), x.data_ptr(), t, ad.data_ptr(), y.data_ptr(),
                                          idx.data_ptr(), w.data_ptr(),
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, q.lib.qmoe_status_string(st)
    torch.cuda.synchronize()
    return x, ad, (ref_y, ref_i, ref_w), (y, idx, w)


def test_noalloc_matches_workspace_call_on_consecutive_calls(layer):
    import int4_group_quantized_amd as q
    from layers import assert_close
    from oracle import moe
    S, Lc, Ld = layer
    for t, seed in ((40, 1), (3, 2), (64, 3)):       # token-sorted, decode, token-sorted again
        print(f"noalloc t={t}", flush=True)
        x, ad, ref, got = run_both(q, S, Ld, t, seed)
        for r, g in zip(ref, got):
            assert torch.equal(r, g), f"t={t}: allocation-free call differs from the workspace call"
        out = moe.moe_layer(x.cpu().numpy(), Lc, ad.cpu().numpy())
        assert np.array_equal(got[1].cpu().numpy(), out["idx"])
        assert_close(got[0].cpu().numpy(), out["y64"], what=f"noalloc t={t}")


def test_noalloc_refuses_token_counts_beyond_its_scratch(layer):
    import int4_group_quantized_amd as q
    S, Lc, Ld = layer
    c = Ld.c()
    t = 1
    while q.lib.moe_switchglu_int4_workspace_bytes(ctypes.byref(c), t) <= q._lib.NOALLOC_SCRATCH_BYTES:
        t *= 2
    x = torch.zeros((t, S.hidden), dtype=torch.float16, device="cuda")
    y = torch.empty_like(x)
    st = q.lib.moe_switchglu_int4_noalloc(ctypes.byref(c), x.data_ptr(), t, None, y.data_ptr(), None, None,
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == q._lib.QMOE_ERR_WORKSPACE
