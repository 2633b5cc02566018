"""Guard bands around every output: each output buffer sits inside a larger allocation whose
head and tail hold a poison pattern, and after the call the poison must be untouched (no
kernel writes outside its output), while the output itself equals the same call's output
into a plain buffer."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from layers import Shape, build_layer, to_device

pytestmark = pytest.mark.gpu
DEV = "cuda"
PAD = 256   # bytes of guard on each side (keeps the interior 16-byte aligned)
POISON = 0xA5


@pytest.fixture(scope="module")
def q():
    import int4_group_quantized_amd as q
    assert torch.cuda.is_available()
    return q


class Guarded:
    """A device buffer of `shape` / `dtype` with PAD poisoned bytes before and after."""

    def __init__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.raw = torch.full((n + 2 * PAD,), POISON, dtype=torch.uint8, device=DEV)
        self.n = n
        self.t = self.raw[PAD:PAD + n].view(dtype).view(shape)

    def check(self, what):
        torch.cuda.synchronize()
        head = self.raw[:PAD].cpu().numpy()
        tail = self.raw[PAD + self.n:].cpu().numpy()
        assert np.all(head == POISON) and np.all(tail == POISON), f"{what}: write outside the output"


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


S = Shape(hidden=512, inter=512, shared_inter=512, n_experts=16, top_k=4, rank=8, n_adapters=2)


@pytest.fixture(scope="module")
def layer():
    Lc = build_layer(synth.Workload.TEST, 60, S)
    return Lc, to_device(Lc, S, DEV)


@pytest.mark.parametrize("T", [1, 5, 40, 300])
def test_moe_layer_outputs(q, layer, T):
    _, Ld = layer
    x = torch.from_numpy(synth.activations(T, S.hidden, synth.Workload.TEST, 60, T)).to(DEV)
    ad = torch.from_numpy((np.arange(T) % 2).astype(np.int32)).to(DEV)
    ref = q.moe_switchglu_int4(Ld, x, ad, return_routing=True)
    y, idx, w = Guarded((T, S.hidden), torch.float16), Guarded((T, 4), torch.int32), Guarded((T, 4), torch.float32)
    ws = q.moe_workspace(Ld, T, DEV)
    c = Ld.c()
    st = q.lib.moe_switchglu_int4(ctypes.byref(c), x.data_ptr(), T, ad.data_ptr(), y.t.data_ptr(),
                                  idx.t.data_ptr(), w.t.data_ptr(), ws.data_ptr(), ws.numel(), stream())
    assert st == 0
    for g, r, name in ((y, ref[0], "y"), (idx, ref[1], "idx_out"), (w, ref[2], "w_out")):
        g.check(name)
        assert torch.equal(g.t, r), name
    # the routed and the allocation-free forms
    route = torch.from_numpy(synth.expert_choices(T, 4, S.n_experts, synth.Workload.TEST, 60, T)).to(DEV)
    y2, w2 = Guarded((T, S.hidden), torch.float16), Guarded((T, 4), torch.float32)
    st = q.lib.moe_switchglu_int4_routed(ctypes.byref(c), x.data_ptr(), T, ad.data_ptr(), route.data_ptr(),
                                         y2.t.data_ptr(), w2.t.data_ptr(), ws.data_ptr(), ws.numel(), stream())
    assert st == 0
    y2.check("routed y")
    w2.check("routed w_out")
    y3, i3, w3 = Guarded((T, S.hidden), torch.float16), Guarded((T, 4), torch.int32), Guarded((T, 4), torch.float32)
    st = q.lib.moe_switchglu_int4_noalloc(ctypes.byref(c), x.data_ptr(), T, ad.data_ptr(), y3.t.data_ptr(),
                                          i3.t.data_ptr(), w3.t.data_ptr(), stream())
    assert st == 0
    for g, r, name in ((y3, ref[0], "noalloc y"), (i3, ref[1], "noalloc idx_out"), (w3, ref[2], "noalloc w_out")):
        g.check(name)
        assert torch.equal(g.t, r), name


@pytest.mark.parametrize("m", [1, 3, 40])
def test_qlinear_and_lora_outputs(q, m):
    w = torch.from_numpy(synth.normal_f32((384, 1024), 0.02, synth.Workload.TEST, 61, synth.Role.DENSE)).to(DEV)
    qw = q.quantize_affine(w, 4)
    x = torch.from_numpy(synth.activations(m, 1024, synth.Workload.TEST, 61, m)).to(DEV)
    ref = q.qlinear_int4(x, qw)
    y = Guarded((m, 384), torch.float16)
    c = qw.c()
    assert q.lib.qlinear_int4(x.data_ptr(), m, ctypes.byref(c), None, None, y.t.data_ptr(), stream()) == 0
    y.check("qlinear y")
    assert torch.equal(y.t, ref)
    A = torch.from_numpy(synth.normal_f16((2, 16, 1024), 0.01, synth.Workload.TEST, 61, synth.Role.LORA_A_UP)).to(DEV)
    B = torch.from_numpy(synth.normal_f16((2, 384, 16), 0.01, synth.Workload.TEST, 61, synth.Role.LORA_B_UP)).to(DEV)
    lo = q.Lora(A, B, 2.0)
    acc = Guarded((m, 384), torch.float32)
    acc.t.zero_()
    lc = lo.c()
    assert q.lib.lora_apply(x.data_ptr(), m, ctypes.byref(lc), None, acc.t.data_ptr(), stream()) == 0
    acc.check("lora_apply y_acc")


def test_quantize_unpack_dequantize_outputs(q):
    rows, cols = 96, 512
    w = torch.from_numpy(synth.normal_f32((rows, cols), 0.02, synth.Workload.TEST, 62, synth.Role.DENSE)).to(DEV)
    for bits in (4, 8):
        p = Guarded((rows, cols * bits // 32), torch.int32)
        s = Guarded((rows, cols // 64), torch.float16)
        b = Guarded((rows, cols // 64), torch.float16)
        assert q.lib.qmoe_quantize_affine(w.data_ptr(), rows, cols, bits, 64, p.t.data_ptr(), s.t.data_ptr(),
                                          b.t.data_ptr(), stream()) == 0
        for g, name in ((p, "packed"), (s, "scales"), (b, "biases")):
            g.check(f"quantize {bits}-bit {name}")
        u = Guarded((rows, cols), torch.uint8)
        assert q.lib.qmoe_unpack(p.t.data_ptr(), rows, cols, bits, u.t.data_ptr(), stream()) == 0
        u.check(f"unpack {bits}-bit")
        d = Guarded((rows, cols), torch.float32)
        qw = q.QWeight(p.t, s.t, b.t, bits, rows, cols)
        c = qw.c()
        assert q.lib.qmoe_dequantize(ctypes.byref(c), d.t.data_ptr(), stream()) == 0
        d.check(f"dequantize {bits}-bit")


@pytest.mark.parametrize("B", [1, 64])
def test_supergroup_and_act8_outputs(q, B):
    w = torch.from_numpy(synth.normal_f32((512, 1024), 0.02, synth.Workload.TEST, 63, synth.Role.SUPERGROUP)).to(DEV)
    W = q.quantize_supergroup(w, 4)
    x = torch.from_numpy(synth.activations(B, 1024, synth.Workload.TEST, 63, B)).to(DEV)
    for name, fn, ref in (("qlinear_supergroup", q.lib.qlinear_supergroup, q.qlinear_supergroup(x, W)),
                          ("qlinear_supergroup_a8", q.lib.qlinear_supergroup_a8, q.qlinear_supergroup_a8(x, W))):
        y = Guarded((B, 512), torch.float16)
        assert fn(x.data_ptr(), B, W.p4.data_ptr(), W.p2.data_ptr(), W.scales.data_ptr(), 512, 1024, 4,
                  y.t.data_ptr(), stream()) == 0
        y.check(name)
        assert torch.equal(y.t, ref), name
    qx, sx = Guarded((B, 1024), torch.int8), Guarded((B,), torch.float16)
    assert q.lib.qmoe_quantize_act8(x.data_ptr(), B, 1024, qx.t.data_ptr(), sx.t.data_ptr(), stream()) == 0
    qx.check("act8 codes")
    sx.check("act8 scales")
    p4, p2, sc = Guarded((128, 128), torch.int32), Guarded((384, 64), torch.int32), Guarded((512,), torch.float16)
    assert q.lib.qmoe_quantize_supergroup(w.data_ptr(), 512, 1024, 4, p4.t.data_ptr(), p2.t.data_ptr(),
                                          sc.t.data_ptr(), stream()) == 0
    for g, name in ((p4, "p4"), (p2, "p2"), (sc, "super-group scales")):
        g.check(name)


def test_router_and_prerouter_outputs(q):
    t, e, k = 9, 64, 4
    logits = torch.randn((t, e), device=DEV, generator=torch.Generator(device=DEV).manual_seed(64))
    idx, w = Guarded((t, k), torch.int32), Guarded((t, k), torch.float32)
    assert q.lib.router_topk(logits.data_ptr(), t, e, k, None, idx.t.data_ptr(), w.t.data_ptr(), stream()) == 0
    idx.check("router_topk idx")
    w.check("router_topk weights")
    D, E, F = 512, 64, 512
    R = synth.Role.MISC
    f16 = lambda shape, i: torch.from_numpy(synth.normal_f16(shape, 0.02, synth.Workload.TEST, 64, R, i)).to(DEV)
    P = q.PrerouterHead(f16((E, D + 2 * E), 0), f16((E,), 1), f16((F, D + 2 * E), 2), f16((F,), 3),
                        f16((E, F), 4), f16((E,), 5))
    h = torch.from_numpy(synth.activations(t, D, synth.Workload.TEST, 64)).to(DEV)
    now = torch.from_numpy(synth.expert_choices(t, k, E, synth.Workload.TEST, 64, 1)).to(DEV)
    prev = torch.from_numpy(synth.expert_choices(t, k, E, synth.Workload.TEST, 64, 2)).to(DEV)
    act, lg = Guarded((t, F), torch.float16), Guarded((t, E), torch.float32)
    pi, pw = Guarded((t, k), torch.int32), Guarded((t, k), torch.float32)
    c = P.c()
    assert q.lib.prerouter_forward(ctypes.byref(c), h.data_ptr(), t, k, now.data_ptr(), prev.data_ptr(),
                                   act.t.data_ptr(), lg.t.data_ptr(), pi.t.data_ptr(), pw.t.data_ptr(), stream()) == 0
    for g, name in ((act, "act"), (lg, "logits"), (pi, "pred_idx"), (pw, "pred_w")):
        g.check(f"prerouter {name}")
