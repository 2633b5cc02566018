"""Parity of the prerouter head (HIP, through the C ABI) with the oracle on seeded inputs."""
import numpy as np
import pytest
import torch

import synth
from layers import assert_close
from oracle import moe
from oracle import prerouter as pr

pytestmark = pytest.mark.gpu
DEV = "cuda"
W = synth.Workload.TEST
R = synth.Role.MISC


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.fixture(scope="module")
def q():
    import int4_group_quantized_amd as q
    assert torch.cuda.is_available()
    return q


def make_head(D, E, F, seed):
    n = D + 2 * E
    return pr.PrerouterHead(synth.normal_f16((E, n), 0.02, W, seed, R, 0), synth.normal_f16((E,), 0.02, W, seed, R, 1),
                            synth.normal_f16((F, n), 0.02, W, seed, R, 2), synth.normal_f16((F,), 0.02, W, seed, R, 3),
                            synth.normal_f16((E, F), 0.05, W, seed, R, 4), synth.normal_f16((E,), 0.02, W, seed, R, 5))


def routing(t, E, k, seed):
    g = np.random.default_rng(seed)
    return np.array([g.choice(E, k, replace=False) for _ in range(t)], np.int32)


@pytest.mark.parametrize("D,E,F,k,t", [(2048, 256, 512, 4, 1), (2048, 256, 512, 4, 5), (2048, 256, 512, 8, 9),
                                       (512, 64, 1024, 8, 3), (4096, 128, 512, 2, 20), (8192, 256, 512, 4, 2)])
def test_prerouter_matches_oracle(q, D, E, F, k, t):
    """Hidden activations and logits to the float bar; the predicted routing is the router's
    exact selection on the kernel's own logits (fp16-rounded logits tie often: the rule, not
    the float path, decides those)."""
    print(f"prerouter D={D} E={E} F={F} k={k} t={t}", flush=True)
    P = make_head(D, E, F, D + E + k)
    h = synth.activations(t, D, W, 7, t)
    now, prev = routing(t, E, k, 1), routing(t, E, k, 2)
    Pd = q.PrerouterHead(*(dev(getattr(P, n)) for n in ("w_init", "b_init", "w1", "b1", "w2", "b2")))
    act, logits, idx, w = q.prerouter_forward(Pd, dev(h), dev(now), dev(prev))
    a_ref, l_ref = pr.forward(P, h, now, prev)
    assert_close(host(act), a_ref.astype(np.float64), what="prerouter act")
    lg = host(logits)
    assert_close(lg.astype(np.float16), l_ref.astype(np.float64), what="prerouter logits")
    assert np.array_equal(lg.astype(np.float16).astype(np.float32), lg)     # fp16-rounded values
    sel, wts = moe.topk_f32(lg, k)
    assert np.array_equal(host(idx), sel)
    np.testing.assert_allclose(host(w), wts, rtol=1e-5, atol=1e-6)
    n_alt = prediction_matches_oracle(host(idx), l_ref, k)
    print(f"  prediction: {t - n_alt} of {t} tokens select the oracle's set, {n_alt} a near-tie alternative", flush=True)


def prediction_matches_oracle(sel_dev, l_ref, k):
    """The device's predicted set against the oracle's own prediction (top-K of the oracle's
    logits, lower index on ties).  fp16 logits of the two sides may differ by a rounding step,
    so a token may differ only where the oracle's K-th and (K+1)-th logits lie within two fp16
    steps of each other, and then every device pick must lie in that band.  Returns the
    number of such tokens."""
    lr = np.asarray(l_ref, np.float32)
    ref_sel, _ = moe.topk_f32(lr, k)
    n_alt = 0
    for t in range(lr.shape[0]):
        if set(sel_dev[t].tolist()) == set(ref_sel[t].tolist()):
            continue
        order = np.argsort(-lr[t], kind="stable")
        lk, lk1 = float(lr[t][order[k - 1]]), float(lr[t][order[k]])
        step = 2.0 ** (np.floor(np.log2(max(abs(lk), 2.0 ** -14))) - 10)
        assert lk - lk1 <= 2 * step, (t, sel_dev[t], ref_sel[t], lk, lk1)
        assert all(lr[t][i] >= lk - 2 * step for i in sel_dev[t]), (t, sel_dev[t], ref_sel[t])
        n_alt += 1
    return n_alt


def test_prerouter_indices_out_of_range_are_clamped(q):
    """Indices outside [0, E) act as the nearest valid expert (no out-of-bounds reads)."""
    D, E, F, k, t = 512, 16, 512, 2, 2
    P = make_head(D, E, F, 3)
    h = synth.activations(t, D, W, 8)
    now = np.array([[-5, 3], [1, 99]], np.int32)
    prev = np.array([[0, 15], [2, 3]], np.int32)
    Pd = q.PrerouterHead(*(dev(getattr(P, n)) for n in ("w_init", "b_init", "w1", "b1", "w2", "b2")))
    _, logits, _, _ = q.prerouter_forward(Pd, dev(h), dev(now), dev(prev), predict=False)
    _, l_ref = pr.forward(P, h, np.clip(now, 0, E - 1), prev)
    assert_close(host(logits).astype(np.float16), l_ref.astype(np.float64), what="clamped")
