"""Pins for the oracle's prerouter head (CPU only)."""
import numpy as np
import torch

import synth
from oracle import prerouter as pr

W = synth.Workload.TEST


def _head(D=256, E=16, F=64, seed=0):
    g = np.random.default_rng(seed)
    n = D + 2 * E
    mk = lambda *s: (g.standard_normal(s) * 0.05).astype(np.float16)
    return pr.PrerouterHead(mk(E, n), mk(E), mk(F, n), mk(F), mk(E, F), mk(E))


def test_gelu_erf_known_values_and_torch():
    """gelu(0) = 0; gelu(1) = Phi(1) = 0.841344746068543; gelu(-1) = -(1 - Phi(1)) =
    -0.158655253931457; gelu(x) -> x for large x; and torch's exact (erf) GELU on CPU."""
    v = pr.gelu_erf(np.array([0.0, 1.0, -1.0, 8.0]))
    assert v[0] == 0.0
    assert abs(v[1] - 0.841344746068543) < 1e-15 and abs(v[2] + 0.158655253931457) < 1e-15
    assert abs(v[3] - 8.0) < 1e-12
    z = np.linspace(-6, 6, 1001)
    ref = torch.nn.functional.gelu(torch.from_numpy(z)).numpy()
    assert np.max(np.abs(pr.gelu_erf(z) - ref)) < 1e-14


def test_features_layout():
    h = np.arange(8, dtype=np.float16).reshape(2, 4)
    f = pr.features(h, np.array([[1, 3], [0, 2]]), np.array([[2, 3], [1, 1 + 2]]), E=4)
    assert f.shape == (2, 4 + 8)
    assert f[0, :4].tolist() == [0, 1, 2, 3]
    assert f[0, 4:8].tolist() == [0, 1, 0, 1] and f[0, 8:].tolist() == [0, 0, 1, 1]
    assert f[1, 4:8].tolist() == [1, 0, 1, 0] and f[1, 8:].tolist() == [0, 1, 0, 1]


def test_linear_init_branch_is_column_sums():
    """With fc1 and fc2 zeroed, gelu(0) = 0 and the head is fp16(fp16(W_init[:, :D] h + the
    K columns of this token's experts + the K columns of the previous token's + b_init) +
    fp16(b2)), written out with explicit column sums."""
    P = _head(seed=1)
    P.w1[:] = 0
    P.b1[:] = 0
    P.w2[:] = 0
    D, E = P.hidden, P.n_experts
    g = np.random.default_rng(2)
    h = (g.standard_normal((3, D))).astype(np.float16)
    now = np.array([g.choice(E, 4, replace=False) for _ in range(3)])
    prev = np.array([g.choice(E, 4, replace=False) for _ in range(3)])
    a, logits = pr.forward(P, h, now, prev)
    assert np.all(a == 0)
    Wi = P.w_init.astype(np.float64)
    for t in range(3):
        y0 = Wi[:, :D] @ h[t].astype(np.float64) + P.b_init.astype(np.float64)
        for e in now[t]:
            y0 = y0 + Wi[:, D + e]
        for e in prev[t]:
            y0 = y0 + Wi[:, D + E + e]
        want = (y0.astype(np.float16).astype(np.float64) + P.b2.astype(np.float64)).astype(np.float16)
        assert np.array_equal(logits[t], want)


def test_forward_matches_torch_fp32_modules():
    """The whole head against torch's CPU Linear / GELU modules in float32 on the same fp16
    parameters (an independent implementation of the same layers), rounding to fp16 after
    each layer as fp16 modules do: within two fp16 steps (the float32 sums round z a step
    apart now and then)."""
    P = _head(D=512, E=32, F=128, seed=3)
    D, E = P.hidden, P.n_experts
    g = np.random.default_rng(4)
    h = g.standard_normal((5, D)).astype(np.float16)
    now = np.array([g.choice(E, 8, replace=False) for _ in range(5)])
    prev = np.array([g.choice(E, 8, replace=False) for _ in range(5)])
    a, logits = pr.forward(P, h, now, prev)

    def lin(w, b):
        m = torch.nn.Linear(w.shape[1], w.shape[0])
        m.weight.data = torch.from_numpy(w.astype(np.float32))
        m.bias.data = torch.from_numpy(b.astype(np.float32))
        return m
    f = torch.zeros((5, D + 2 * E))
    f[:, :D] = torch.from_numpy(h.astype(np.float32))
    for t in range(5):
        f[t, D + torch.from_numpy(now[t])] = 1.0
        f[t, D + E + torch.from_numpy(prev[t])] = 1.0
    r16 = lambda v: v.half().float()
    z = r16(lin(P.w1, P.b1)(f))
    ta = r16(torch.nn.functional.gelu(z))
    tl = r16(r16(lin(P.w_init, P.b_init)(f)) + r16(lin(P.w2, P.b2)(ta)))
    d = np.abs(logits.astype(np.float64) - tl.detach().numpy().astype(np.float64))
    assert np.all(d <= np.abs(logits.astype(np.float64)) * 2.0 ** -9 + 2.0 ** -20)
    assert np.mean(a.astype(np.float32) == ta.detach().numpy()) > 0.98
