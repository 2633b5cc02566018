"""GPU parity of the building blocks against the oracle, through the C ABI.

Bit-exact: quantized words, scales, biases, unpacked codes, fp32 dequantized weights,
top-K indices on given logits, super-group codes and scales.  Floating point: max abs
2e-2 and relative L2 1e-3 against the float64 oracle.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import affine, moe, supergroup
from layers import assert_close

pytestmark = pytest.mark.gpu
W = synth.Workload.TEST
DEV = "cuda"


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


def ulp_distance(a, b):
    """Largest distance in fp16 steps between two fp16 arrays (ordered-integer view)."""
    def ordered(v):
        i = np.asarray(v, np.float16).view(np.int16).astype(np.int32)
        return np.where(i < 0, -32768 - i, i)
    return int(np.max(np.abs(ordered(a) - ordered(b))))


def special_matrix(rows, cols, seed):
    """N(0, 0.02) with planted degenerate groups, outliers and on-grid groups."""
    g = np.random.default_rng(seed)
    w = (g.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    w[0, :64] = 0.5                      # constant group: scale 0
    w[1, 64:128] = 0.0
    w[2, 5] = 3.0                        # outlier
    w[3, :64] = (np.arange(64) % 16 * 0.25 - 1).astype(np.float32)   # on an int4 grid
    return w


# ------------------------------------------------------------------------------ quantize

@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("shape", [(512, 2048), (7, 64), (33, 192), (256, 2048), (2048, 512)])
def test_quantize_bit_exact(q, bits, shape):
    print(f"quantize bits={bits} shape={shape}", flush=True)
    w = special_matrix(*shape, seed=shape[0] * 31 + bits)
    ref = affine.quantize(w, bits)
    got = q.quantize_affine(dev(w), bits)
    assert np.array_equal(host(got.packed).view(np.uint32), ref.packed)
    assert np.array_equal(host(got.scales).view(np.uint16), ref.scales.view(np.uint16))
    assert np.array_equal(host(got.biases).view(np.uint16), ref.biases.view(np.uint16))


def test_quantize_full_expert_stack_slice(q):
    """A config-sized matrix from the seeded generator (gate_proj of expert 0)."""
    w = synth.normal_f32((512, 2048), 0.02, synth.Workload.MOE_DECODE, 0, synth.Role.EXP_GATE, 0)
    ref = affine.quantize(w, 4)
    got = q.quantize_affine(dev(w), 4)
    assert np.array_equal(host(got.packed).view(np.uint32), ref.packed)
    assert np.array_equal(host(got.scales).view(np.uint16), ref.scales.view(np.uint16))


@pytest.mark.parametrize("bits", [4, 8])
def test_unpack_and_dequantize_bit_exact(q, bits):
    words = synth.random_words((96, 2048 * bits // 32), W, 1, synth.Role.WORDS, bits)
    sc = synth.uniform_f16((96, 32), -0.05, 0.05, W, 1, synth.Role.SCALES, bits)
    bi = synth.uniform_f16((96, 32), -1.0, 1.0, W, 1, synth.Role.BIASES, bits)
    qw = affine.QWeight(words, sc, bi, bits, 64)
    g = q.QWeight.from_arrays(words, sc, bi, bits, DEV)
    assert np.array_equal(host(q.unpack(g)), affine.unpack(words, bits))
    assert np.array_equal(host(q.dequantize(g)).view(np.uint32), affine.dequantize_f32(qw).view(np.uint32))


def test_dequantize_expert_stack(q):
    E = 3
    words = synth.random_words((E, 64, 64), W, 2, synth.Role.WORDS)
    sc = synth.uniform_f16((E, 64, 8), 0.0, 0.02, W, 2, synth.Role.SCALES)
    bi = synth.uniform_f16((E, 64, 8), -0.1, 0.0, W, 2, synth.Role.BIASES)
    g = q.QWeight.from_arrays(words, sc, bi, 4, DEV)
    out = host(q.dequantize(g)).reshape(E, 64, 512)
    for e in range(E):
        ref = affine.dequantize_f32(affine.QWeight(words[e], sc[e], bi[e], 4, 64))
        assert np.array_equal(out[e].view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------------------------ qlinear

def _qw(rows, cols, bits, idx):
    w = synth.normal_f32((rows, cols), 0.02, W, 3, synth.Role.DENSE, idx)
    return affine.quantize(w, bits)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("m,rows,cols", [(1, 512, 2048), (1, 2048, 512), (3, 96, 1024),
                                         (8, 40, 1536), (13, 64, 2048), (1, 1, 512),
                                         (2, 130, 4096)])
def test_qlinear_matches_oracle(q, bits, m, rows, cols):
    print(f"qlinear bits={bits} m={m} rows={rows} cols={cols}", flush=True)
    ref_w = _qw(rows, cols, bits, rows + cols + m)
    x = synth.activations(m, cols, W, 3, m)
    y = host(q.qlinear_int4(dev(x), q.QWeight.from_arrays(ref_w.packed, ref_w.scales, ref_w.biases, bits, DEV)))
    assert_close(y, moe.qlinear(x, ref_w), what="qlinear")


def test_qlinear_decode_workload_with_seeded_generator(q):
    """The decode GEMV workload: x [1 x 2048] ~ N(0,1), W [512 x 2048] ~ N(0, 0.02)."""
    w = synth.normal_f32((512, 2048), 0.02, synth.Workload.GEMV, 0, synth.Role.DENSE)
    x = synth.activations(1, 2048, synth.Workload.GEMV)
    ref_w = affine.quantize(w, 4)
    gw = q.quantize_affine(dev(w), 4)       # the device quantizer feeds the device GEMV
    assert np.array_equal(host(gw.packed).view(np.uint32), ref_w.packed)
    y = host(q.qlinear_int4(dev(x), gw))
    ref = moe.qlinear(x, ref_w)
    assert_close(y, ref, what="gemv workload")
    assert ulp_distance(y, moe.to_f16(ref)) <= 1   # within one fp16 step of exact rounding


def test_qlinear_integer_case_exact(q):
    """scale 1, bias 0, integer x: every partial sum is an integer below 2^24, so the
    device result is exact."""
    g = np.random.default_rng(5)
    N, K, T = 64, 2048, 2
    codes = g.integers(0, 16, size=(N, K)).astype(np.uint8)
    qw = affine.QWeight(affine.pack(codes, 4), np.ones((N, 32), np.float16),
                        np.zeros((N, 32), np.float16), 4, 64)
    x = g.integers(-2, 3, size=(T, K)).astype(np.float16)
    y = host(q.qlinear_int4(dev(x), q.QWeight.from_arrays(qw.packed, qw.scales, qw.biases, 4, DEV)))
    ref = (x.astype(np.int64) @ codes.astype(np.int64).T).astype(np.float16)
    assert np.array_equal(y, ref)


def test_qlinear_with_lora_and_adapters(q):
    rows, cols, T, n_ad, r = 512, 2048, 8, 4, 16
    ref_w = _qw(rows, cols, 4, 77)
    A = synth.normal_f16((n_ad, r, cols), 0.01, W, 4, synth.Role.LORA_A_GATE)
    B = synth.normal_f16((n_ad, rows, r), 0.01, W, 4, synth.Role.LORA_B_GATE)
    L = moe.Lora(A, B, 2.0)
    ad = synth.adapter_index(T, 2)
    x = synth.activations(T, cols, W, 4)
    gw = q.QWeight.from_arrays(ref_w.packed, ref_w.scales, ref_w.biases, 4, DEV)
    y = host(q.qlinear_int4(dev(x), gw, q.Lora(dev(A), dev(B), 2.0), dev(ad)))
    assert_close(y, moe.qlinear(x, ref_w, L, ad), what="qlinear+lora")


# ------------------------------------------------------------------------------ router

@pytest.mark.parametrize("t,e,k", [(1, 256, 4), (16, 256, 8), (512, 256, 4), (5, 1024, 32),
                                   (3, 7, 7), (2, 64, 1)])
def test_router_topk_bit_exact_on_given_logits(q, t, e, k):
    g = np.random.default_rng(t * 1000 + e + k)
    logits = g.standard_normal((t, e)).astype(np.float32)
    bias = np.zeros(e, np.float32)
    bias[:min(16, e)] = 2.0
    for b in (None, bias):
        idx, w = q.router_topk(dev(logits), k, None if b is None else dev(b))
        ridx, rw = moe.topk_f32(logits, k, b)
        assert np.array_equal(host(idx), ridx)
        np.testing.assert_allclose(host(w), rw, rtol=0, atol=1e-6)


def test_router_topk_exact_ties(q):
    logits = np.zeros((4, 256), np.float32)
    logits[0, [200, 3, 77, 150]] = 1.0
    logits[1, :] = 0.25                                  # all tied -> 0, 1, 2, 3
    logits[2, [9, 8]] = 5.0
    logits[2, [255, 0]] = 4.0
    logits[3, :] = -np.arange(256, dtype=np.float32)[::-1]   # increasing: top are 255...
    idx, w = q.router_topk(dev(logits), 4)
    ridx, rw = moe.topk_f32(logits, 4)
    assert np.array_equal(host(idx), ridx)
    assert host(idx)[1].tolist() == [0, 1, 2, 3]
    assert host(idx)[2].tolist() == [8, 9, 0, 255]
    np.testing.assert_allclose(host(w)[1], 0.25, atol=1e-7)


# ------------------------------------------------------------------------------ LoRA

@pytest.mark.parametrize("t,in_dim,out_dim,r,n_ad", [(1, 2048, 512, 16, 1), (16, 2048, 512, 16, 4),
                                                     (3, 512, 2048, 16, 2), (2, 1024, 300, 64, 1)])
def test_lora_apply(q, t, in_dim, out_dim, r, n_ad):
    A = synth.normal_f16((n_ad, r, in_dim), 0.01, W, 5, synth.Role.LORA_A_UP, r)
    B = synth.normal_f16((n_ad, out_dim, r), 0.01, W, 5, synth.Role.LORA_B_UP, r)
    L = moe.Lora(A, B, 32.0 / r)
    x = synth.activations(t, in_dim, W, 5, t)
    ad = (np.arange(t) % n_ad).astype(np.int32)
    y0 = synth.normal_f32((t, out_dim), 1.0, W, 5, synth.Role.MISC)
    got = host(q.lora_apply(dev(x), q.Lora(dev(A), dev(B), L.scale), dev(y0.copy()), dev(ad)))
    ref = y0.astype(np.float64) + moe.lora_delta(x, L, ad)
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-6)


# ------------------------------------------------------------------------------ super-group

@pytest.mark.parametrize("rows,cols,period", [(3072, 1024, 4), (64, 512, 4), (48, 2048, 2),
                                              (16, 512, 1)])
def test_supergroup_quantize_bit_exact(q, rows, cols, period):
    w = synth.normal_f32((rows, cols), 0.02, synth.Workload.SUPERGROUP, 0, synth.Role.SUPERGROUP, rows + period)
    w[0, :] = 0.0                                                       # epsilon floor
    ref, _ = supergroup.quantize(w, period)
    got = q.quantize_supergroup(dev(w), period)
    assert np.array_equal(host(got.scales).view(np.uint16), ref.scales.view(np.uint16))
    assert np.array_equal(host(got.p4).view(np.uint32), ref.p4)
    if period > 1:
        assert np.array_equal(host(got.p2).view(np.uint32), ref.p2)


@pytest.mark.parametrize("b", [1, 3, 8, 9, 64, 100])
def test_supergroup_gemm(q, b):
    """GEMV (b <= 8) and MFMA (b > 8, ragged token tiles at 9 and 100) forms."""
    rows, cols = 3072, 1024
    w = synth.normal_f32((rows, cols), 0.02, synth.Workload.SUPERGROUP, 0, synth.Role.SUPERGROUP)
    ref, _ = supergroup.quantize(w, 4)
    x = synth.activations(b, cols, synth.Workload.SUPERGROUP, 0, b)
    W_ = q.SuperGroupWeight(dev(ref.p4.view(np.int32)), dev(ref.p2.view(np.int32)), dev(ref.scales),
                            4, rows, cols)
    y = host(q.qlinear_supergroup(dev(x), W_))
    assert_close(y, supergroup.gemm(x, ref), what="supergroup")


@pytest.mark.parametrize("period,rows,cols,b", [(1, 128, 2048, 20), (2, 200, 1024, 33), (3, 96, 3072, 17),
                                                (4, 64, 512, 40)])
def test_supergroup_gemm_shapes(q, period, rows, cols, b):
    """Other periods (all 4-bit at 1), row counts that are not a multiple of 64, K of two
    and three 1024-input chunks, and K = 512 (GEMV form) in batched calls."""
    w = synth.normal_f32((rows, cols), 0.02, synth.Workload.TEST, 21, synth.Role.SUPERGROUP, period)
    ref, _ = supergroup.quantize(w, period)
    x = synth.activations(b, cols, synth.Workload.TEST, 21, period)
    p2 = dev(ref.p2.view(np.int32)) if ref.p2.size else torch.empty(0, dtype=torch.int32, device=DEV)
    W_ = q.SuperGroupWeight(dev(ref.p4.view(np.int32)), p2, dev(ref.scales), period, rows, cols)
    y = host(q.qlinear_supergroup(dev(x), W_))
    assert_close(y, supergroup.gemm(x, ref), what="supergroup")


# ------------------------------------------------------------------------------ super-group, 8-bit activations

def _sg_weight(q, ref, period, rows, cols):
    p2 = dev(ref.p2.view(np.int32)) if ref.p2.size else torch.empty(0, dtype=torch.int32, device=DEV)
    return q.SuperGroupWeight(dev(ref.p4.view(np.int32)), p2, dev(ref.scales), period, rows, cols)


def _check_a8(y, ref64):
    """Within one fp16 step of the oracle (the kernel scales in fp32, the oracle in float64:
    they round to different fp16 values only next to a rounding boundary), and equal almost
    everywhere."""
    r16 = ref64.astype(np.float16)
    assert ulp_distance(y, r16) <= 1
    assert np.mean(y.view(np.uint16) != r16.view(np.uint16)) < 1e-3


@pytest.mark.parametrize("b,cols", [(1, 1024), (5, 512), (64, 1024), (100, 2048), (3, 8192)])
def test_act8_codes_bit_exact(q, b, cols):
    """The integer decisions of the activation quantizer: codes and fp16 scales equal the
    oracle's bit for bit (same fp32 division, ties to even), including an all-zero row (the
    epsilon scale), a row already on an 8-bit grid and a row with one large outlier."""
    x = synth.activations(b, cols, synth.Workload.SUPERGROUP, 1, b)
    x[0, :] = 0
    if b > 2:
        x[1, :] = (np.arange(cols) % 255 - 127) * np.float16(2.0 ** -5)
        x[2, 7] = np.float16(300.0)
    qx, sx = q.quantize_act8(dev(x))
    ref_q, ref_s = supergroup.quantize_activations(x)
    assert np.array_equal(host(sx).view(np.uint16), ref_s.view(np.uint16))
    assert np.array_equal(host(qx), ref_q)


@pytest.mark.parametrize("b", [1, 3, 8, 9, 16, 64, 100])
def test_supergroup_a8_gemm(q, b):
    """The integer path at the benchmark shape (3072 x 1024, rho = 1/4): dot4 form (b <= 8)
    and int8 MFMA form (b > 8; ragged 16-token tiles at 9 and 100)."""
    rows, cols = 3072, 1024
    w = synth.normal_f32((rows, cols), 0.02, synth.Workload.SUPERGROUP, 0, synth.Role.SUPERGROUP)
    ref, _ = supergroup.quantize(w, 4)
    x = synth.activations(b, cols, synth.Workload.SUPERGROUP, 2, b)
    y = host(q.qlinear_supergroup_a8(dev(x), _sg_weight(q, ref, 4, rows, cols)))
    _check_a8(y, supergroup.gemm_a8(x, ref))


@pytest.mark.parametrize("period,rows,cols,b", [(1, 128, 2048, 20), (2, 200, 1024, 33), (3, 96, 3072, 17),
                                                (4, 64, 512, 40), (4, 64, 8192, 2), (4, 192, 4096, 24)])
def test_supergroup_a8_gemm_shapes(q, period, rows, cols, b):
    """Other periods (all 4-bit at 1), row counts that are not a multiple of 64, K of two,
    three and four 1024-input chunks, K = 512 (dot4 form in a batched call) and K = 8192 with
    two tokens per pass of the dot4 form."""
    w = synth.normal_f32((rows, cols), 0.02, synth.Workload.TEST, 22, synth.Role.SUPERGROUP, period)
    ref, _ = supergroup.quantize(w, period)
    x = synth.activations(b, cols, synth.Workload.TEST, 22, period)
    y = host(q.qlinear_supergroup_a8(dev(x), _sg_weight(q, ref, period, rows, cols)))
    _check_a8(y, supergroup.gemm_a8(x, ref))


def test_supergroup_a8_integer_case_exact(q):
    """Activations already on the grid (scale 2^-5: one entry 127 per row, the rest small)
    and unit weight scales: every output is an integer v times 2^-5 with |v| <= 2048, exact
    in fp16, so the result is exact."""
    rows, cols, b = 64, 1024, 12
    w = synth.normal_f32((rows, cols), 0.02, synth.Workload.TEST, 23, synth.Role.SUPERGROUP)
    ref, codes = supergroup.quantize(w, 4)
    ref.scales[:] = np.float16(1.0)
    k = np.random.default_rng(5).integers(-2, 3, size=(b, cols))
    k[:, 0] = 127
    x = (k * 2.0 ** -5).astype(np.float16)
    y = host(q.qlinear_supergroup_a8(dev(x), _sg_weight(q, ref, 4, rows, cols)))
    v = k.astype(np.int64) @ codes.astype(np.int64).T
    assert np.all(np.abs(v) <= 2048)
    exact = v * 2.0 ** -5
    assert np.array_equal(y.astype(np.float64), exact)


# ------------------------------------------------------------------------------ group 32, bf16 parameters

_PD = {"f16": 0, "bf16": 1}


def _qw_g(rows, cols, bits, group, pdt, idx):
    w = synth.normal_f32((rows, cols), 0.02, W, 5, synth.Role.DENSE, idx)
    w[0, :group] = 0.25                          # a constant group: scale 0
    w[1, 3] = 2.0                                # an outlier
    return affine.quantize(w, bits, group, pdt)


def _dev_qw(q, ref):
    return q.QWeight.from_arrays(ref.packed, ref.scales, ref.biases, ref.bits, DEV, group=ref.group,
                                 param_dtype=_PD[ref.param_dtype])


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("shape", [(64, 2048), (7, 512), (33, 1536)])
def test_quantize_group32_bit_exact(q, bits, shape):
    w = special_matrix(*shape, seed=shape[0] + bits)
    ref = affine.quantize(w, bits, 32)
    got = q.quantize_affine(dev(w), bits, group=32)
    assert np.array_equal(host(got.packed).view(np.uint32), ref.packed)
    assert np.array_equal(host(got.scales).view(np.uint16), ref.scales.view(np.uint16))
    assert np.array_equal(host(got.biases).view(np.uint16), ref.biases.view(np.uint16))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("group,pdt", [(32, "f16"), (32, "bf16"), (64, "bf16")])
def test_dequantize_group32_bf16_bit_exact(q, bits, group, pdt):
    """Packed words and parameters taken as given (the import path): the fp32 dequantized
    weights equal the oracle's single rounding of s * q + b bit for bit."""
    ref = _qw_g(96, 1024, bits, group, pdt, 1)
    got = host(q.dequantize(_dev_qw(q, ref)))
    assert np.array_equal(got.view(np.uint32), affine.dequantize_f32(ref).view(np.uint32))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("group,pdt", [(32, "f16"), (32, "bf16"), (64, "bf16")])
@pytest.mark.parametrize("m,rows,cols", [(1, 512, 2048), (5, 96, 1024), (12, 130, 4096)])
def test_qlinear_group32_bf16(q, bits, group, pdt, m, rows, cols):
    """The dense linear on group-32 and/or bf16-parameter weights (the GEMV fast path at
    m <= 8, the general path above), to the float bar; 4-bit within one fp16 step of the
    correctly rounded oracle (8-bit codes enter as 1 + q/256, whose per-group affine terms
    cancel more of the fp32 sum, as with fp16 parameters)."""
    ref = _qw_g(rows, cols, bits, group, pdt, m + rows)
    x = synth.activations(m, cols, W, 5, m)
    y = host(q.qlinear_int4(dev(x), _dev_qw(q, ref)))
    exact = moe.qlinear(x, ref)
    assert_close(y, exact, what="qlinear g32/bf16")
    if bits == 4:
        assert ulp_distance(y, moe.to_f16(exact)) <= 1


def test_qlinear_group32_bf16_with_lora(q):
    rows, cols, T, n_ad, r = 512, 2048, 8, 4, 16
    ref = _qw_g(rows, cols, 4, 32, "bf16", 9)
    A = synth.normal_f16((n_ad, r, cols), 0.01, W, 6, synth.Role.LORA_A_GATE)
    B = synth.normal_f16((n_ad, rows, r), 0.01, W, 6, synth.Role.LORA_B_GATE)
    ad = synth.adapter_index(T, 2)
    x = synth.activations(T, cols, W, 6)
    y = host(q.qlinear_int4(dev(x), _dev_qw(q, ref), q.Lora(dev(A), dev(B), 2.0), dev(ad)))
    assert_close(y, moe.qlinear(x, ref, moe.Lora(A, B, 2.0), ad), what="qlinear g32/bf16 + lora")
