"""The C-ABI library loads, exports every entry point its header declares, agrees with the
binding on struct layout, and rejects bad arguments before touching the GPU (CPU only:
every call here fails validation, so nothing is launched)."""
import ctypes
import os
import re

import pytest

import int4_group_quantized_amd as q
from int4_group_quantized_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "qmoe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("qlinear_int4", "moe_switchglu_int4", "lora_apply", "router_topk"):
        assert n in names


def test_every_declared_function_is_exported():
    lib = ctypes.CDLL(q.LIB_PATH)
    names = declared_functions()
    assert len(names) == 20
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTED)


def test_version_status_and_struct_layout():
    assert q.lib.qmoe_abi_version() == 1
    assert q.lib.qmoe_status_string(0) == b"ok"
    assert q.lib.qmoe_status_string(-4) == b"workspace missing or too small"
    assert q.lib.qmoe_abi_struct_size(0) == ctypes.sizeof(_lib.QWeightC)
    assert q.lib.qmoe_abi_struct_size(1) == ctypes.sizeof(_lib.LoraC)
    assert q.lib.qmoe_abi_struct_size(2) == ctypes.sizeof(_lib.MoELayerC)
    assert q.lib.qmoe_abi_struct_size(3) == ctypes.sizeof(_lib.PrerouterC)
    assert q.lib.qmoe_abi_struct_size(7) == 0


FAKE = 0x100000  # a 16-byte aligned fake device address; never dereferenced (validation fails first)


def qw(rows=512, cols=2048, bits=4, n_experts=1, packed=FAKE, group=64, param_dtype=0):
    return _lib.QWeightC(packed, FAKE, FAKE, rows, cols, bits, group, n_experts, param_dtype)


def test_quantize_rejects_bad_arguments():
    f = q.lib.qmoe_quantize_affine
    assert f(None, 4, 64, 4, 64, FAKE, FAKE, FAKE, None) == _lib.QMOE_ERR_INVALID_ARG
    assert f(FAKE, 0, 64, 4, 64, FAKE, FAKE, FAKE, None) == _lib.QMOE_ERR_INVALID_ARG
    assert f(FAKE, 4, 64, 3, 64, FAKE, FAKE, FAKE, None) == _lib.QMOE_ERR_UNSUPPORTED
    assert f(FAKE, 4, 64, 4, 16, FAKE, FAKE, FAKE, None) == _lib.QMOE_ERR_UNSUPPORTED
    assert f(FAKE, 4, 96, 4, 64, FAKE, FAKE, FAKE, None) == _lib.QMOE_ERR_UNSUPPORTED
    assert f(FAKE + 4, 4, 64, 4, 64, FAKE, FAKE, FAKE, None) == _lib.QMOE_ERR_MISALIGNED


def test_qlinear_rejects_bad_arguments():
    f = q.lib.qlinear_int4
    w = qw()
    assert f(None, 1, ctypes.byref(w), None, None, FAKE, None) == _lib.QMOE_ERR_INVALID_ARG
    assert f(FAKE, 0, ctypes.byref(w), None, None, FAKE, None) == _lib.QMOE_ERR_INVALID_ARG
    assert f(FAKE, 5000, ctypes.byref(w), None, None, FAKE, None) == _lib.QMOE_ERR_UNSUPPORTED
    bad = qw(cols=1000)
    assert f(FAKE, 1, ctypes.byref(bad), None, None, FAKE, None) == _lib.QMOE_ERR_UNSUPPORTED
    bad = qw(bits=2)
    assert f(FAKE, 1, ctypes.byref(bad), None, None, FAKE, None) == _lib.QMOE_ERR_UNSUPPORTED
    bad = qw(packed=FAKE + 8)
    assert f(FAKE, 1, ctypes.byref(bad), None, None, FAKE, None) == _lib.QMOE_ERR_MISALIGNED
    assert f(FAKE, 1, ctypes.byref(w), None, None, FAKE + 2, None) == _lib.QMOE_ERR_MISALIGNED
    lo = _lib.LoraC(FAKE, FAKE, 65, 1, 2048, 512, 2.0)
    assert f(FAKE, 1, ctypes.byref(w), ctypes.byref(lo), None, FAKE * 8, None) == _lib.QMOE_ERR_UNSUPPORTED
    lo = _lib.LoraC(FAKE, FAKE, 16, 1, 1024, 512, 2.0)
    assert f(FAKE, 1, ctypes.byref(w), ctypes.byref(lo), None, FAKE * 8, None) == _lib.QMOE_ERR_INVALID_ARG
    # output overlapping the input
    assert f(FAKE, 1, ctypes.byref(w), None, None, FAKE + 16, None) == _lib.QMOE_ERR_INVALID_ARG
    # group 32 / bf16 parameters are accepted by the dense linear's validation, other values not
    for bad in (qw(group=16), qw(group=128), qw(param_dtype=2)):
        assert f(FAKE, 1, ctypes.byref(bad), None, None, FAKE * 8, None) == _lib.QMOE_ERR_UNSUPPORTED


def test_router_topk_rejects_bad_arguments():
    f = q.lib.router_topk
    assert f(None, 1, 256, 4, None, FAKE, FAKE, None) == _lib.QMOE_ERR_INVALID_ARG
    assert f(FAKE, 1, 256, 0, None, FAKE, FAKE, None) == _lib.QMOE_ERR_INVALID_ARG
    assert f(FAKE, 1, 256, 33, None, FAKE, FAKE, None) == _lib.QMOE_ERR_UNSUPPORTED
    assert f(FAKE, 1, 2048, 4, None, FAKE, FAKE, None) == _lib.QMOE_ERR_UNSUPPORTED
    assert f(FAKE, 1, 4, 5, None, FAKE, FAKE, None) == _lib.QMOE_ERR_UNSUPPORTED


def test_lora_apply_rejects_bad_arguments():
    f = q.lib.lora_apply
    lo = _lib.LoraC(FAKE, FAKE, 16, 1, 2048, 512, 2.0)
    assert f(None, 1, ctypes.byref(lo), None, FAKE, None) == _lib.QMOE_ERR_INVALID_ARG
    bad = _lib.LoraC(FAKE, FAKE, 0, 1, 2048, 512, 2.0)
    assert f(FAKE, 1, ctypes.byref(bad), None, FAKE, None) == _lib.QMOE_ERR_INVALID_ARG
    bad = _lib.LoraC(FAKE, FAKE, 16, 1, 1000, 512, 2.0)
    assert f(FAKE, 1, ctypes.byref(bad), None, FAKE, None) == _lib.QMOE_ERR_UNSUPPORTED


def layer_c(**kw):
    H, I, E = 2048, 512, 256
    d = dict(hidden=H, inter=I, shared_inter=512, n_experts=E, top_k=4, add_residual=0,
             router=qw(E, H, 8), shared_gate=qw(1, H, 8), exp_gate=qw(I, H, 4, E),
             exp_up=qw(I, H, 4, E), exp_down=qw(H, I, 4, E), sh_gate=qw(512, H), sh_up=qw(512, H),
             sh_down=qw(H, 512))
    d.update(kw)
    return _lib.MoELayerC(**d)


def test_moe_workspace_and_validation():
    L = layer_c()
    ws1 = q.lib.moe_switchglu_int4_workspace_bytes(ctypes.byref(L), 1)
    ws512 = q.lib.moe_switchglu_int4_workspace_bytes(ctypes.byref(L), 512)
    assert 0 < ws1 < ws512
    assert q.lib.moe_switchglu_int4_workspace_bytes(ctypes.byref(L), 0) == 0
    f = q.lib.moe_switchglu_int4
    X, Y = FAKE, FAKE * 16
    assert f(ctypes.byref(L), X, 1, None, Y, None, None, None, 0, None) == _lib.QMOE_ERR_WORKSPACE
    assert f(ctypes.byref(L), X, 1, None, Y, None, None, FAKE * 64, ws1 - 1, None) == _lib.QMOE_ERR_WORKSPACE
    assert f(ctypes.byref(L), X, 1, None, Y, None, None, FAKE * 64 + 16, ws1, None) == _lib.QMOE_ERR_MISALIGNED
    assert f(ctypes.byref(L), X, 1, None, X, None, None, FAKE * 64, ws1, None) == _lib.QMOE_ERR_INVALID_ARG
    for bad in (layer_c(top_k=0), layer_c(top_k=300), layer_c(hidden=1000),
                layer_c(router=qw(256, 2048, 4)), layer_c(exp_down=qw(512, 2048, 4, 256)),
                layer_c(n_experts=2000), layer_c(exp_gate=qw(512, 2048, 4, 256, group=32)),
                layer_c(sh_up=qw(512, 2048, param_dtype=1))):
        st = f(ctypes.byref(bad), X, 1, None, Y, None, None, FAKE * 64, 1 << 30, None)
        assert st in (_lib.QMOE_ERR_INVALID_ARG, _lib.QMOE_ERR_UNSUPPORTED), st
    lo = _lib.LoraC(FAKE, FAKE, 16, 4, 2048, 1024, 2.0)  # wrong out_dim for the shared gate
    bad = layer_c(lora_gate=ctypes.pointer(lo))
    assert f(ctypes.byref(bad), X, 1, None, Y, None, None, FAKE * 64, 1 << 30, None) == _lib.QMOE_ERR_INVALID_ARG


def test_moe_workspace_grows_with_the_token_count():
    """A workspace sized for max_tokens serves every smaller call: the size never drops as the
    token count grows, across the changes of split and work-item size (every T to 4096)."""
    L = layer_c()
    sizes = [q.lib.moe_switchglu_int4_workspace_bytes(ctypes.byref(L), t) for t in range(1, 4097)]
    assert all(b >= a for a, b in zip(sizes, sizes[1:]))


def test_supergroup_rejects_bad_arguments():
    f = q.lib.qlinear_supergroup
    assert f(FAKE, 1, FAKE, FAKE, FAKE, 3070, 1024, 4, FAKE * 4, None) == _lib.QMOE_ERR_UNSUPPORTED
    assert f(FAKE, 1, FAKE, None, FAKE, 3072, 1024, 4, FAKE * 4, None) == _lib.QMOE_ERR_INVALID_ARG
    assert f(FAKE, 1, FAKE, FAKE, FAKE, 3072, 1000, 4, FAKE * 4, None) == _lib.QMOE_ERR_UNSUPPORTED
    g = q.lib.qmoe_quantize_supergroup
    assert g(FAKE, 3072, 1024, 0, FAKE, FAKE, FAKE, None) == _lib.QMOE_ERR_INVALID_ARG
    assert g(FAKE, 3072, 1024, 5, FAKE, FAKE, FAKE, None) == _lib.QMOE_ERR_UNSUPPORTED


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(TypeError):
        q.quantize_affine(torch.zeros(4, 64))


def test_integer_path_rejects_bad_arguments():
    f = q.lib.qmoe_quantize_act8
    assert f(None, 1, 1024, FAKE, FAKE, None) == _lib.QMOE_ERR_INVALID_ARG
    assert f(FAKE, 0, 1024, FAKE, FAKE, None) == _lib.QMOE_ERR_INVALID_ARG
    assert f(FAKE, 1, 1000, FAKE, FAKE, None) == _lib.QMOE_ERR_UNSUPPORTED
    assert f(FAKE + 2, 1, 1024, FAKE, FAKE, None) == _lib.QMOE_ERR_MISALIGNED
    g = q.lib.qlinear_supergroup_a8
    assert g(FAKE, 1, FAKE, FAKE, FAKE, 3070, 1024, 4, FAKE * 4, None) == _lib.QMOE_ERR_UNSUPPORTED
    assert g(FAKE, 1, FAKE, None, FAKE, 3072, 1024, 4, FAKE * 4, None) == _lib.QMOE_ERR_INVALID_ARG
    assert g(FAKE, 1, FAKE, FAKE, FAKE, 3072, 1000, 4, FAKE * 4, None) == _lib.QMOE_ERR_UNSUPPORTED
    assert g(FAKE, 5000, FAKE, FAKE, FAKE, 3072, 1024, 4, FAKE * 4, None) == _lib.QMOE_ERR_UNSUPPORTED
    assert g(FAKE + 8, 1, FAKE, FAKE, FAKE, 3072, 1024, 4, FAKE * 4, None) == _lib.QMOE_ERR_MISALIGNED


def test_prerouter_rejects_bad_arguments():
    f = q.lib.prerouter_forward
    P = _lib.PrerouterC(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2048, 256, 512)
    X, A, L = FAKE * 2, FAKE * 4, FAKE * 8
    assert f(None, X, 1, 4, FAKE, FAKE, A, L, None, None, None) == _lib.QMOE_ERR_INVALID_ARG
    assert f(ctypes.byref(P), X, 0, 4, FAKE, FAKE, A, L, None, None, None) == _lib.QMOE_ERR_INVALID_ARG
    assert f(ctypes.byref(P), X, 1, 4, FAKE, FAKE, A, L, FAKE, None, None) == _lib.QMOE_ERR_INVALID_ARG
    assert f(ctypes.byref(P), X, 1, 33, FAKE, FAKE, A, L, None, None, None) == _lib.QMOE_ERR_UNSUPPORTED
    for bad in (_lib.PrerouterC(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2000, 256, 512),
                _lib.PrerouterC(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2048, 254, 512),
                _lib.PrerouterC(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2048, 256, 500)):
        assert f(ctypes.byref(bad), X, 1, 4, FAKE, FAKE, A, L, None, None, None) == _lib.QMOE_ERR_UNSUPPORTED
    assert f(ctypes.byref(P), X + 2, 1, 4, FAKE, FAKE, A, L, None, None, None) == _lib.QMOE_ERR_MISALIGNED


def test_header_is_plain_c(tmp_path):
    """include/qmoe.h is a C header: a C99 translation unit that includes it and takes the
    address of every declared function compiles with gcc (no C++ or HIP types leak in)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = tmp_path / "abi.c"
    refs = "\n".join(f"    (entry)&{n}," for n in declared_functions())
    src.write_text('#include "qmoe.h"\ntypedef void (*entry)(void);\nentry qmoe_entry_points[] = {\n'
                   + refs + "\n};\n")
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-I",
                        os.path.dirname(HEADER), "-c", str(src), "-o", str(tmp_path / "abi.o")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_package_fails_loudly_without_the_library(tmp_path):
    """With the built library absent the package does not import (no CPU or oracle fallback):
    a copy of the Python sources without libqmoe.so raises ImportError on import."""
    import shutil
    import subprocess
    import sys
    pkg = os.path.dirname(q.__file__)
    dst = tmp_path / "int4_group_quantized_amd"
    dst.mkdir()
    for f in os.listdir(pkg):
        if f.endswith(".py"):
            shutil.copy(os.path.join(pkg, f), dst / f)
    r = subprocess.run([sys.executable, "-c", "import int4_group_quantized_amd"], cwd=tmp_path,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "ImportError" in r.stderr and "not built" in r.stderr


def test_moe_rejects_misaligned_parameters_and_index_arrays():
    """Scales and biases are read with 16-byte loads and are checked like the packed words;
    the int32/fp32 routing outputs, adapter indices and router bias must be 4-byte aligned."""
    f = q.lib.moe_switchglu_int4
    X, Y, WS = FAKE, FAKE * 16, FAKE * 64
    ok = layer_c()
    ws1 = q.lib.moe_switchglu_int4_workspace_bytes(ctypes.byref(ok), 1)
    mis_s = _lib.QWeightC(FAKE, FAKE + 8, FAKE, 512, 2048, 4, 64, 256, 0)
    mis_b = _lib.QWeightC(FAKE, FAKE, FAKE + 2, 2048, 512, 4, 64, 256, 0)
    for bad in (layer_c(exp_gate=mis_s), layer_c(exp_down=mis_b), layer_c(router_bias=FAKE + 2)):
        assert f(ctypes.byref(bad), X, 1, None, Y, None, None, WS, ws1, None) == _lib.QMOE_ERR_MISALIGNED
    for idx, w, ad in ((FAKE + 2, None, None), (None, FAKE + 1, None), (None, None, FAKE + 3)):
        assert f(ctypes.byref(ok), X, 1, ad, Y, idx, w, WS, ws1, None) == _lib.QMOE_ERR_MISALIGNED
    g = q.lib.qlinear_int4
    w = _lib.QWeightC(FAKE, FAKE + 4, FAKE, 512, 2048, 4, 64, 1, 0)
    assert g(FAKE, 1, ctypes.byref(w), None, None, FAKE * 8, None) == _lib.QMOE_ERR_MISALIGNED


def test_noalloc_rejects_what_its_scratch_cannot_hold():
    """The allocation-free call validates like the layer call and rejects a token count whose
    workspace exceeds the fixed scratch (QMOE_NOALLOC_SCRATCH_BYTES) before any device work."""
    f = q.lib.moe_switchglu_int4_noalloc
    L = layer_c()
    X, Y = FAKE, FAKE * 4096
    assert q.lib.moe_switchglu_int4_workspace_bytes(ctypes.byref(L), 512) <= _lib.NOALLOC_SCRATCH_BYTES
    assert q.lib.moe_switchglu_int4_workspace_bytes(ctypes.byref(L), 1024) > _lib.NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(L), X, 1024, None, Y, None, None, None) == _lib.QMOE_ERR_WORKSPACE
    assert b"scratch" in q.lib.qmoe_last_error()
    assert f(ctypes.byref(L), None, 1, None, Y, None, None, None) == _lib.QMOE_ERR_INVALID_ARG
    assert f(ctypes.byref(L), X, 1, None, X, None, None, None) == _lib.QMOE_ERR_INVALID_ARG
    assert f(ctypes.byref(L), X + 2, 1, None, Y, None, None, None) == _lib.QMOE_ERR_MISALIGNED
    assert f(ctypes.byref(layer_c(top_k=0)), X, 1, None, Y, None, None, None) == _lib.QMOE_ERR_INVALID_ARG


def test_routed_call_validates_like_the_layer_call():
    f = q.lib.moe_switchglu_int4_routed
    L = layer_c()
    ws1 = q.lib.moe_switchglu_int4_workspace_bytes(ctypes.byref(L), 1)
    X, Y, R, WS = FAKE, FAKE * 16, FAKE * 32, FAKE * 64
    assert f(ctypes.byref(L), X, 1, None, None, Y, None, WS, ws1, None) == _lib.QMOE_ERR_INVALID_ARG
    assert f(ctypes.byref(L), X, 1, None, R + 2, Y, None, WS, ws1, None) == _lib.QMOE_ERR_MISALIGNED
    assert f(ctypes.byref(L), X, 1, None, R, Y, None, WS, ws1 - 1, None) == _lib.QMOE_ERR_WORKSPACE
    assert f(ctypes.byref(L), X, 1, None, R, X, None, WS, ws1, None) == _lib.QMOE_ERR_INVALID_ARG
    assert f(ctypes.byref(layer_c(top_k=0)), X, 1, None, R, Y, None, WS, ws1, None) == _lib.QMOE_ERR_INVALID_ARG


def test_moe_takes_the_port_format_for_its_routed_experts():
    """Routed expert stacks may be group 32 and/or bf16 parameters (one format for all three,
    hidden and inter 512, 1024 or 2048); the router, shared gate and shared expert may not."""
    ws = q.lib.moe_switchglu_int4_workspace_bytes
    H, I, E = 2048, 512, 256
    for group, pdt in ((32, 1), (32, 0), (64, 1)):
        L = layer_c(exp_gate=qw(I, H, 4, E, group=group, param_dtype=pdt),
                    exp_up=qw(I, H, 4, E, group=group, param_dtype=pdt),
                    exp_down=qw(H, I, 4, E, group=group, param_dtype=pdt))
        assert ws(ctypes.byref(L), 1) > 0, (group, pdt)
    mixed = layer_c(exp_gate=qw(I, H, 4, E, group=32, param_dtype=1), exp_up=qw(I, H, 4, E, group=32, param_dtype=1),
                    exp_down=qw(H, I, 4, E, group=32, param_dtype=0))
    wide = layer_c(hidden=1536, router=qw(E, 1536, 8), shared_gate=qw(1, 1536, 8),
                   exp_gate=qw(I, 1536, 4, E, group=32), exp_up=qw(I, 1536, 4, E, group=32),
                   exp_down=qw(1536, I, 4, E, group=32), sh_gate=qw(512, 1536), sh_up=qw(512, 1536),
                   sh_down=qw(1536, 512))
    std_wide = layer_c(hidden=1536, router=qw(E, 1536, 8), shared_gate=qw(1, 1536, 8),
                       exp_gate=qw(I, 1536, 4, E), exp_up=qw(I, 1536, 4, E), exp_down=qw(1536, I, 4, E),
                       sh_gate=qw(512, 1536), sh_up=qw(512, 1536), sh_down=qw(1536, 512))
    assert ws(ctypes.byref(std_wide), 1) > 0
    for bad in (mixed, wide, layer_c(router=qw(E, H, 8, group=32)), layer_c(sh_down=qw(H, 512, param_dtype=1))):
        assert ws(ctypes.byref(bad), 1) == 0
