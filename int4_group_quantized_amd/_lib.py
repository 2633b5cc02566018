"""ctypes loader for libqmoe.so and the C structs of include/qmoe.h.

The library is required: importing this module without a built libqmoe.so raises
ImportError (there is no fallback of any kind).

torch is imported before the library is opened: torch ships its own HIP runtime
(libamdhip64, soname libamdhip64.so.7), and libqmoe.so's dependency on that soname must
resolve to the copy torch already loaded, so that both use one runtime — the same device
memory, streams and kernel registry.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede loading libqmoe.so, see above)

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqmoe.so")

QMOE_OK = 0
QMOE_ERR_INVALID_ARG = -1
QMOE_ERR_UNSUPPORTED = -2
QMOE_ERR_MISALIGNED = -3
QMOE_ERR_WORKSPACE = -4
QMOE_ERR_HIP = -5
NOALLOC_SCRATCH_BYTES = 32 << 20   # QMOE_NOALLOC_SCRATCH_BYTES of include/qmoe.h


class QWeightC(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("biases", ctypes.c_void_p), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("param_dtype", ctypes.c_int32)]


class PrerouterC(ctypes.Structure):
    _fields_ = [("w_init", ctypes.c_void_p), ("b_init", ctypes.c_void_p), ("w1", ctypes.c_void_p),
                ("b1", ctypes.c_void_p), ("w2", ctypes.c_void_p), ("b2", ctypes.c_void_p),
                ("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("ffn", ctypes.c_int32)]


class LoraC(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("rank", ctypes.c_int32),
                ("n_adapters", ctypes.c_int32), ("in_dim", ctypes.c_int32),
                ("out_dim", ctypes.c_int32), ("scale", ctypes.c_float)]


class MoELayerC(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("add_residual", ctypes.c_int32),
                ("router", QWeightC), ("shared_gate", QWeightC), ("exp_gate", QWeightC),
                ("exp_up", QWeightC), ("exp_down", QWeightC), ("sh_gate", QWeightC),
                ("sh_up", QWeightC), ("sh_down", QWeightC),
                ("lora_gate", ctypes.POINTER(LoraC)), ("lora_up", ctypes.POINTER(LoraC)),
                ("lora_down", ctypes.POINTER(LoraC)), ("router_bias", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIGS = {
    "qmoe_abi_version": (ctypes.c_int, []),
    "qmoe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "qmoe_abi_struct_size": (ctypes.c_size_t, [ctypes.c_int]),
    "qmoe_last_error": (ctypes.c_char_p, []),
    "qmoe_quantize_affine": (ctypes.c_int, [_P, _I, _I, _I, _I, _P, _P, _P, _P]),
    "qmoe_unpack": (ctypes.c_int, [_P, _I, _I, _I, _P, _P]),
    "qmoe_dequantize": (ctypes.c_int, [ctypes.POINTER(QWeightC), _P, _P]),
    "qlinear_int4": (ctypes.c_int, [_P, _I, ctypes.POINTER(QWeightC), ctypes.POINTER(LoraC), _P, _P, _P]),
    "router_topk": (ctypes.c_int, [_P, _I, _I, _I, _P, _P, _P, _P]),
    "lora_apply": (ctypes.c_int, [_P, _I, ctypes.POINTER(LoraC), _P, _P, _P]),
    "moe_switchglu_int4_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(MoELayerC), _I]),
    "moe_switchglu_int4": (ctypes.c_int, [ctypes.POINTER(MoELayerC), _P, _I, _P, _P, _P, _P, _P,
                                          ctypes.c_size_t, _P]),
    "moe_switchglu_int4_stage": (ctypes.c_int, [ctypes.POINTER(MoELayerC), _I, _P, _I, _P, _P, _P,
                                                _P, _P, ctypes.c_size_t, _P]),
    "moe_switchglu_int4_noalloc": (ctypes.c_int, [ctypes.POINTER(MoELayerC), _P, _I, _P, _P, _P, _P, _P]),
    "moe_switchglu_int4_routed": (ctypes.c_int, [ctypes.POINTER(MoELayerC), _P, _I, _P, _P, _P, _P, _P,
                                                 ctypes.c_size_t, _P]),
    "qmoe_quantize_supergroup": (ctypes.c_int, [_P, _I, _I, _I, _P, _P, _P, _P]),
    "qlinear_supergroup": (ctypes.c_int, [_P, _I, _P, _P, _P, _I, _I, _I, _P, _P]),
    "qmoe_quantize_act8": (ctypes.c_int, [_P, _I, _I, _P, _P, _P]),
    "prerouter_forward": (ctypes.c_int, [ctypes.POINTER(PrerouterC), _P, _I, _I, _P, _P, _P, _P, _P, _P, _P]),
    "qlinear_supergroup_a8": (ctypes.c_int, [_P, _I, _P, _P, _P, _I, _I, _I, _P, _P]),
}
EXPORTED = tuple(_SIGS)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m int4_group_quantized_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    for which, cls in enumerate((QWeightC, LoraC, MoELayerC, PrerouterC)):
        if lib.qmoe_abi_struct_size(which) != ctypes.sizeof(cls):
            raise ImportError(f"ABI struct {cls.__name__} size mismatch with {LIB_PATH}")
    return lib


lib = _load()


class QmoeError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        msg = lib.qmoe_status_string(status).decode()
        if status == QMOE_ERR_HIP:
            msg += ": " + lib.qmoe_last_error().decode()
        super().__init__(f"{call} failed: {msg} ({status})")


def check(status: int, call: str) -> None:
    if status != QMOE_OK:
        raise QmoeError(status, call)
