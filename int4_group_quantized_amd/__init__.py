"""MI355X-native int4 group-quantized MoE SwitchGLU layer with unmerged LoRA.

A thin Python binding over libqmoe.so (include/qmoe.h): group-wise affine int4/8-bit
quantization, the quantized linear, router top-K, LoRA delta, the MoE SwitchGLU layer and
the mixed ternary/4-bit super-group GEMM, all computed by hand-written gfx950 HIP
kernels.  Importing the package requires the built library (see build.py).
"""
from ._lib import LIB_PATH, EXPORTED, QmoeError, lib  # noqa: F401
from .api import (  # noqa: F401
    Lora,
    PARAM_BF16,
    PARAM_F16,
    MoECall,
    STAGE_ALL,
    STAGE_DOWN,
    STAGE_GATE_UP,
    STAGE_ROUTE,
    MoELayer,
    QWeight,
    PrerouterHead,
    prerouter_forward,
    SuperGroupWeight,
    dequantize,
    lora_apply,
    moe_switchglu_int4,
    moe_switchglu_int4_noalloc,
    moe_switchglu_int4_routed,
    moe_workspace,
    moe_workspace_bytes,
    qlinear_int4,
    qlinear_supergroup,
    qlinear_supergroup_a8,
    quantize_act8,
    quantize_affine,
    quantize_supergroup,
    router_topk,
    unpack,
)
