"""Switch top-1 mixture-of-experts layer (forward and backward) for AMD Instinct MI355X (gfx950).

The computation lives in libswitch_moe.so (hand-written HIP kernels behind the
C ABI of include/switch_moe.h); this package only builds and binds it.
"""
from .native import (  # noqa: F401
    BF16, EXPERT_CHOICE, F32, GATE_DESC, GATE_SCALE, RENORM, RESIDUAL_ALL, TOKEN_CHOICE, TOKEN_ORDER, StageEvents, SwitchError, SwitchMoE, lib,
    switch_assign_capacity,
    switch_capacity, switch_combine, switch_dispatch, switch_expert_ffn, switch_moe_backward, switch_moe_forward,
    switch_moe_forward_train, switch_quantize_mxfp4, switch_route,
)
