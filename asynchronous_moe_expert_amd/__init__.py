"""MI355X-native expert step of asynchronous expert-parallel MoE serving.

libmoestep.so (HIP kernels for gfx950 behind a C ABI, include/moe_step.h) does the work;
this package binds it (ctypes) and strings the three calls together on one stream.
"""
from ._native import (  # noqa: F401
    ERR_DUPLICATE,
    ERR_EXPERT_NONLOCAL,
    ERR_KSLOT_RANGE,
    ERR_ROW_RANGE,
    ERR_SLOT_RANGE,
    ERR_STALE_GEN,
    ERR_TOKEN_RANGE,
    EXPORTS,
    LIB_PATH,
    MOE_BF16,
    MOE_F32,
    MOE_FP8_E4M3,
    CombineState,
    MoeError,
    combine_args,
    combine_call,
    load,
    moe_assemble,
    moe_combine_noalloc_max_arrivals,
    moe_combine_release,
    moe_combine_workspace_size,
    moe_expert_ffn_grouped,
    moe_ffn_workspace_size,
    moe_pack_ffn_weights,
    moe_state_reset,
    moe_strerror,
    moe_version,
)
from .step import ExpertStep, SharedExpert  # noqa: F401
