"""libqlora: the QLoRA frozen-base NF4 LoRA linear layer on AMD CDNA4 (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
include/qlora.h; this package is a thin ctypes binding over it (see _lib.py)
plus the seeded synthetic-input generators (inputs.py).
"""
from ._lib import (  # noqa: F401
    AdamwParam,
    AdamwParamSet,
    Dropout,
    FwdItem,
    NF4Blocked,
    NF4Weight,
    QLORA_MAX_GROUP,
    QLORA_OP_BWD,
    QLORA_OP_BWD_DROPOUT,
    QLORA_OP_FWD,
    QLORA_OP_FWD_DROPOUT,
    QLORA_OP_QUANTIZE,
    QloraError,
    header_functions,
    lib,
    qlora_abi_version,
    qlora_adamw_step,
    qlora_dequant_bf16,
    qlora_dequant_bf16_blocked,
    qlora_dropout_mask,
    qlora_grad_sumsq,
    qlora_sumsq_workspace_bytes,
    qlora_linear_bwd,
    qlora_linear_bwd_dropout,
    qlora_linear_fwd,
    qlora_linear_fwd_dropout,
    qlora_linear_fwd_many,
    qlora_merge_nf4,
    qlora_nf4_blocked_sizes,
    qlora_nf4_sizes,
    qlora_quantize_blocked_workspace_bytes,
    qlora_quantize_nf4,
    qlora_quantize_nf4_blocked,
    qlora_status_string,
    qlora_time_next_weight_kernel,
    qlora_workspace_bytes,
)
