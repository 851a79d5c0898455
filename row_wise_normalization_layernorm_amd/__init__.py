"""MI355X-native row-wise normalization (LayerNorm, RMSNorm): the forward, with
an optional fused residual add, and the backward; float32, binary16 or
bfloat16 rows with float32 statistics.

The compute path is libmi_norm.so (hand-written HIP for gfx950, C ABI in
include/mi_norm.h); this package is its thin Python binding plus the seeded
synthetic workloads used by tests and benchmarks.
"""
from ._binding import (  # noqa: F401
    MI_NORM_ERR_HIP,
    MI_NORM_BF16,
    MI_NORM_ERR_INVALID,
    MI_NORM_F16,
    MI_NORM_F32,
    MI_NORM_OK,
    OP_ADD_LAYERNORM,
    OP_ADD_RMSNORM,
    OP_LAYERNORM,
    OP_LAYERNORM_BWD,
    OP_RMSNORM,
    OP_RMSNORM_BWD,
    BwdProblem,
    bwd_problem,
    layernorm_bwd,
    rmsnorm_bwd,
    mi_layernorm_bwd,
    mi_norm_bwd,
    mi_norm_bwd_check,
    mi_norm_bwd_eligible,
    mi_norm_bwd_noalloc,
    mi_norm_bwd_noalloc_limit,
    mi_norm_bwd_select,
    mi_norm_bwd_variant,
    mi_norm_bwd_workspace_size,
    mi_rmsnorm_bwd,
    MiNormError,
    Problem,
    add_layernorm,
    add_rmsnorm,
    header_functions,
    layernorm,
    lib,
    mi_add_layernorm_fwd,
    mi_add_layernorm_fwd_variant,
    mi_add_rmsnorm_fwd,
    mi_add_rmsnorm_fwd_variant,
    mi_copy_f32,
    mi_calib_launch,
    mi_layernorm_fwd,
    mi_layernorm_fwd_variant,
    mi_norm_check,
    mi_norm_eligible,
    mi_norm_fwd,
    mi_norm_fwd_variant,
    mi_norm_select,
    mi_norm_status_string,
    mi_norm_variant_count,
    mi_norm_variant_get_info,
    mi_norm_variant_name,
    mi_norm_version,
    mi_rmsnorm_fwd,
    mi_rmsnorm_fwd_variant,
    problem,
    rmsnorm,
)


def __getattr__(name):
    # the autograd layer imports torch; load it on first use only
    if name in ("layer_norm", "rms_norm", "LayerNorm", "RMSNorm"):
        from . import autograd
        return getattr(autograd, name)
    raise AttributeError(name)
