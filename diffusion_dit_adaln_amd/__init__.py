"""Fused adaLN normalisation for MI355X (gfx950): Python binding of ``libadaln``.

The entry points are the C-ABI calls of ``include/adaln.h`` under the same names;
this package only marshals torch tensors (device pointers, strides, the current
HIP stream) into them and turns a non-OK status into an exception.  Every step of
the computation runs in the library's HIP kernels; there is no fallback.
"""
from ._binding import (  # noqa: F401
    ABI_VERSION,
    AdalnError,
    adaln_abi_version,
    adaln_check_layernorm_modulate,
    adaln_check_layernorm_modulate_fp8_quant,
    adaln_check_qk_rmsnorm_rope,
    adaln_check_residual_gate_channel_first,
    adaln_check_residual_gate_layernorm_modulate,
    adaln_check_residual_gate_rmsnorm_scale_shift,
    adaln_check_rmsnorm_scale_shift,
    adaln_diag_device_plan,
    adaln_diag_finalize,
    adaln_diag_launch_plan,
    adaln_diag_quant_fp8,
    adaln_diag_round_bf16,
    adaln_diag_stream,
    adaln_diag_stream_copy,
    adaln_layernorm_modulate,
    adaln_layernorm_modulate_fp8_quant,
    adaln_qk_rmsnorm_rope,
    adaln_reduction_layout,
    adaln_residual_gate_channel_first,
    adaln_residual_gate_layernorm_modulate,
    adaln_residual_gate_rmsnorm_scale_shift,
    adaln_rmsnorm_scale_shift,
    adaln_status_string,
    library_path,
    load_library,
)
