"""MI355X-native (gfx950) TTT layers.

The compute runs in libttt.so (C ABI, include/ttt.h): hand-written HIP kernels for the
TTT-Linear, TTT-MLP and delta-rule forward passes (plain inner models, and the paper's with
layer norm and residual) and the TTT-Linear and TTT-MLP backward passes (causal and
non-causal).  This package holds the ctypes
binding (argument marshalling only), the in-tree build script and the seeded synthetic
workloads.
"""
from ._binding import (  # noqa: F401
    LIB_PATH,
    SIGNATURES,
    TTT_BF16,
    TTT_E_HIP,
    TTT_E_INVALID,
    TTT_E_NONFINITE,
    TTT_E_UNSUPPORTED,
    TTT_F32,
    TTT_OK,
    TTTError,
    delta_rule_fwd,
    get_check_finite,
    last_error,
    load_library,
    set_check_finite,
    set_split_debug,
    ttt_linear_bwd,
    ttt_linear_bwd_noalloc,
    ttt_linear_fwd,
    ttt_linear_ln_bwd,
    ttt_linear_ln_fwd,
    ttt_linear_nc_bwd,
    ttt_mlp_bwd,
    ttt_mlp_fwd,
    ttt_mlp_fwd_workspace_size,
    ttt_mlp_fwd_ws,
    ttt_mlp_ln_bwd,
    ttt_mlp_ln_fwd,
    ttt_mlp_ln_fwd_ws,
    ttt_mlp_nc_bwd,
)
