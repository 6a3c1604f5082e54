"""Exact attention for AMD MI355X (gfx950): C-ABI library + thin binding.

The computation lives in libfa.so (hand-written HIP kernels, see csrc/); this
package only marshals torch tensors into its C calls (fa.py) and provides the
seeded synthetic input generator (inputs.py).
"""
from .fa import (  # noqa: F401
    FA_BF16, FA_FP16, FA_FP32, FA_OK, FA_ERR_HIP, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED,
    LIB_PATH, default_scale, fa_bwd, fa_bwd_ex, fa_bwd_ex_workspace_bytes, fa_bwd_workspace_bytes,
    fa_fwd, fa_fwd_ex, fa_last_error_detail, fa_status_string, fa_version, load_library,
)
