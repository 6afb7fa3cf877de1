"""Block-sparse attention backward (and the forward it differentiates) for AMD MI355X (gfx950).

The compute lives in ``libbsa_bwd.so`` (hand-written HIP kernels behind the C
ABI of ``include/bsa_bwd.h``); this package only marshals torch tensors into
that ABI.  See ``_binding`` for the functions, which keep the C names.
"""
from ._binding import (  # noqa: F401
    BSA_DTYPE_BF16,
    BSA_DTYPE_BOOL,
    BSA_DTYPE_F16,
    BSA_DTYPE_F32,
    BSA_DTYPE_FP8_E4M3FN,
    BSA_DTYPE_FP8_E5M2,
    BSA_ERR_INNER,
    BSA_ERR_PARAM_INVALID,
    BSA_ERR_PARAM_NULLPTR,
    BSA_ERR_RUNTIME,
    BSA_OK,
    LIB_PATH,
    NO_WINDOW,
    WS_REGIONS,
    BsaError,
    block_sparse_attention,
    block_sparse_attention_grad,
    bsa_bwd,
    bsa_bwd_fp8,
    bsa_bwd_fp8_workspace_size,
    bsa_bwd_noalloc,
    bsa_bwd_workspace_layout,
    bsa_bwd_workspace_size,
    bsa_fwd,
    bsa_fwd_fp8,
    bsa_fwd_fp8_workspace_size,
    bsa_fwd_workspace_size,
    bsa_last_error,
    bsa_profile_start,
    bsa_profile_stop,
    bsa_stage_name,
    bsa_tensor,
    header_functions,
    load_library,
)
