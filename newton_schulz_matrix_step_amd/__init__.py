"""MI355X (gfx950) Muon optimizer step (and the AdamW step of the hybrid
setup's other parameters) behind a C ABI.

The computation lives in ``libmuon_mi355x.so`` (hand-written HIP kernels);
this package is its thin ctypes binding.  PyTorch supplies device memory and
streams only.
"""

from ._abi import (  # noqa: F401
    EXPORTED_SYMBOLS,
    LIB_PATH,
    MUON_BF16,
    MUON_COMPUTE_BF16,
    MUON_COMPUTE_FP32,
    MUON_ERR_DTYPE,
    MUON_ERR_HIP,
    MUON_ERR_INVALID_ARG,
    MUON_ERR_NO_DEVICE,
    MUON_ERR_OOM,
    MUON_F32,
    MUON_INIT_DEBUG,
    MUON_INIT_FAIL_ALLOC,
    MUON_INIT_PROFILE,
    MUON_OK,
    ROLE_NAMES,
    AdamWHparams,
    Hparams,
    MuonError,
    load,
    make_adamw_tensor,
    make_matrix,
    muon_adamw_hparams,
    muon_adamw_step,
    muon_adamw_step_raw,
    muon_adamw_tensor,
    muon_abi_version,
    muon_destroy,
    muon_init,
    muon_kernel_stats_read,
    muon_kernel_stats_reset,
    muon_last_error,
    muon_matrix,
    muon_orthogonalize,
    muon_read_norms,
    muon_status_str,
    muon_step,
    muon_step_noalloc,
    muon_step_raw,
    muon_workspace_bytes,
    profile_roles,
    muon_hparams,
)
