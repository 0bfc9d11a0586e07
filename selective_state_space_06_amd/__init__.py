"""libmamba_scan: Mamba's selective state-space scan (S6) and its one-token decode step,
hand-written in HIP for AMD Instinct MI355X (gfx950), behind the C ABI of
include/mamba_scan.h.  This package is the thin Python binding (ctypes + torch for device
memory and streams); every step of the computation runs in the HIP kernels.
"""
from ._binding import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    MSS_BF16,
    MSS_F32,
    MSS_I32,
    MssError,
    causal_conv1d_fwd,
    causal_conv1d_update,
    conv1d_fwd_raw,
    conv1d_update_raw,
    Tensor,
    load_library,
    profile_enable,
    profile_fwd,
    scan_bwd_raw,
    scan_bwd_varlen_raw,
    scan_fwd_raw,
    scan_fwd_varlen_raw,
    scan_fwd_with_state_raw,
    selective_scan_bwd,
    selective_scan_fwd,
    selective_scan_fwd_varlen,
    selective_scan_fwd_with_state,
    selective_state_update,
    state_update_raw,
    status_string,
    version,
)
