"""Fused exact attention for MI355X (gfx950): HIP kernels behind a C ABI (include/fa.h).

    import exact_io_aware_fwd_amd as fa
    o, lse = fa.fwd(q, k, v, causal=True)                 # q [B,Hq,N,d], k/v [B,Hkv,N,d]
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=True)
"""
from .binding import (  # noqa: F401
    FA_BF16,
    FA_ERR_HIP,
    FA_ERR_INVALID_ARGUMENT,
    FA_ERR_UNSUPPORTED,
    FA_F16,
    FA_OK,
    FaError,
    bwd,
    bwd_workspace_size,
    declared_symbols,
    fwd,
    last_error,
    load,
    status_string,
)
