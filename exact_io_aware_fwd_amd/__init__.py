"""Fused exact attention for MI355X (gfx950): HIP kernels behind a C ABI (include/fa.h).

    import exact_io_aware_fwd_amd as fa
    o, lse = fa.fwd(q, k, v, causal=True)                 # q [B,Hq,N,d], k/v [B,Hkv,N,d]
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=True)
    o, lse = fa.fwd_splitkv(q_new, k_cache, v_cache, causal=True)   # few queries, long cache
    o, lse = fa.fwd_fp8(*fa.fp8_prepare(q, k, v, signs), causal=True)  # FP8 path
"""
from .binding import (  # noqa: F401
    FA_BF16,
    FA_ERR_HIP,
    FA_ERR_INVALID_ARGUMENT,
    FA_ERR_UNSUPPORTED,
    FA_F16,
    FA_OK,
    FaError,
    block_lists_to_tensors,
    bwd,
    bwd_masked,
    bwd_noalloc,
    bwd_workspace_size,
    declared_symbols,
    fp8_prepare,
    fp8_quantize,
    fp8_quantize_v,
    fwd,
    fwd_fp8,
    fwd_masked,
    fwd_splitkv,
    last_error,
    lse_combine,
    load,
    splitkv_num_splits,
    splitkv_workspace_size,
    status_string,
)
