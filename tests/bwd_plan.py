"""fa_bwd's dK/dV plan, written out from its documented rule (include/fa.h, fa_bwd and
fa_bwd_workspace_size): dK/dV records of 256 or 128 keys, and the chunks each record's
query steps are split into.  Tests use it to assert which path a shape takes."""
from __future__ import annotations


def dense_plan(B: int, Hq: int, Hkv: int, N: int, causal: bool) -> tuple[int, int]:
    """(keys per record, chunks per record): chunks enough to give the CUs 256 (512 when
    causal) workgroups, at most 16, each at least 32 query steps of the longest record
    (256 for 256-key records); 256-key records when they reach that target alone or give
    as many workgroups as 128-key records would."""
    steps = (Hq // Hkv) * -(-N // 32)
    target = 512 if causal else 256

    def chunks(r, m):
        return max(min(target // r, 16, steps // m), 1)

    r256, r128 = B * Hkv * -(-N // 256), B * Hkv * -(-N // 128)
    if r256 >= target or r256 * chunks(r256, 256) >= r128 * chunks(r128, 32):
        return 256, chunks(r256, 256)
    return 128, chunks(r128, 32)


def rowterm_bytes(B: int, Hq: int, N: int) -> int:
    """The row-term part of the workspace: two fp32 values per query row, rows padded to 32."""
    return B * Hq * -(-N // 32) * 32 * 8
