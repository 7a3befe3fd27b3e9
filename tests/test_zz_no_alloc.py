"""GPU test of fa_bwd_noalloc, the backward whose workspace is the library's static device
scratch (for callers that cannot allocate): through the C ABI, two calls in a row on one
stream, the second with smaller inputs, each equal bit for bit to fa_bwd with a caller
workspace on the same inputs (the same kernels and plan, so the same bits), and the
smaller one also within the oracle's tolerance (dQ/dK/dV rel-L2 <= 1e-2).  The first
call takes a split dK/dV plan (fp32 partials in the scratch), so the second one starts
from scratch contents a larger call left behind."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import exact_io_aware_fwd_amd as fa
from tests.bwd_plan import dense_plan
from tests.gpu_util import GRAD_TOL, rel_l2, say, to_dev

pytestmark = pytest.mark.gpu


def _case(seed, B, Hq, Hkv, N, d, dt, causal):
    q, k, v, do = workloads.random_case(seed, B, Hq, Hkv, N, d, dt, with_do=True)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = fa.fwd(qd, kd, vd, causal=causal, softmax_scale=scale)
    return (q, k, v, do), (qd, kd, vd, o, lse, dod), scale


def test_bwd_noalloc_matches_bwd_on_two_calls():
    cases = [(9900, 2, 8, 2, 1500, 128, torch.bfloat16, True),    # split plan: partials in the scratch
             (9910, 1, 4, 1, 300, 64, torch.float16, False)]      # smaller, unsplit
    assert dense_plan(2, 8, 2, 1500, True)[1] > 1 and dense_plan(1, 4, 1, 300, False)[1] == 1
    for seed, B, Hq, Hkv, N, d, dt, causal in cases:
        need = fa.bwd_workspace_size(B, Hq, Hkv, N, d, dt, causal)
        assert 0 < need <= fa.binding.NOALLOC_SCRATCH_BYTES
        say(f"[bwd noalloc] B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} {dt} causal={causal}; workspace {need} bytes")
        cpu, (qd, kd, vd, o, lse, dod), scale = _case(seed, B, Hq, Hkv, N, d, dt, causal)
        got = fa.bwd_noalloc(qd, kd, vd, o, lse, dod, causal=causal, softmax_scale=scale)
        want = fa.bwd(qd, kd, vd, o, lse, dod, causal=causal, softmax_scale=scale)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), got, want):
            assert torch.equal(a, b), f"{name} differs from fa_bwd"
    # the second (smaller) call against the oracle as well
    q, k, v, do = cpu
    ref = oracle.attention_bwd(q, k, v, do, causal, scale)
    errs = [rel_l2(x.cpu(), r) for x, r in zip(got, ref)]
    say(f"    rel-L2 vs oracle {errs}")
    assert all(e <= GRAD_TOL for e in errs), errs


def test_bwd_noalloc_refuses_sizes_beyond_its_scratch():
    # a split plan whose fp32 partials alone fill 64 MiB: (128-key records, 8 chunks)
    B, Hq, Hkv, N, d = 1, 16, 4, 2048, 128
    assert dense_plan(B, Hq, Hkv, N, True) == (128, 8)
    assert fa.bwd_workspace_size(B, Hq, Hkv, N, d, torch.bfloat16, True) > fa.binding.NOALLOC_SCRATCH_BYTES
    q = torch.empty(B, Hq, N, d, dtype=torch.bfloat16, device="cuda:0")
    kv = torch.empty(B, Hkv, N, d, dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty(B, Hq, N, dtype=torch.float32, device="cuda:0")
    with pytest.raises(fa.FaError, match="static scratch"):
        fa.bwd_noalloc(q, kv, kv, q, lse, q, causal=True)
