"""GPU parity of fa_bwd on the dK/dV plans that the short-sequence tests do not reach.

* The benchmarked call itself: the grouped-query long-context workload (B=2, Hq=32,
  Hkv=8, N=8192, d=128, bf16, causal) with the exact inputs bench.py draws (Q, K, V from
  seeds 4000-4002, dO from 4003).  Its plan is 256-key records, one chunk each (the
  unsplit 64-key dK/dV pass, four query heads a record).  The oracle checks two whole
  K/V groups — (batch 0, K/V head 0) and (batch 1, K/V head 7) — O and LSE of their
  query heads, dQ of every query head in them, and the group's dK and dV.
* 256-key records split into chunks (the chunked 64-key pass plus the ordered reduction
  of the fp32 partials), d = 64 and 128, fp16 and bf16, causal and not, including a
  ragged last record whose causal range has fewer query steps than chunks, so that some
  chunks have nothing to add and write zero partials.

Each case first asserts, from the documented plan rule, that the shape takes the path
it is meant to test.  Tolerances as everywhere ("Flash Attention" wiki, "Numerical
validation"; the target values of this path): O max error / max|O_ref| <= 1.5e-2 (bf16),
2e-3 (fp16), LSE max abs <= 1e-4, dQ/dK/dV rel-L2 <= 1e-2 against the fp64 oracle of
"FlashAttention Primer", "Backward pass: recomputation instead of storage".
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import exact_io_aware_fwd_amd as fa
from tests.bwd_plan import dense_plan, rowterm_bytes
from tests.gpu_util import GRAD_TOL, LSE_TOL, O_TOL, lse_err, o_err, rel_l2, say

pytestmark = pytest.mark.gpu


def _check_groups(q, k, v, do, out, causal, scale, groups, label):
    """Oracle check of whole K/V groups: O, LSE and dQ of the group's query heads, the
    group's dK and dV.  `out` = (o, lse, dq, dk, dv) on the device."""
    o, lse, dq, dk, dv = (t.cpu() for t in out)
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    for b, g in groups:
        hs, ks = slice(g * G, (g + 1) * G), slice(g, g + 1)
        sl = (slice(b, b + 1), hs)
        args = (q[sl], k[b:b + 1, ks], v[b:b + 1, ks])
        O_ref, L_ref = oracle.attention_fwd(*args, causal, scale)
        eo, el = o_err(o[sl], O_ref), lse_err(lse[sl], L_ref)
        dQ, dK, dV = oracle.attention_bwd(*args, do[sl], causal, scale)
        e = [rel_l2(dq[sl], dQ), rel_l2(dk[b:b + 1, ks], dK), rel_l2(dv[b:b + 1, ks], dV)]
        say(f"    {label} batch {b} K/V head {g}: O {eo:.2e} LSE {el:.2e} dQ {e[0]:.2e} dK {e[1]:.2e} dV {e[2]:.2e}")
        assert eo <= O_TOL[q.dtype] and el <= LSE_TOL, (b, g, eo, el)
        assert all(np.isfinite(x) and x <= GRAD_TOL for x in e), (b, g, e)


def _run(q, k, v, do, causal, scale):
    qd, kd, vd, dod = (t.to("cuda:0") for t in (q, k, v, do))
    o, lse = fa.fwd(qd, kd, vd, causal=causal, softmax_scale=scale)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def test_benchmarked_backward_sampled_groups():
    w = workloads.WORKLOADS[workloads.HEADLINE]
    q, k, v = workloads.make_inputs(w)
    do = workloads.randn(w.seeds[2] + 1, (w.B, w.Hq, w.N, w.d), w.torch_dtype)   # as bench.py draws it
    causal = True
    assert dense_plan(w.B, w.Hq, w.Hkv, w.N, causal) == (256, 1)
    # an unsplit plan needs only the row terms in the workspace
    assert fa.bwd_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.d, q.dtype, causal) == rowterm_bytes(w.B, w.Hq, w.N)
    say(f"[bwd plans] {w.name}: the benchmarked fa_fwd + fa_bwd, two whole K/V groups")
    out = _run(q, k, v, do, causal, w.scale)
    _check_groups(q, k, v, do, out, causal, w.scale, [(0, 0), (w.B - 1, w.Hkv - 1)], w.name)


# (B, Hq, Hkv, N, d, dtype, causal, expected plan, sampled (batch, K/V head) groups)
SPLIT_CASES = [
    (1, 32, 8, 8192, 128, torch.bfloat16, True, (256, 2), [(0, 0), (0, 7)]),
    (1, 32, 8, 8192, 64, torch.float16, True, (256, 2), [(0, 3)]),
    (1, 32, 8, 4096, 128, torch.float16, False, (256, 2), [(0, 0), (0, 7)]),
    (1, 16, 4, 4100, 64, torch.bfloat16, False, (256, 2), [(0, 0), (0, 3)]),
    # ragged causal: the last record (keys 16384-16415) has 4 query steps for 7 chunks
    (1, 4, 1, 16416, 128, torch.bfloat16, True, (256, 7), [(0, 0)]),
]


@pytest.mark.parametrize("case", SPLIT_CASES,
                         ids=lambda c: f"B{c[0]}Hq{c[1]}Hkv{c[2]}N{c[3]}d{c[4]}{'f16' if c[5] == torch.float16 else 'bf16'}"
                                       f"{'c' if c[6] else 'nc'}")
def test_split_256_key_records(case):
    B, Hq, Hkv, N, d, dt, causal, plan, groups = case
    assert dense_plan(B, Hq, Hkv, N, causal) == plan
    q, k, v, do = workloads.random_case(8800 + N + d, B, Hq, Hkv, N, d, dt, with_do=True)
    scale = float(np.float32(1 / math.sqrt(d)))
    say(f"[bwd plans] split 256-key records {plan}: B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} {dt} causal={causal}")
    out = _run(q, k, v, do, causal, scale)
    _check_groups(q, k, v, do, out, causal, scale, groups, f"plan {plan}")
