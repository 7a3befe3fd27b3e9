"""GPU parity at one long sequence: 32805 tokens (2^15 plus a ragged tail of 37), two query
heads over one K/V head, d = 128, bf16, causal, against the fp64 oracle on whole tensors.

At this length the row-term workspace holds 1026 blocks of 32 rows per head, every key
tile's causal range spans up to 513 tiles, and the dK/dV plan is 256-key records split
into three chunks (asserted from the documented rule), so indexing that only short tests
reach is exercised at length.  Tolerances as everywhere: O max error / max |O_ref| <=
1.5e-2 (bf16), LSE max abs <= 1e-4, dQ/dK/dV rel-L2 <= 1e-2 ("FlashAttention Primer",
"Backward pass: recomputation instead of storage"; "Flash Attention" wiki, "Numerical
validation").  The oracle takes about half a minute here.
"""
from __future__ import annotations

import math
import time

import numpy as np
import pytest
import torch

import oracle
import workloads
import exact_io_aware_fwd_amd as fa
from tests.bwd_plan import dense_plan
from tests.gpu_util import GRAD_TOL, LSE_TOL, O_TOL, lse_err, o_err, rel_l2, say, to_dev

pytestmark = pytest.mark.gpu


def test_long_sequence_fwd_bwd_whole_tensors():
    B, Hq, Hkv, N, d, dt = 1, 2, 1, 32768 + 37, 128, torch.bfloat16
    assert dense_plan(B, Hq, Hkv, N, True) == (256, 3)
    q, k, v, do = workloads.random_case(9990, B, Hq, Hkv, N, d, dt, with_do=True)
    scale = float(np.float32(1 / math.sqrt(d)))
    say(f"[long] B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} bf16 causal: fa_fwd + fa_bwd")
    qd, kd, vd, dod = to_dev(q, k, v, do)
    o, lse = fa.fwd(qd, kd, vd, causal=True, softmax_scale=scale)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, causal=True, softmax_scale=scale)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    O_ref, L_ref = oracle.attention_fwd(q, k, v, True, scale)
    dQ, dK, dV = oracle.attention_bwd(q, k, v, do, True, scale)
    say(f"    oracle {time.perf_counter() - t0:.1f} s")
    eo, el = o_err(o.cpu(), O_ref), lse_err(lse.cpu(), L_ref)
    e = [rel_l2(dq.cpu(), dQ), rel_l2(dk.cpu(), dK), rel_l2(dv.cpu(), dV)]
    say(f"    O {eo:.2e} LSE {el:.2e} dQ {e[0]:.2e} dK {e[1]:.2e} dV {e[2]:.2e}")
    assert eo <= O_TOL[dt] and el <= LSE_TOL
    assert all(np.isfinite(x) and x <= GRAD_TOL for x in e)
