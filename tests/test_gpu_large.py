"""GPU parity where byte offsets pass 2^31 and 2^32: 2048 sequences of 300 tokens, 32
query heads over 8 K/V heads, d = 128, bf16 (Q alone is 5.0 GB; the last head starts
5.0 GB into it) through fa_fwd, fa_bwd and, packed head-major with a window,
fa_fwd_masked / fa_bwd_masked.  The oracle checks sampled sequences, the last one
included, at the usual tolerances (O max error / max|O_ref| <= 1.5e-2, LSE <= 1e-4,
gradients rel-L2 <= 1e-2).

Every sequence holds one seeded block except the sampled ones, which get seeds of their
own: an offset that wrapped onto another sequence would read different data there.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.masks as om
import workloads
import exact_io_aware_fwd_amd as fa
from tests.gpu_util import GRAD_TOL, LSE_TOL, O_TOL, rel_l2, say

pytestmark = pytest.mark.gpu

B, HQ, HKV, N, D = 2048, 32, 8, 300, 128
SAMPLED = (0, 1037, B - 1)
DT = torch.bfloat16
SCALE = float(np.float32(1 / math.sqrt(D)))


def _block(seed, h):
    return workloads.randn(seed, (h, N, D), DT)


def _inputs():
    """CPU blocks per sampled sequence (and the shared one), and the [B, H, N, d] device
    tensors built from them."""
    shared = [_block(7000 + i, h) for i, h in enumerate((HQ, HKV, HKV, HQ))]
    own = {b: [_block(7100 + 4 * j + i, h) for i, h in enumerate((HQ, HKV, HKV, HQ))] for j, b in enumerate(SAMPLED)}
    dev = []
    for i, h in enumerate((HQ, HKV, HKV, HQ)):
        t = shared[i].to("cuda:0").unsqueeze(0).expand(B, h, N, D).contiguous()
        for b in SAMPLED:
            t[b] = own[b][i].to("cuda:0")
        dev.append(t)
    return own, dev


@pytest.fixture(scope="module")
def data():
    own, dev = _inputs()
    yield own, dev
    del dev
    torch.cuda.empty_cache()


def _check_fwd(o, lse, O_ref, L_ref):
    eo = float(np.max(np.abs(o - O_ref)) / np.max(np.abs(O_ref)))
    el = float(np.max(np.abs(lse - L_ref)))
    assert eo <= O_TOL[DT] and el <= LSE_TOL, (eo, el)
    return eo, el


def _check_grads(got, ref):
    errs = [rel_l2(g, r) for g, r in zip(got, ref)]
    assert all(np.isfinite(e) and e <= GRAD_TOL for e in errs), errs
    return errs


@pytest.mark.parametrize("causal", [False, True])
def test_large_offsets_fwd_bwd(data, causal):
    own, (q, k, v, do) = data
    say(f"[large] fa_fwd / fa_bwd B={B} Hq={HQ} Hkv={HKV} N={N} d={D} causal={causal}; Q {q.numel() * 2 / 2**30:.2f} GiB")
    o, lse = fa.fwd(q, k, v, causal=causal, softmax_scale=SCALE)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, softmax_scale=SCALE)
    torch.cuda.synchronize()
    for b in SAMPLED:
        qb, kb, vb, dob = (t.unsqueeze(0) for t in own[b])
        O_ref, L_ref = oracle.attention_fwd(qb, kb, vb, causal, SCALE)
        eo, el = _check_fwd(o[b:b + 1].float().cpu().double().numpy(), lse[b:b + 1].cpu().double().numpy(), O_ref, L_ref)
        ref = oracle.attention_bwd(qb, kb, vb, dob, causal, SCALE)
        errs = _check_grads([t[b:b + 1].float().cpu().double().numpy() for t in (dq, dk, dv)], ref)
        say(f"    sequence {b}: O {eo:.2e} LSE {el:.2e} dQ {errs[0]:.2e} dK {errs[1]:.2e} dV {errs[2]:.2e}")


def test_large_offsets_packed_window(data):
    own, (q, k, v, do) = data
    window = (100, 0)
    # head-major packed views [H, B*N, d] of the same data: sequence b owns rows b*N .. b*N+N-1
    qp, kp, vp, dop = (t.transpose(0, 1).reshape(t.shape[1], B * N, D) for t in (q, k, v, do))
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device="cuda:0")
    say(f"[large] fa_fwd_masked / fa_bwd_masked packed, {B} sequences of {N}, window {window}")
    o, lse = fa.fwd_masked(qp, kp, vp, window, SCALE, cu, cu, N, N)
    dq, dk, dv = fa.bwd_masked(qp, kp, vp, o, lse, dop, window, SCALE, cu, cu, N, N)
    torch.cuda.synchronize()
    cu1 = np.array([0, N], dtype=np.int32)
    for b in SAMPLED:
        rows = slice(b * N, (b + 1) * N)
        O_ref, L_ref = om.attention_fwd_masked(*own[b][:3], SCALE, cu1, cu1, window)
        eo, el = _check_fwd(o[:, rows].float().cpu().double().numpy(), lse[:, rows].cpu().double().numpy(), O_ref,
                            L_ref)
        ref = om.attention_bwd_masked(*own[b], SCALE, cu1, cu1, window)
        errs = _check_grads([t[:, rows].float().cpu().double().numpy() for t in (dq, dk, dv)], ref)
        say(f"    sequence {b}: O {eo:.2e} LSE {el:.2e} dQ {errs[0]:.2e} dK {errs[1]:.2e} dV {errs[2]:.2e}")
