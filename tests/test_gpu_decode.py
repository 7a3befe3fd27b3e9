"""GPU parity of the split-KV forward (fa_fwd_splitkv) and the log-sum-exp combine
(fa_lse_combine) against the fp64 oracle (oracle.attention_fwd_kv, oracle.lse_combine).

Same tolerances as the forward: O max|O - O_ref| / max|O_ref| <= 2e-3 (fp16), 1.5e-2
(bf16); LSE max abs <= 1e-4.  Cases: one and several new tokens, causal (bottom-right)
and not, row groups (G*Nq > 32), ragged key counts (1 .. 4097), explicit split counts
from 1 to one split per 32 keys, MQA, both dtypes and head sizes, and the two decode
workloads at full size.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
import exact_io_aware_fwd_amd as fa
from tests.gpu_util import LSE_TOL, O_TOL, lse_err, o_err, say, to_dev

pytestmark = pytest.mark.gpu


def _inputs(seed, B, Hq, Hkv, Nq, Nk, d, dtype):
    return (workloads.randn(seed, (B, Hq, Nq, d), dtype), workloads.randn(seed + 1, (B, Hkv, Nk, d), dtype),
            workloads.randn(seed + 2, (B, Hkv, Nk, d), dtype))


def check_splitkv(q, k, v, causal, scale, num_splits=0, label=""):
    say(f"[splitkv] {label} q={tuple(q.shape)} k={tuple(k.shape)} {q.dtype} causal={causal} splits={num_splits}")
    qd, kd, vd = to_dev(q, k, v)
    o, lse = fa.binding.fwd_splitkv(qd, kd, vd, causal=causal, softmax_scale=scale, num_splits=num_splits)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_fwd_kv(q, k, v, causal, scale)
    eo, el = o_err(o.cpu(), O_ref), lse_err(lse.cpu(), L_ref)
    assert np.isfinite(eo) and np.isfinite(el)
    assert eo <= O_TOL[q.dtype], f"O error {eo:.3e} > {O_TOL[q.dtype]}"
    assert el <= LSE_TOL, f"LSE error {el:.3e} > {LSE_TOL}"
    return o, lse


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Nq,Nk,causal", [(1, 1, False), (1, 31, False), (1, 33, True), (3, 70, True),
                                          (4, 1000, False), (8, 4097, True), (16, 129, True), (37, 300, True),
                                          (5, 5, True)])
def test_splitkv_shapes(dtype, d, Nq, Nk, causal):
    q, k, v = _inputs(100 + Nq + Nk + d, 1, 8, 2, Nq, Nk, d, dtype)
    check_splitkv(q, k, v, causal, float(np.float32(d ** -0.5)), label=f"Nq={Nq} Nk={Nk}")


@pytest.mark.parametrize("num_splits", [1, 2, 3, 7, 64, 10_000])
def test_splitkv_split_counts(num_splits):
    q, k, v = _inputs(300, 2, 8, 4, 2, 2000, 128, torch.bfloat16)
    check_splitkv(q, k, v, True, 0.0883883, num_splits=num_splits, label="splits")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,Hq,Hkv,N,causal,S", [(1, 8, 2, 128, True, 0), (1, 8, 2, 1000, True, 0),
                                                 (1, 4, 4, 1024, False, 0), (2, 4, 1, 1100, True, 5),
                                                 (1, 2, 1, 777, False, 16), (1, 6, 3, 300, True, 10_000)])
def test_prefill_key_split(dtype, d, B, Hq, Hkv, N, causal, S):
    """As many queries as keys (>= 128): fa_fwd_splitkv cuts every query block's keys into
    64-key-aligned splits and merges the parts; ragged N, causal splits past a block's
    diagonal (empty parts), explicit counts up to one split per tile, GQA and MQA."""
    q, k, v = _inputs(400 + N + d + S, B, Hq, Hkv, N, N, d, dtype)
    check_splitkv(q, k, v, causal, float(np.float32(d ** -0.5)), num_splits=S, label=f"prefill N={N}")


def test_prefill_key_split_matches_fa_fwd_on_a_small_grid():
    """Two key splits against fa_fwd on a small grid (one sequence of 1024 tokens, 32
    query heads over 8 K/V heads): both within the oracle's tolerance, and within the
    bf16 output rounding of each other; at d = 128 the default is one split (fa_fwd)."""
    q, k, v = _inputs(450, 1, 32, 8, 1024, 1024, 128, torch.bfloat16)
    assert fa.splitkv_num_splits(1, 32, 8, 1024, 1024, 128) == 1
    o1, l1 = check_splitkv(q, k, v, True, 0.0883883, num_splits=2, label="small grid")
    o2, l2 = fa.fwd(*to_dev(q, k, v), causal=True, softmax_scale=0.0883883)
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() <= 2 ** -7 * o2.float().abs().max().item()
    assert (l1 - l2).abs().max().item() <= 2e-5


@pytest.mark.parametrize("Hq,causal", [(256, False), (16, True)], ids=["q64-waves", "small-grid"])
def test_prefill_one_split_is_fa_fwd(Hq, causal):
    """With one key split the key-split route is fa_fwd itself: the same bits, on a grid
    where fa_fwd runs 64-query waves (256 query heads, N = 512, non-causal) and on a small
    one (16 heads, causal) where it runs two waves per 32 queries."""
    q, k, v = _inputs(460 + Hq, 1, Hq, Hq // 8, 512, 512, 128, torch.bfloat16)
    qd, kd, vd = to_dev(q, k, v)
    o1, l1 = fa.fwd_splitkv(qd, kd, vd, causal=causal, softmax_scale=0.0883883, num_splits=1)
    o2, l2 = fa.fwd(qd, kd, vd, causal=causal, softmax_scale=0.0883883)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_splitkv_mqa_and_mha():
    q, k, v = _inputs(310, 1, 16, 1, 3, 777, 128, torch.bfloat16)      # MQA: 48 rows -> two row groups
    check_splitkv(q, k, v, True, 0.0883883, label="mqa")
    q, k, v = _inputs(320, 2, 4, 4, 2, 515, 64, torch.float16)          # MHA
    check_splitkv(q, k, v, False, 0.125, label="mha")


def test_splitkv_equals_forward_when_square():
    # with Nq == Nk and causal the queries are the whole sequence: both entry points
    # must agree with the same oracle
    q, k, v = _inputs(330, 1, 4, 2, 200, 200, 128, torch.bfloat16)
    check_splitkv(q, k, v, True, 0.0883883, label="square")


@pytest.mark.parametrize("name", sorted(workloads.DECODE_WORKLOADS))
def test_decode_workloads(name):
    w = workloads.DECODE_WORKLOADS[name]
    q, k, v = workloads.make_decode_inputs(w)
    for causal in w.causal:
        check_splitkv(q, k, v, causal, w.scale, label=name)


def test_splitkv_deterministic():
    q, k, v = _inputs(340, 1, 8, 2, 2, 3000, 128, torch.bfloat16)
    qd, kd, vd = to_dev(q, k, v)
    o1, l1 = fa.binding.fwd_splitkv(qd, kd, vd, causal=True)
    o2, l2 = fa.binding.fwd_splitkv(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_splitkv_empty():
    q, k, v = _inputs(350, 1, 4, 2, 0, 16, 64, torch.float16)
    o, lse = fa.binding.fwd_splitkv(*to_dev(q, k, v))
    torch.cuda.synchronize()
    assert o.numel() == 0 and lse.numel() == 0


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
def test_lse_combine_parity(dtype, d):
    g = np.random.default_rng(360 + d)
    rows, S = 300, 9
    Op = g.standard_normal((rows, S, d)).astype(np.float32)
    Lp = (g.standard_normal((rows, S)) * 20).astype(np.float32)
    Lp[::7, 3] = -np.inf                      # empty parts
    Lp[5, :] = -np.inf                        # a row with no part at all
    Lp[6, :] = [800.0 + i for i in range(S)]  # huge statistics
    say(f"[combine] rows={rows} S={S} d={d} {dtype}")
    o, lse = fa.binding.lse_combine(torch.from_numpy(Op).cuda(), torch.from_numpy(Lp).cuda(), dtype)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.lse_combine(Op, Lp)
    o_c, l_c = o.double().cpu().numpy(), lse.double().cpu().numpy()
    assert np.all(o_c[5] == 0) and np.isneginf(l_c[5])
    keep = np.isfinite(L_ref)
    assert o_err(o_c[keep], O_ref[keep]) <= O_TOL[dtype]
    # LSE near 808 (row 6) is stored in fp32 with a spacing of 6.1e-5: allow 4 spacings there
    tol = np.maximum(LSE_TOL, 4 * np.spacing(np.abs(L_ref[keep]).astype(np.float32)).astype(np.float64))
    assert np.all(np.abs(l_c[keep] - L_ref[keep]) <= tol)
