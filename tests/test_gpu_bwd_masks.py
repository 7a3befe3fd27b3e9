"""GPU parity of the mask-family backward (fa_bwd_masked) against the fp64 oracle in
oracle/masks.py: unequal query/key lengths (bottom-right), sliding windows on one or both
sides, packed variable-length batches with empty sequences, GQA, both dtypes and head
sizes, and the full-size sliding-window and packed workloads on sampled heads.

Tolerance as for the 16-bit backward (gpu_util): rel-L2 of dQ, dK, dV <= 1e-2 against
the oracle's gradients (the kernel is fed its own forward's O and LSE).  Rows that see no
key must get dQ = 0 exactly and keys no query sees dK = dV = 0 exactly.  Where an exact
gradient is identically zero (a window of one key per query gives P = 1, hence dQ = 0),
its norm is compared with ||dV_ref|| instead, as in the square backward tests at N = 1.
Without a mask the result must equal fa_bwd bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.masks as om
import workloads
from tests.gpu_util import GRAD_TOL, rel_l2, say, to_dev
import exact_io_aware_fwd_amd as fa

pytestmark = pytest.mark.gpu


def _rand(seed, shape, dtype=torch.bfloat16):
    return workloads.randn(seed, shape, dtype)


def _check_grads(got, ref, empty_q, unseen_k, label=""):
    names = ("dQ", "dK", "dV")
    errs = []
    nv = np.linalg.norm(ref[2].ravel())
    for n, g, r in zip(names, got, ref):
        g = g.float().cpu().double().numpy()
        nr = np.linalg.norm(r.ravel())
        e = rel_l2(g, r) if nr > 1e-9 * nv else float(np.linalg.norm((g - r).ravel()) / max(nv, 1e-30))
        errs.append(e)
        assert np.all(np.isfinite(g)), f"{n} not finite"
        assert e <= GRAD_TOL, f"{label} {n} rel-L2 {e:.3e}"
    dq, dk, dv = (g.float().cpu().numpy() for g in got)
    assert np.all(dq[empty_q] == 0), "rows that see no key must get dQ = 0"
    assert np.all(dk[unseen_k] == 0) and np.all(dv[unseen_k] == 0), "keys no query sees must get dK = dV = 0"
    say(f"    dQ {errs[0]:.2e} dK {errs[1]:.2e} dV {errs[2]:.2e}; empty rows {int(empty_q.sum())}, "
        f"unseen keys {int(unseen_k.sum())}")


def _fixed_case(B, Hq, Hkv, Nq, Nk, d, window, dt, seed):
    q, k, v = _rand(seed, (B, Hq, Nq, d), dt), _rand(seed + 1, (B, Hkv, Nk, d), dt), _rand(seed + 2, (B, Hkv, Nk, d), dt)
    do = _rand(seed + 3, (B, Hq, Nq, d), dt)
    say(f"[bwd masked fixed] q={tuple(q.shape)} k={tuple(k.shape)} window={window} {dt}")
    qd, kd, vd, dod = to_dev(q, k, v, do)
    o, lse = fa.fwd_masked(qd, kd, vd, window)
    grads = fa.bwd_masked(qd, kd, vd, o, lse, dod, window)
    torch.cuda.synchronize()
    scale = float(np.float32(1 / np.sqrt(d)))
    ref = om.attention_bwd_masked(q, k, v, do, scale, window=window)
    vis = om.visible(Nq, Nk, window)
    empty_q = np.broadcast_to(~vis.any(axis=1)[None, None, :, None], (B, Hq, Nq, d))
    unseen_k = np.broadcast_to(~vis.any(axis=0)[None, None, :, None], (B, Hkv, Nk, d))
    _check_grads(grads, ref, empty_q, unseen_k)


FIXED = [
    # (B, Hq, Hkv, Nq, Nk, d, window, dtype)
    (2, 4, 2, 300, 700, 128, (-1, 0), torch.bfloat16),
    (1, 4, 1, 700, 300, 64, (-1, 0), torch.float16),
    (1, 2, 2, 513, 513, 128, (63, 0), torch.bfloat16),
    (1, 4, 2, 1000, 1000, 64, (100, 50), torch.float16),
    (1, 2, 2, 257, 300, 128, (0, 0), torch.bfloat16),
    (2, 2, 1, 200, 200, 64, (-1, 7), torch.bfloat16),
    (1, 2, 1, 2049, 2049, 128, (511, 0), torch.bfloat16),
    (1, 2, 2, 640, 900, 128, (-1, -1), torch.bfloat16),
]


@pytest.mark.parametrize("case", FIXED, ids=lambda c: "B{}Hq{}Hkv{}Nq{}Nk{}d{}_w{}_{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5], f"{c[6][0]}_{c[6][1]}", str(c[7])[6:]))
def test_bwd_masked_fixed(case):
    _fixed_case(*case, seed=9600 + case[3])


def test_bwd_masked_packed():
    lq, lk = [0, 1, 255, 256, 257, 600, 5, 130], [3, 0, 255, 700, 1, 600, 64, 130]
    Hq, Hkv, d = 4, 2, 128
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q, k, v = _rand(9650, (Hq, cq[-1], d)), _rand(9651, (Hkv, ck[-1], d)), _rand(9652, (Hkv, ck[-1], d))
    do = _rand(9653, (Hq, cq[-1], d))
    scale = float(np.float32(1 / np.sqrt(d)))
    qd, kd, vd, dod = to_dev(q, k, v, do)
    cqd, ckd = torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda()
    for window in ((-1, -1), (-1, 0), (30, 2)):
        say(f"[bwd masked packed] window={window}")
        o, lse = fa.fwd_masked(qd, kd, vd, window, scale, cqd, ckd, max(lq), max(lk))
        grads = fa.bwd_masked(qd, kd, vd, o, lse, dod, window, scale, cqd, ckd, max(lq), max(lk))
        torch.cuda.synchronize()
        ref = om.attention_bwd_masked(q, k, v, do, scale, cq, ck, window)
        empty_q = np.zeros((Hq, cq[-1], d), dtype=bool)
        unseen_k = np.zeros((Hkv, ck[-1], d), dtype=bool)
        for b in range(len(lq)):
            vis = om.visible(lq[b], lk[b], window)
            empty_q[:, cq[b]:cq[b + 1]] = (~vis.any(axis=1))[None, :, None]
            unseen_k[:, ck[b]:ck[b + 1]] = (~vis.any(axis=0))[None, :, None]
        _check_grads(grads, ref, empty_q, unseen_k, label=str(window))


def test_bwd_masked_equals_bwd_bitwise():
    q, k, v, do = to_dev(_rand(9660, (1, 8, 1000, 128)), _rand(9661, (1, 2, 1000, 128)), _rand(9662, (1, 2, 1000, 128)),
                         _rand(9663, (1, 8, 1000, 128)))
    say("[bwd masked] equals fa_bwd bit for bit")
    for causal, window in ((False, (-1, -1)), (True, (-1, 0))):
        o, lse = fa.fwd(q, k, v, causal=causal)
        g1 = fa.bwd(q, k, v, o, lse, do, causal=causal)
        g2 = fa.bwd_masked(q, k, v, o, lse, do, window)
        torch.cuda.synchronize()
        for a, b in zip(g1, g2):
            assert torch.equal(a, b)


@pytest.mark.parametrize("name", [workloads.MASK_HEADLINE, "varlen_b8_hq32_hkv8_d128_bf16_causal"])
def test_bwd_mask_workloads_full_size_sampled_heads(name):
    """The full-size sliding-window and packed workloads (dO seeded), the oracle on two
    sampled query heads each with its K/V head; dK/dV of a K/V head sum over its query
    heads, so the oracle runs every query head of that group and the kernel's dK/dV are
    compared for those K/V heads."""
    w = workloads.MASK_WORKLOADS[name]
    q, k, v, cq, ck, _ = workloads.make_mask_inputs(w)
    do = _rand(w.seeds[0] + 50, tuple(q.shape))
    say(f"[bwd masked] {w.name} full size, sampled heads")
    qd, kd, vd, dod = to_dev(q, k, v, do)
    G = w.Hq // w.Hkv
    if w.packed:
        mq, mk = max(w.seqlens_q), max(w.seqlens_k)
        cqd, ckd = torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda()
        o, lse = fa.fwd_masked(qd, kd, vd, w.window, w.scale, cqd, ckd, mq, mk)
        dq, dk, dv = fa.bwd_masked(qd, kd, vd, o, lse, dod, w.window, w.scale, cqd, ckd, mq, mk)
    else:
        o, lse = fa.fwd_masked(qd, kd, vd, w.window, w.scale)
        dq, dk, dv = fa.bwd_masked(qd, kd, vd, o, lse, dod, w.window, w.scale)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    for hk in (0, w.Hkv - 1):
        hs = slice(hk * G, (hk + 1) * G)
        if w.packed:
            ref = om.attention_bwd_masked(q[hs], k[hk:hk + 1], v[hk:hk + 1], do[hs], w.scale, cq, ck, w.window)
            got = (dq[hs], dk[hk:hk + 1], dv[hk:hk + 1])
        else:
            ref = om.attention_bwd_masked(q[:1, hs], k[:1, hk:hk + 1], v[:1, hk:hk + 1], do[:1, hs], w.scale,
                                          window=w.window)
            got = (dq[:1, hs], dk[:1, hk:hk + 1], dv[:1, hk:hk + 1])
        for n, g, r in zip(("dQ", "dK", "dV"), got, ref):
            e = rel_l2(g.float().double().numpy(), r)
            say(f"    K/V head {hk}: {n} rel-L2 {e:.2e}")
            assert e <= GRAD_TOL, f"{n} rel-L2 {e:.3e}"
