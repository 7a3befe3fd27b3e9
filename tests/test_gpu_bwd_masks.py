"""GPU parity of the mask-family backward (fa_bwd_masked) against the fp64 oracle in
oracle/masks.py: unequal query/key lengths (bottom-right), sliding windows on one or both
sides, packed variable-length batches with empty sequences, block-sparse tile lists
(shared and per head, with windows, packed, empty lists), GQA, both dtypes and head
sizes, and the full-size sliding-window, packed and block-sparse workloads on sampled
heads.

Tolerance as for the 16-bit backward (gpu_util): rel-L2 of dQ, dK, dV <= 1e-2 against
the oracle's gradients (the kernel is fed its own forward's O and LSE).  Rows that see no
key must get dQ = 0 exactly and keys no query sees dK = dV = 0 exactly.  Where an exact
gradient is identically zero (a window of one key per query gives P = 1, hence dQ = 0),
its norm is compared with ||dV_ref|| instead, as in the square backward tests at N = 1.
Without a mask the result must equal fa_bwd bit for bit, and lists naming every tile
must equal no lists bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.masks as om
import workloads
from tests.gpu_util import GRAD_TOL, rel_l2, say, to_dev
import exact_io_aware_fwd_amd as fa
from tests.bwd_plan import dense_plan

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


def _random_lists(seed, B, Hm, Lq, Lk, density):
    g = np.random.Generator(np.random.PCG64(seed))
    nqb, nkt = -(-Lq // 256), -(-Lk // 64)
    return [[[sorted(int(t) for t in np.nonzero(g.random(nkt) < density)[0]) for _ in range(nqb)]
             for _ in range(Hm)] for _ in range(B)]


def _list_masks(lists, lq, lk, window, Hq, G):
    """Per sequence and query head: rows that see no key; per K/V head: keys no query sees."""
    empty_q, unseen_k = [], []
    for b in range(len(lq)):
        eq, uk = [], []
        for h in range(Hq):
            hm = lists[b][0] if len(lists[b]) == 1 else lists[b][h]
            vis = om.visible(lq[b], lk[b], window, hm)
            eq.append(~vis.any(axis=1))
            uk.append(vis.any(axis=0))
        empty_q.append(np.stack(eq))
        unseen_k.append(np.stack([~np.any(uk[g * G:(g + 1) * G], axis=0) for g in range(Hq // G)]))
    return empty_q, unseen_k


@pytest.mark.parametrize("Hm,window,density,d,dt", [
    (1, (-1, -1), 0.3, 128, torch.bfloat16), (4, (-1, 0), 0.5, 128, torch.bfloat16),
    (4, (200, 100), 0.7, 64, torch.float16), (1, (-1, 0), 0.0, 128, torch.bfloat16),
    (4, (-1, -1), 0.15, 64, torch.bfloat16)])
def test_bwd_masked_block_lists(Hm, window, density, d, dt):
    B, Hq, Hkv, Nq, Nk = 2, 4, 2, 1100, 900
    G = Hq // Hkv
    q, k, v = _rand(9670, (B, Hq, Nq, d), dt), _rand(9671, (B, Hkv, Nk, d), dt), _rand(9672, (B, Hkv, Nk, d), dt)
    do = _rand(9673, (B, Hq, Nq, d), dt)
    lists = _random_lists(9674 + Hm, B, Hm, Nq, Nk, density)
    say(f"[bwd masked lists] Hm={Hm} window={window} density={density} d={d} {dt}")
    qd, kd, vd, dod = to_dev(q, k, v, do)
    bc, bi = fa.block_lists_to_tensors(lists, Nq, Nk, "cuda:0")
    o, lse = fa.fwd_masked(qd, kd, vd, window, block_cnt=bc, block_idx=bi)
    grads = fa.bwd_masked(qd, kd, vd, o, lse, dod, window, block_cnt=bc, block_idx=bi)
    torch.cuda.synchronize()
    scale = float(np.float32(1 / np.sqrt(d)))
    ref = om.attention_bwd_masked(q, k, v, do, scale, window=window, block_lists=lists)
    eq, uk = _list_masks(lists, [Nq] * B, [Nk] * B, window, Hq, G)
    empty_q = np.broadcast_to(np.stack(eq)[..., None], (B, Hq, Nq, d))
    unseen_k = np.broadcast_to(np.stack(uk)[..., None], (B, Hkv, Nk, d))
    _check_grads(grads, ref, empty_q, unseen_k)


def test_bwd_masked_block_lists_packed():
    lq, lk = [0, 1, 255, 256, 600, 5, 300], [3, 0, 255, 700, 600, 64, 130]
    Hq, Hkv, d = 4, 2, 128
    G = Hq // Hkv
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q, k, v = _rand(9680, (Hq, cq[-1], d)), _rand(9681, (Hkv, ck[-1], d)), _rand(9682, (Hkv, ck[-1], d))
    do = _rand(9683, (Hq, cq[-1], d))
    mq, mk = max(lq), max(lk)
    g = np.random.Generator(np.random.PCG64(9684))     # per sequence, its own blocks and tiles
    lists = [[[sorted(int(t) for t in np.nonzero(g.random(-(-lk[b] // 64)) < 0.5)[0])
               for _ in range(-(-lq[b] // 256))] for _ in range(Hq)] for b in range(len(lq))]
    scale = float(np.float32(1 / np.sqrt(d)))
    qd, kd, vd, dod = to_dev(q, k, v, do)
    cqd, ckd = torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda()
    bc, bi = fa.block_lists_to_tensors(lists, mq, mk, "cuda:0")
    for window in ((-1, -1), (-1, 0), (100, 20)):
        say(f"[bwd masked lists packed] window={window}")
        o, lse = fa.fwd_masked(qd, kd, vd, window, scale, cqd, ckd, mq, mk, bc, bi)
        grads = fa.bwd_masked(qd, kd, vd, o, lse, dod, window, scale, cqd, ckd, mq, mk, bc, bi)
        torch.cuda.synchronize()
        ref = om.attention_bwd_masked(q, k, v, do, scale, cq, ck, window, lists)
        eq, uk = _list_masks(lists, lq, lk, window, Hq, G)
        empty_q = np.zeros((Hq, cq[-1], d), dtype=bool)
        unseen_k = np.zeros((Hkv, ck[-1], d), dtype=bool)
        for b in range(len(lq)):
            empty_q[:, cq[b]:cq[b + 1]] = eq[b][..., None]
            unseen_k[:, ck[b]:ck[b + 1]] = uk[b][..., None]
        _check_grads(grads, ref, empty_q, unseen_k, label=str(window))


@pytest.mark.parametrize("d,dt,window", [(128, torch.bfloat16, (-1, -1)), (64, torch.float16, (-1, 0))])
def test_bwd_masked_block_lists_split_key_blocks(d, dt, window):
    """Lists with global columns (a band plus every 8th tile) give a few key blocks many more
    query steps than the rest; those run as several chunks whose fp32 partials are summed in
    a fixed order.  Parity with the oracle, and two calls agree bit for bit."""
    B, Hq, Hkv, N = 1, 8, 2, 2100
    G = Hq // Hkv
    q, k, v, do = (_rand(9700 + i, (B, Hq if i in (0, 3) else Hkv, N, d), dt) for i in range(4))
    lists = [[workloads.local_global_tiles(N, N, band=3, stride=8)]]
    say(f"[bwd masked lists split] N={N} d={d} {dt} window={window}")
    qd, kd, vd, dod = to_dev(q, k, v, do)
    bc, bi = fa.block_lists_to_tensors(lists, N, N, "cuda:0")
    o, lse = fa.fwd_masked(qd, kd, vd, window, block_cnt=bc, block_idx=bi)
    g1 = fa.bwd_masked(qd, kd, vd, o, lse, dod, window, block_cnt=bc, block_idx=bi)
    g2 = fa.bwd_masked(qd, kd, vd, o, lse, dod, window, block_cnt=bc, block_idx=bi)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    scale = float(np.float32(1 / np.sqrt(d)))
    ref = om.attention_bwd_masked(q, k, v, do, scale, window=window, block_lists=lists)
    eq, uk = _list_masks(lists, [N], [N], window, Hq, G)
    empty_q = np.broadcast_to(np.stack(eq)[..., None], (B, Hq, N, d))
    unseen_k = np.broadcast_to(np.stack(uk)[..., None], (B, Hkv, N, d))
    _check_grads(g1, ref, empty_q, unseen_k)


def test_bwd_masked_all_tiles_listed_equals_no_lists():
    B, Hq, Hkv, N, d = 1, 4, 2, 1000, 128
    q, k, v, do = (_rand(9690 + i, (B, Hq if i in (0, 3) else Hkv, N, d)) for i in range(4))
    qd, kd, vd, dod = to_dev(q, k, v, do)
    lists = [[[list(range(-(-N // 64))) for _ in range(-(-N // 256))]]]
    bc, bi = fa.block_lists_to_tensors(lists, N, N, "cuda:0")
    say("[bwd masked lists] every tile listed equals no lists, bit for bit; two calls agree")
    for window in ((-1, -1), (300, 0)):
        o, lse = fa.fwd_masked(qd, kd, vd, window)
        g1 = fa.bwd_masked(qd, kd, vd, o, lse, dod, window)
        g2 = fa.bwd_masked(qd, kd, vd, o, lse, dod, window, block_cnt=bc, block_idx=bi)
        g3 = fa.bwd_masked(qd, kd, vd, o, lse, dod, window, block_cnt=bc, block_idx=bi)
        torch.cuda.synchronize()
        for a, b, c in zip(g1, g2, g3):
            assert torch.equal(a, b) and torch.equal(b, c)


@pytest.mark.parametrize("B,causal", [(2, False), (4, False), (4, True), (2, True)])
def test_bwd_masked_equals_bwd_bitwise(B, causal):
    """Without a mask the general mode equals fa_bwd bit for bit where fa_bwd does not split
    its dK/dV records into chunks with fp32 partials (a split sums in another order): from
    256 blocks of 256 keys on (512 when causal), where it runs 64 keys a wave.  Where it
    splits (B = 2 causal: 256 records of 256 keys, two chunks each) dQ is still equal bit for
    bit and dK, dV differ only by the order of the fp32 partial sums before rounding."""
    Hq, Hkv, N = 8, 4, 8192
    q, k, v, do = to_dev(_rand(9660, (B, Hq, N, 128)), _rand(9661, (B, Hkv, N, 128)), _rand(9662, (B, Hkv, N, 128)),
                         _rand(9663, (B, Hq, N, 128)))
    split = dense_plan(B, Hq, Hkv, N, causal)[1] > 1
    assert split == (B == 2 and causal)
    say(f"[bwd masked] equals fa_bwd {'within rounding (split dK/dV)' if split else 'bit for bit'}, "
        f"B={B} causal={causal}")
    for window in ((-1, 0),) if causal else ((-1, -1),):
        o, lse = fa.fwd(q, k, v, causal=causal)
        g1 = fa.bwd(q, k, v, o, lse, do, causal=causal)
        g2 = fa.bwd_masked(q, k, v, o, lse, do, window)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(g1, g2)):
            if split and i > 0:   # fp32 sums in another order, then one rounding to bf16
                diff = (a.float() - b.float()).abs()
                assert diff.max().item() <= 2.0 ** -6 * b.float().abs().max().item()
                assert (diff.norm() / b.float().norm()).item() <= 1e-3
            else:
                assert torch.equal(a, b)


@pytest.mark.parametrize("d,dt,window", [(128, torch.bfloat16, (200, 0)), (64, torch.float16, (100, 40)),
                                          (128, torch.float16, (-1, -1)), (64, torch.bfloat16, (-1, 0))])
def test_bwd_masked_packed_many_key_blocks(d, dt, window):
    """Eight packed sequences of ragged, unequal lengths (empty ones included) on 16 K/V
    heads: over a thousand 128-key blocks, windows cutting through steps and key blocks,
    both head sizes and dtypes; the oracle checks the first and the last K/V head with
    their query heads whole."""
    lq, lk = [2100, 0, 1, 513, 1999, 256, 700, 1030], [2100, 5, 0, 600, 1999, 255, 900, 1030]
    Hq, Hkv = 32, 16
    G = Hq // Hkv
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q, k, v = _rand(9660, (Hq, cq[-1], d), dt), _rand(9661, (Hkv, ck[-1], d), dt), _rand(9662, (Hkv, ck[-1], d), dt)
    do = _rand(9663, (Hq, cq[-1], d), dt)
    scale = float(np.float32(1 / np.sqrt(d)))
    say(f"[bwd masked many key blocks] packed {len(lq)} sequences Hq={Hq} Hkv={Hkv} d={d} {dt} window={window}")
    qd, kd, vd, dod = to_dev(q, k, v, do)
    cqd, ckd = torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda()
    o, lse = fa.fwd_masked(qd, kd, vd, window, scale, cqd, ckd, max(lq), max(lk))
    dq, dk, dv = fa.bwd_masked(qd, kd, vd, o, lse, dod, window, scale, cqd, ckd, max(lq), max(lk))
    torch.cuda.synchronize()
    for hk in (0, Hkv - 1):
        hs = slice(hk * G, (hk + 1) * G)
        ref = om.attention_bwd_masked(q[hs], k[hk:hk + 1], v[hk:hk + 1], do[hs], scale, cq, ck, window)
        empty_q = np.zeros((G, cq[-1], d), dtype=bool)
        unseen_k = np.zeros((1, ck[-1], d), dtype=bool)
        for b in range(len(lq)):
            vis = om.visible(lq[b], lk[b], window)
            empty_q[:, cq[b]:cq[b + 1]] = (~vis.any(axis=1))[None, :, None]
            unseen_k[:, ck[b]:ck[b + 1]] = (~vis.any(axis=0))[None, :, None]
        _check_grads((dq[hs], dk[hk:hk + 1], dv[hk:hk + 1]), ref, empty_q, unseen_k, label=f"K/V head {hk}")


@pytest.mark.parametrize("name", [workloads.MASK_HEADLINE, "varlen_b8_hq32_hkv8_d128_bf16_causal",
                                  "bsparse_b1_hq16_hkv4_n8192_d128_bf16"])
def test_bwd_mask_workloads_full_size_sampled_heads(name):
    """The full-size sliding-window and packed workloads (dO seeded), the oracle on two
    sampled query heads each with its K/V head; dK/dV of a K/V head sum over its query
    heads, so the oracle runs every query head of that group and the kernel's dK/dV are
    compared for those K/V heads."""
    w = workloads.MASK_WORKLOADS[name]
    q, k, v, cq, ck, lists = workloads.make_mask_inputs(w)
    do = _rand(w.seeds[0] + 50, tuple(q.shape))
    say(f"[bwd masked] {w.name} full size, sampled heads")
    qd, kd, vd, dod = to_dev(q, k, v, do)
    G = w.Hq // w.Hkv
    mq, mk = max(w.seqlens_q), max(w.seqlens_k)
    bc, bi = fa.block_lists_to_tensors(lists, mq, mk, "cuda:0") if lists is not None else (None, None)
    if w.packed:
        cqd, ckd = torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda()
        o, lse = fa.fwd_masked(qd, kd, vd, w.window, w.scale, cqd, ckd, mq, mk, bc, bi)
        dq, dk, dv = fa.bwd_masked(qd, kd, vd, o, lse, dod, w.window, w.scale, cqd, ckd, mq, mk, bc, bi)
    else:
        o, lse = fa.fwd_masked(qd, kd, vd, w.window, w.scale, block_cnt=bc, block_idx=bi)
        dq, dk, dv = fa.bwd_masked(qd, kd, vd, o, lse, dod, w.window, w.scale, block_cnt=bc, block_idx=bi)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    for hk in (0, w.Hkv - 1):
        hs = slice(hk * G, (hk + 1) * G)
        sub = None if lists is None else [lb if len(lb) == 1 else lb[hs] for lb in lists]
        if w.packed:
            ref = om.attention_bwd_masked(q[hs], k[hk:hk + 1], v[hk:hk + 1], do[hs], w.scale, cq, ck, w.window,
                                          sub)
            got = (dq[hs], dk[hk:hk + 1], dv[hk:hk + 1])
        else:
            ref = om.attention_bwd_masked(q[:1, hs], k[:1, hk:hk + 1], v[:1, hk:hk + 1], do[:1, hs], w.scale,
                                          window=w.window, block_lists=sub)
            got = (dq[:1, hs], dk[:1, hk:hk + 1], dv[:1, hk:hk + 1])
        for n, g, r in zip(("dQ", "dK", "dV"), got, ref):
            e = rel_l2(g.float().double().numpy(), r)
            say(f"    K/V head {hk}: {n} rel-L2 {e:.2e}")
            assert e <= GRAD_TOL, f"{n} rel-L2 {e:.3e}"


def test_bwd_masked_inconsistent_lists_stay_in_bounds():
    """As for the forward: lists that break the contract give unspecified but finite
    gradients and no invalid access (counts and tiles are clamped; the transpose only
    compares list entries)."""
    B, Hq, Hkv, N, d = 1, 4, 2, 700, 128
    q, k, v, do = to_dev(_rand(9980, (B, Hq, N, d)), _rand(9981, (B, Hkv, N, d)), _rand(9982, (B, Hkv, N, d)),
                         _rand(9983, (B, Hq, N, d)))
    nqb, cap = -(-N // 256), -(-N // 64)
    g = torch.Generator().manual_seed(9984)
    cnt = torch.randint(-3, cap + 6, (B, Hq, nqb), generator=g, dtype=torch.int32).cuda()
    idx = torch.randint(-10, 2 * cap, (B, Hq, nqb, cap), generator=g, dtype=torch.int32).cuda()
    say("[bwd masked] inconsistent block lists")
    for window in ((-1, -1), (200, 0)):
        o, lse = fa.fwd_masked(q, k, v, window, block_cnt=cnt, block_idx=idx)
        grads = fa.bwd_masked(q, k, v, o, lse, do, window, block_cnt=cnt, block_idx=idx)
        torch.cuda.synchronize()
        for t in grads:
            assert torch.isfinite(t.float()).all()


def test_bwd_masked_refuses_a_host_workspace_and_a_short_lse():
    """The binding checks the caller's workspace (a GPU tensor on q's device) and the LSE
    shape ([Hq, total] packed, [B, Hq, N] fixed) before the ABI call: a host pointer or a
    short LSE would otherwise reach the kernels."""
    B, Hq, Hkv, N, d = 1, 4, 2, 200, 64
    q, k, v, do = to_dev(_rand(9990, (B, Hq, N, d)), _rand(9991, (B, Hkv, N, d)), _rand(9992, (B, Hkv, N, d)),
                         _rand(9993, (B, Hq, N, d)))
    o, lse = fa.fwd_masked(q, k, v, (-1, 0))
    torch.cuda.synchronize()
    say("[bwd masked] host workspace and short LSE are refused")
    with pytest.raises(ValueError):
        fa.bwd_masked(q, k, v, o, lse, do, (-1, 0), workspace=torch.empty(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError):
        fa.bwd_masked(q, k, v, o, lse[:, :, :-1].contiguous(), do, (-1, 0))
    qp, kp, vp, op, dop = (t[0] for t in (q, k, v, o, do))        # packed: one sequence of N
    cu = torch.tensor([0, N], dtype=torch.int32, device="cuda:0")
    with pytest.raises(ValueError):
        fa.bwd_masked(qp, kp, vp, op, lse, dop, (-1, 0), cu_seqlens_q=cu, cu_seqlens_k=cu)   # lse not [Hq, N]
    dq = fa.bwd_masked(qp, kp, vp, op, lse[0], dop, (-1, 0), cu_seqlens_q=cu, cu_seqlens_k=cu)[0]
    torch.cuda.synchronize()
    assert torch.isfinite(dq.float()).all()
