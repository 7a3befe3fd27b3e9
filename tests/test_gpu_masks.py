"""GPU parity of the mask-family forward (fa_fwd_masked) against the fp64 oracle in
oracle/masks.py: packed variable-length batches, unequal query/key lengths (bottom-right
aligned), sliding windows on one or both sides, block-sparse tile lists (shared and per
head, including empty lists), rows that see no key, and the full-size workloads on
sampled heads or rows.

Tolerances are those of the 16-bit forward (gpu_util): O max|O - O_ref| / max|O_ref|
<= 1.5e-2 (bf16) / 2e-3 (fp16); LSE max abs <= 1e-4; rows that see no key must be
exactly O = 0 and LSE = -inf.  With no mask (and with the causal window on equal
lengths) the result must equal fa_fwd bit for bit: same arithmetic, same order.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.masks as om
import workloads
from tests.gpu_util import LSE_TOL, O_TOL, say, to_dev
import exact_io_aware_fwd_amd as fa

pytestmark = pytest.mark.gpu


def _compare(o, lse, O_ref, L_ref, dtype):
    o = o.float().cpu().double().numpy() if hasattr(o, "cpu") else o
    lse = lse.cpu().double().numpy() if hasattr(lse, "cpu") else lse
    empty = np.isneginf(L_ref)
    assert np.array_equal(np.isneginf(lse), empty), "rows with no visible key must have LSE = -inf (and only they)"
    assert np.all(o[empty] == 0), "rows with no visible key must be zero"
    ok = ~empty
    if not ok.any():
        return 0.0, 0.0
    eo = float(np.max(np.abs(o[ok] - O_ref[ok])) / max(np.max(np.abs(O_ref[ok])), 1e-30))
    el = float(np.max(np.abs(lse[ok] - L_ref[ok])))
    say(f"    O err {eo:.2e}, LSE err {el:.2e}, empty rows {int(empty.sum())}")
    assert np.isfinite(eo) and eo <= O_TOL[dtype], f"O error {eo:.3e}"
    assert el <= LSE_TOL, f"LSE error {el:.3e}"
    return eo, el


def _lists_dev(lists, maxq, maxk):
    return fa.block_lists_to_tensors(lists, maxq, maxk, "cuda:0") if lists is not None else (None, None)


def run_fixed(q, k, v, window, lists=None, scale=None, label=""):
    B, Hq, Nq, d = q.shape
    Nk = k.shape[2]
    scale = float(np.float32(1 / np.sqrt(d))) if scale is None else scale
    say(f"[masked fixed] {label} q={tuple(q.shape)} k={tuple(k.shape)} window={window} lists={lists is not None}")
    bc, bi = _lists_dev(lists, Nq, Nk)
    qd, kd, vd = to_dev(q, k, v)
    o, lse = fa.fwd_masked(qd, kd, vd, window, scale, block_cnt=bc, block_idx=bi)
    torch.cuda.synchronize()
    O_ref, L_ref = om.attention_fwd_masked(q, k, v, scale, window=window, block_lists=lists)
    return _compare(o, lse, O_ref, L_ref, q.dtype)


def run_packed(q, k, v, lq, lk, window, lists=None, scale=None, label=""):
    Hq, Nq, d = q.shape
    Nk = k.shape[1]
    scale = float(np.float32(1 / np.sqrt(d))) if scale is None else scale
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    say(f"[masked packed] {label} lq={list(lq)[:6]} lk={list(lk)[:6]} H={Hq}/{k.shape[0]} d={d} window={window} "
        f"lists={lists is not None}")
    mq, mk = max(max(lq), 0), max(max(lk), 0)
    bc, bi = _lists_dev(lists, mq, mk)
    qd, kd, vd = to_dev(q, k, v)
    o, lse = fa.fwd_masked(qd, kd, vd, window, scale, torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda(),
                           mq, mk, bc, bi)
    torch.cuda.synchronize()
    O_ref, L_ref = om.attention_fwd_masked(q, k, v, scale, cq, ck, window, lists)
    return _compare(o, lse, O_ref, L_ref, q.dtype)


def _rand(seed, shape, dtype=torch.bfloat16):
    return workloads.randn(seed, shape, dtype)


def test_mask_workload_mix_small():
    w = workloads.MASK_WORKLOADS["mix_small_d64_bf16"]
    q, k, v, cq, ck, lists = workloads.make_mask_inputs(w)
    run_packed(q, k, v, w.seqlens_q, w.seqlens_k, w.window, lists, w.scale, label=w.name)


FIXED = [
    # (B, Hq, Hkv, Nq, Nk, d, window, dtype)
    (2, 4, 2, 300, 700, 128, (-1, 0), torch.bfloat16),
    (1, 4, 1, 700, 300, 64, (-1, 0), torch.float16),        # more queries than keys: empty rows
    (1, 2, 2, 513, 513, 128, (63, 0), torch.bfloat16),
    (1, 2, 1, 1000, 1000, 64, (100, 50), torch.float16),
    (1, 2, 2, 257, 300, 128, (0, 0), torch.bfloat16),        # one key per query at most
    (2, 2, 1, 129, 129, 64, (-1, 7), torch.bfloat16),
    (1, 1, 1, 1, 5000, 128, (-1, -1), torch.bfloat16),
    (1, 2, 2, 2049, 2049, 128, (511, 0), torch.bfloat16),
]


@pytest.mark.parametrize("case", FIXED, ids=lambda c: "B{}Hq{}Hkv{}Nq{}Nk{}d{}_w{}_{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5], f"{c[6][0]}_{c[6][1]}", str(c[7])[6:]))
def test_masked_fixed(case):
    B, Hq, Hkv, Nq, Nk, d, window, dt = case
    q, k, v = _rand(9800 + Nq, (B, Hq, Nq, d), dt), _rand(9801 + Nk, (B, Hkv, Nk, d), dt), _rand(9802, (B, Hkv, Nk, d), dt)
    run_fixed(q, k, v, window)


def _random_lists(seed, B, Hm, Lq, Lk, density):
    g = np.random.Generator(np.random.PCG64(seed))
    nqb, nkt = -(-Lq // 256), -(-Lk // 64)
    return [[[sorted(int(t) for t in np.nonzero(g.random(nkt) < density)[0]) for _ in range(nqb)]
             for _ in range(Hm)] for _ in range(B)]


@pytest.mark.parametrize("Hm,window,density", [(1, (-1, -1), 0.3), (4, (-1, 0), 0.5), (4, (200, 100), 0.7),
                                               (1, (-1, 0), 0.0)])
def test_masked_block_lists(Hm, window, density):
    B, Hq, Hkv, N, d = 2, 4, 2, 1100, 128
    q, k, v = _rand(9900, (B, Hq, N, d)), _rand(9901, (B, Hkv, N, d)), _rand(9902, (B, Hkv, N, d))
    lists = _random_lists(9903 + Hm, B, Hm, N, N, density)
    run_fixed(q, k, v, window, lists, label=f"Hm={Hm} density={density}")


def test_masked_packed_edge_sequences():
    lq, lk = [0, 1, 255, 256, 257, 600, 5], [3, 0, 255, 700, 1, 600, 64]
    Hq, Hkv, d = 4, 2, 128
    q, k, v = _rand(9950, (Hq, sum(lq), d)), _rand(9951, (Hkv, sum(lk), d)), _rand(9952, (Hkv, sum(lk), d))
    for window in ((-1, -1), (-1, 0), (30, 2)):
        run_packed(q, k, v, lq, lk, window, label="edge lengths")


def test_masked_equals_fwd_bitwise():
    q, k, v = to_dev(_rand(9960, (2, 8, 1000, 128)), _rand(9961, (2, 2, 1000, 128)), _rand(9962, (2, 2, 1000, 128)))
    say("[masked] equals fa_fwd bit for bit")
    for causal, window in ((False, (-1, -1)), (True, (-1, 0))):
        o1, l1 = fa.fwd(q, k, v, causal=causal)
        o2, l2 = fa.fwd_masked(q, k, v, window)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_masked_deterministic():
    w = workloads.MASK_WORKLOADS["mix_small_d64_bf16"]
    q, k, v, cq, ck, lists = workloads.make_mask_inputs(w)
    say("[masked] determinism")
    qd, kd, vd = to_dev(q, k, v)
    bc, bi = fa.block_lists_to_tensors(lists, max(w.seqlens_q), max(w.seqlens_k), "cuda:0")
    args = (w.window, w.scale, torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda(), max(w.seqlens_q),
            max(w.seqlens_k), bc, bi)
    o1, l1 = fa.fwd_masked(qd, kd, vd, *args)
    o2, l2 = fa.fwd_masked(qd, kd, vd, *args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_mask_workload_sliding_window_full_size():
    """The N=8192 sliding-window workload in the launch configuration the benchmark
    times, on sampled rows of every head."""
    w = workloads.MASK_WORKLOADS[workloads.MASK_HEADLINE]
    q, k, v, _, _, _ = workloads.make_mask_inputs(w)
    say(f"[masked] {w.name} full size, sampled rows")
    o, lse = fa.fwd_masked(*to_dev(q, k, v), w.window, w.scale)
    torch.cuda.synchronize()
    g = np.random.Generator(np.random.PCG64(11))
    rows = np.unique(np.concatenate([[0, 1, 1023, 1024, 1025, 4095, 8191], g.integers(0, 8192, 9)]))
    O_ref, L_ref = om.attention_fwd_masked(q, k, v, w.scale, window=w.window, rows=rows)
    _compare(o[:, :, rows], lse[:, :, rows], O_ref, L_ref, q.dtype)


@pytest.mark.parametrize("name", ["varlen_b8_hq32_hkv8_d128_bf16_causal", "bsparse_b1_hq16_hkv4_n8192_d128_bf16"])
def test_mask_workloads_full_size_sampled_heads(name):
    """Full-size packed and block-sparse workloads; the oracle runs on three sampled query
    heads (each with its K/V head; heads are independent problems)."""
    w = workloads.MASK_WORKLOADS[name]
    q, k, v, cq, ck, lists = workloads.make_mask_inputs(w)
    say(f"[masked] {w.name} full size, sampled heads")
    qd, kd, vd = to_dev(q, k, v)
    G = w.Hq // w.Hkv
    if w.packed:
        mq, mk = max(w.seqlens_q), max(w.seqlens_k)
        bc, bi = _lists_dev(lists, mq, mk)
        o, lse = fa.fwd_masked(qd, kd, vd, w.window, w.scale, torch.from_numpy(cq).cuda(),
                               torch.from_numpy(ck).cuda(), mq, mk, bc, bi)
    else:
        bc, bi = _lists_dev(lists, w.seqlens_q[0], w.seqlens_k[0])
        o, lse = fa.fwd_masked(qd, kd, vd, w.window, w.scale, block_cnt=bc, block_idx=bi)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    for h in (0, G + 1, w.Hq - 1):
        kh = slice(h // G, h // G + 1)
        if w.packed:
            O_ref, L_ref = om.attention_fwd_masked(q[h:h + 1], k[kh], v[kh], w.scale, cq, ck, w.window, lists)
            _compare(o[h:h + 1], lse[h:h + 1], O_ref, L_ref, q.dtype)
        else:
            O_ref, L_ref = om.attention_fwd_masked(q[:, h:h + 1], k[:, kh], v[:, kh], w.scale, window=w.window,
                                                   block_lists=lists)
            _compare(o[:, h:h + 1], lse[:, h:h + 1], O_ref, L_ref, q.dtype)


def test_masked_inconsistent_lists_stay_in_bounds():
    """Lists that break the contract (unsorted, repeated and out-of-range tiles, counts
    below 0 or above the row length) give unspecified values but no invalid access: the
    kernel clamps every count and tile; the output must be finite."""
    B, Hq, Hkv, N, d = 1, 4, 2, 700, 128
    q, k, v = to_dev(_rand(9970, (B, Hq, N, d)), _rand(9971, (B, Hkv, N, d)), _rand(9972, (B, Hkv, N, d)))
    nqb, cap = -(-N // 256), -(-N // 64)
    g = torch.Generator().manual_seed(9973)
    cnt = torch.randint(-3, cap + 6, (B, Hq, nqb), generator=g, dtype=torch.int32)
    idx = torch.randint(-10, 2 * cap, (B, Hq, nqb, cap), generator=g, dtype=torch.int32)
    say("[masked] inconsistent block lists")
    o, lse = fa.fwd_masked(q, k, v, (-1, -1), block_cnt=cnt.cuda(), block_idx=idx.cuda())
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    assert not torch.isnan(lse).any()
