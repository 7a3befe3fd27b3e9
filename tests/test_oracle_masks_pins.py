"""Pins of the mask-family oracle (oracle/masks.py) to facts outside itself.

* No mask and the causal window reduce to the square forward oracle (pinned in
  test_oracle_pins.py); queries shorter than keys under the causal window reduce to the
  split-KV oracle's bottom-right alignment (pinned in test_oracle_decode_pins.py); longer
  queries leave the first Nq - Nk rows empty and the rest equal the square causal case.
* Packed batches equal their sequences run one at a time through that oracle.
* Closed form: with K = 0 every visible score is 0, so O_i is the mean of V over the
  visible keys and LSE_i = ln(count_i), the count taken from the window's interval
  arithmetic written out per row.
* Dropping a tile from a block list equals deleting its keys; listing every tile equals
  no list; an empty list (or no keys) gives O = 0 and LSE = -inf.
* A scalar brute force (math.exp, math.fsum) over a packed batch with a window and
  block lists.
* Pair counts: N(N+1)/2 for the square causal case, and the window's closed form.
* Backward: reduces to the square backward oracle; central finite differences through
  the forward (a packed batch with a window, and again with block lists that skip a
  tile); closed forms for keys no query sees and rows with no key; with block lists,
  each (head, query block) equals the backward of its queries against only its listed
  keys, the key gradients summed over the blocks.
Each planted mistake in MUTANTS must fail at least one pin.
"""
from __future__ import annotations

import math
import types

import numpy as np
import pytest
import torch

import oracle
import oracle.decode as odec
import oracle.masks as omasks
from workloads import randn


def _fixed(seed, B=1, Hq=4, Hkv=2, Nq=70, Nk=70, d=8):
    return (randn(seed, (B, Hq, Nq, d), torch.float32).double().numpy(),
            randn(seed + 1, (B, Hkv, Nk, d), torch.float32).double().numpy(),
            randn(seed + 2, (B, Hkv, Nk, d), torch.float32).double().numpy())


def pin_reduces_to_square_oracle(mod):
    q, k, v = _fixed(1)
    for window, causal in (((-1, -1), False), ((-1, 0), True)):
        O, L = mod.attention_fwd_masked(q, k, v, 0.3, window=window)
        O2, L2 = oracle.attention_fwd(q, k, v, causal, 0.3)
        assert np.allclose(O, O2, atol=1e-13, rtol=0) and np.allclose(L, L2, atol=1e-13, rtol=0)


def pin_short_queries_bottom_right(mod):
    q, k, v = _fixed(2, Nq=9, Nk=130)
    for window, causal in (((-1, 0), True), ((-1, -1), False)):
        O, L = mod.attention_fwd_masked(q, k, v, 0.4, window=window)
        O2, L2 = odec.attention_fwd_kv(q, k, v, causal, 0.4)
        assert np.allclose(O, O2, atol=1e-13, rtol=0) and np.allclose(L, L2, atol=1e-13, rtol=0)


def pin_long_queries(mod):
    q, k, v = _fixed(3, Nq=50, Nk=20)
    O, L = mod.attention_fwd_masked(q, k, v, 0.4, window=(-1, 0))
    assert np.all(O[:, :, :30] == 0) and np.all(L[:, :, :30] == -np.inf)
    O2, L2 = oracle.attention_fwd(q[:, :, 30:], k, v, True, 0.4)
    assert np.allclose(O[:, :, 30:], O2, atol=1e-13, rtol=0) and np.allclose(L[:, :, 30:], L2, atol=1e-13, rtol=0)


def _packed(seed, lq, lk, Hq=4, Hkv=2, d=8):
    cq, ck = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q = randn(seed, (Hq, cq[-1], d), torch.float32).double().numpy()
    k = randn(seed + 1, (Hkv, ck[-1], d), torch.float32).double().numpy()
    v = randn(seed + 2, (Hkv, ck[-1], d), torch.float32).double().numpy()
    return q, k, v, cq, ck


def pin_packed_is_per_sequence(mod):
    lq, lk = [5, 40, 1, 33], [5, 70, 30, 33]
    q, k, v, cq, ck = _packed(4, lq, lk)
    for causal in (False, True):
        O, L = mod.attention_fwd_masked(q, k, v, 0.35, cq, ck, window=(-1, 0) if causal else (-1, -1))
        for b in range(4):
            sq, sk = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
            O2, L2 = odec.attention_fwd_kv(q[None, :, sq], k[None, :, sk], v[None, :, sk], causal, 0.35)
            assert np.allclose(O[:, sq], O2[0], atol=1e-13, rtol=0)
            assert np.allclose(L[:, sq], L2[0], atol=1e-13, rtol=0)


def pin_window_closed_form(mod):
    Nq, Nk = 40, 55
    q, _, v = _fixed(5, Nq=Nq, Nk=Nk)
    k = np.zeros((1, 2, Nk, 8))
    for left, right in ((5, 0), (0, 0), (3, 7), (-1, 2), (12, -1)):
        O, L = mod.attention_fwd_masked(q, k, v, 0.5, window=(left, right))
        for i in range(Nq):
            p = i + Nk - Nq
            lo = 0 if left < 0 else max(0, p - left)
            hi = Nk - 1 if right < 0 else min(Nk - 1, p + right)
            cnt = hi - lo + 1
            if cnt <= 0:
                assert np.all(O[0, :, i] == 0) and np.all(L[0, :, i] == -np.inf)
                continue
            assert np.allclose(L[0, :, i], math.log(cnt), atol=1e-13, rtol=0)
            ref = v[0, :, lo:hi + 1].mean(axis=1)                       # [Hkv, d]
            assert np.allclose(O[0, :, i], np.repeat(ref, 2, axis=0), atol=1e-13, rtol=0)


def pin_block_lists(mod):
    Nq, Nk = 300, 200                      # query blocks of 256: 2; key tiles of 64: 4
    q, k, v = _fixed(6, Hq=2, Hkv=1, Nq=Nq, Nk=Nk)
    every = [[[[0, 1, 2, 3], [0, 1, 2, 3]]]]          # [B][Hm][query block] -> tiles
    O, L = mod.attention_fwd_masked(q, k, v, 0.3, block_lists=every)
    O2, L2 = mod.attention_fwd_masked(q, k, v, 0.3)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)
    # drop tile 1 for query block 0 = delete keys 64..127 for queries 0..255
    lists = [[[[0, 2, 3], [0, 1, 2, 3]]]]
    O, L = mod.attention_fwd_masked(q, k, v, 0.3, block_lists=lists)
    keep = np.r_[0:64, 128:200]
    O3, L3 = odec.attention_fwd_kv(q[:, :, :256], k[:, :, keep], v[:, :, keep], False, 0.3)
    assert np.allclose(O[:, :, :256], O3, atol=1e-13, rtol=0) and np.allclose(L[:, :, :256], L3, atol=1e-13, rtol=0)
    assert np.allclose(O[:, :, 256:], O2[:, :, 256:], atol=1e-13, rtol=0)
    # per-head lists, and an empty list -> zero rows with LSE = -inf
    q2, k2, v2 = _fixed(7, B=2, Hq=2, Hkv=1, Nq=Nq, Nk=Nk)
    lists = [[[[0, 1, 2, 3], []], [[], [3]]], [[[1], [0, 3]], [[2], [2]]]]
    O, L = mod.attention_fwd_masked(q2, k2, v2, 0.3, block_lists=lists)
    assert np.all(O[0, 0, 256:] == 0) and np.all(L[0, 0, 256:] == -np.inf)
    assert np.all(O[0, 1, :256] == 0) and np.all(L[0, 1, :256] == -np.inf)
    O4, L4 = odec.attention_fwd_kv(q2[1:, 1:, 256:], k2[1:, :, 128:192], v2[1:, :, 128:192], False, 0.3)
    assert np.allclose(O[1, 1, 256:], O4[0, 0], atol=1e-13, rtol=0) and np.allclose(L[1, 1, 256:], L4[0, 0], atol=1e-13)


def pin_empty_sequences(mod):
    q, k, v, cq, ck = _packed(8, [3, 4, 0], [0, 6, 5])
    O, L = mod.attention_fwd_masked(q, k, v, 0.3, cq, ck)
    assert np.all(O[:, 0:3] == 0) and np.all(L[:, 0:3] == -np.inf)
    assert np.all(np.isfinite(L[:, 3:7]))


def pin_scalar_brute_force(mod):
    lq, lk = [7, 3, 9], [7, 12, 4]
    q, k, v, cq, ck = _packed(9, lq, lk, Hq=2, Hkv=1, d=3)
    window = (2, 1)
    lists = [[[[0]]], [[[0]]], [[[0]]]]                 # per sequence: one list for all heads, tile 0
    O, L = mod.attention_fwd_masked(q, k, v, 0.7, cq, ck, window=window, block_lists=lists)
    for b in range(3):
        for h in range(2):
            for i in range(lq[b]):
                p = i + lk[b] - lq[b]
                js = [j for j in range(lk[b]) if p - 2 <= j <= p + 1]
                if not js:
                    assert L[h, cq[b] + i] == -np.inf
                    continue
                s = [0.7 * math.fsum(q[h, cq[b] + i, c] * k[0, ck[b] + j, c] for c in range(3)) for j in js]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                tot = math.fsum(e)
                assert abs(L[h, cq[b] + i] - (mx + math.log(tot))) < 1e-13
                for c in range(3):
                    ref = math.fsum(e[t] * v[0, ck[b] + j, c] for t, j in enumerate(js)) / tot
                    assert abs(O[h, cq[b] + i, c] - ref) < 1e-13


def pin_pair_counts(mod):
    assert mod.visible_pairs([100], [100], (-1, 0)) == 100 * 101 // 2
    # causal window of w keys (left = w - 1): rows i >= w - 1 see w keys, earlier rows i + 1
    w, n = 16, 100
    assert mod.visible_pairs([n], [n], (w - 1, 0)) == sum(min(i + 1, w) for i in range(n))
    assert mod.visible_pairs([5, 300], [9, 300], (-1, -1)) == 45 + 90000


def pin_bwd_reduces_to_square_oracle(mod):
    q, k, v = _fixed(20, Hq=4, Hkv=2, Nq=40, Nk=40)
    do = randn(23, q.shape, torch.float32).double().numpy()
    for window, causal in (((-1, -1), False), ((-1, 0), True)):
        g1 = mod.attention_bwd_masked(q, k, v, do, 0.3, window=window)
        g2 = oracle.attention_bwd(q, k, v, do, causal, 0.3)
        for a, b in zip(g1, g2):
            assert np.allclose(a, b, atol=1e-12, rtol=0)


def pin_bwd_finite_differences(mod):
    # a packed batch with a two-sided window, unequal lengths and an empty sequence:
    # gradients of L = sum(O * W) against central differences
    lq, lk = [5, 0, 7], [9, 3, 4]
    q, k, v, cq, ck = _packed(24, lq, lk, Hq=2, Hkv=1, d=3)
    W = randn(28, q.shape, torch.float32).double().numpy()
    window = (3, 1)
    dq, dk, dv = mod.attention_bwd_masked(q, k, v, W, 0.6, cq, ck, window)

    def loss(qq, kk, vv):
        O, _ = mod.attention_fwd_masked(qq, kk, vv, 0.6, cq, ck, window)
        return float((O * W).sum())

    eps = 1e-6
    for X, g in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(*X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += eps
            Xm[idx] -= eps
            args_p = [Xp if Y is X else Y for Y in (q, k, v)]
            args_m = [Xm if Y is X else Y for Y in (q, k, v)]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - g[idx]) < 1e-7 * max(1.0, abs(fd)), (idx, fd, g[idx])


def pin_bwd_unseen_keys_and_empty_rows(mod):
    # window (0, 0) with Nq = Nk: each query sees only its own key; with Nk > Nq the first
    # Nk - Nq keys are seen by nobody (zero dK, dV); with Nq > Nk the first rows see none
    q, k, v = _fixed(30, Hq=2, Hkv=1, Nq=10, Nk=14, d=4)
    do = randn(33, q.shape, torch.float32).double().numpy()
    dq, dk, dv = mod.attention_bwd_masked(q, k, v, do, 0.5, window=(0, 0))
    assert np.all(dk[:, :, :4] == 0) and np.all(dv[:, :, :4] == 0)
    # a single visible key per row: softmax is 1, so dV_j = sum of dO over the rows that see j
    assert np.allclose(dv[0, 0, 4:], do[0, 0] + do[0, 1], atol=1e-13)
    assert np.allclose(dq, 0, atol=1e-13)        # P = 1 exactly: no dependence on the scores
    q2, k2, v2 = _fixed(31, Hq=2, Hkv=1, Nq=12, Nk=5, d=4)
    do2 = randn(34, q2.shape, torch.float32).double().numpy()
    dq2, _, _ = mod.attention_bwd_masked(q2, k2, v2, do2, 0.5, window=(-1, 0))
    assert np.all(dq2[:, :, :7] == 0)


def pin_bwd_block_lists_as_deleted_keys(mod):
    # full attention, per-head lists over two query blocks: each (head, query block) is the
    # backward of its queries against only its listed keys; dK, dV of a key sum over the
    # blocks that list it; unlisted keys and the rows of an empty list get zeros
    Hq, Nq, Nk = 2, 300, 200
    q, k, v = _fixed(40, Hq=Hq, Hkv=1, Nq=Nq, Nk=Nk, d=4)
    do = randn(43, q.shape, torch.float32).double().numpy()
    lists = [[[[0, 2], [1, 3]], [[3], []]]]
    dq, dk, dv = mod.attention_bwd_masked(q, k, v, do, 0.4, block_lists=lists)
    eq, ek, ev = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for h in range(Hq):
        for qb, tiles in enumerate(lists[0][h]):
            if not tiles:
                continue
            rows = np.arange(256 * qb, min(256 * qb + 256, Nq))
            keys = np.concatenate([np.arange(64 * t, min(64 * t + 64, Nk)) for t in tiles])
            g = mod.attention_bwd_masked(q[:, h:h + 1, rows], k[:, :, keys], v[:, :, keys], do[:, h:h + 1, rows], 0.4)
            eq[:, h:h + 1, rows] = g[0]
            ek[:, :, keys] += g[1]
            ev[:, :, keys] += g[2]
    for a, b in zip((dq, dk, dv), (eq, ek, ev)):
        assert np.allclose(a, b, atol=1e-12, rtol=0)
    assert np.all(dq[0, 1, 256:] == 0)


def pin_bwd_block_lists_finite_differences(mod):
    # a packed batch with a window, unequal lengths and lists that skip a key tile the
    # window would show: gradients of L = sum(O * W) against central differences
    lq, lk = [6, 3], [150, 70]
    q, k, v, cq, ck = _packed(44, lq, lk, Hq=1, Hkv=1, d=2)
    W = randn(48, q.shape, torch.float32).double().numpy()
    window = (100, 10)
    lists = [[[[0, 2]]], [[[1]]]]
    dq, dk, dv = mod.attention_bwd_masked(q, k, v, W, 0.7, cq, ck, window, lists)
    assert np.all(dk[:, 64:128] == 0) and np.all(dv[:, 150:150 + 64] == 0)

    def loss(qq, kk, vv):
        O, _ = mod.attention_fwd_masked(qq, kk, vv, 0.7, cq, ck, window, lists)
        return float((O * W).sum())

    eps = 1e-6
    for X, g in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(*X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += eps
            Xm[idx] -= eps
            args_p = [Xp if Y is X else Y for Y in (q, k, v)]
            args_m = [Xm if Y is X else Y for Y in (q, k, v)]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - g[idx]) < 1e-7 * max(1.0, abs(fd)), (idx, fd, g[idx])


PINS = [pin_reduces_to_square_oracle, pin_short_queries_bottom_right, pin_long_queries, pin_packed_is_per_sequence,
        pin_window_closed_form, pin_block_lists, pin_empty_sequences, pin_scalar_brute_force, pin_pair_counts,
        pin_bwd_reduces_to_square_oracle, pin_bwd_finite_differences, pin_bwd_unseen_keys_and_empty_rows,
        pin_bwd_block_lists_as_deleted_keys, pin_bwd_block_lists_finite_differences]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_masks_oracle_pins(pin):
    pin(omasks)


MUTANTS = {
    "top_left_alignment": ("p = i + (Lk - Lq)", "p = i"),
    "window_left_off_by_one": ("vis &= j >= p - left", "vis &= j > p - left"),
    "window_right_off_by_one": ("vis &= j <= p + right", "vis &= j < p + right"),
    "query_block_128": ("vis &= tile_ok[i // QBLOCK,", "vis &= tile_ok[i // 128,"),
    "empty_row_lse_zero": ("L = np.full(Lq, -np.inf)", "L = np.zeros(Lq)"),
    "packed_keys_from_query_offsets": ("K[h // G, ks:ke], V[h // G, ks:ke]", "K[h // G, qs:qe], V[h // G, qs:qe]"),
    "gqa_modulo": ("_attend(Q[b, h, r], K[b, h // G], V[b, h // G]", "_attend(Q[b, h, r], K[b, h % Hkv], V[b, h % Hkv]"),
    "block_list_first_head_always": ("return hm[0] if len(hm) == 1 else hm[h]", "return hm[0]"),
    "bwd_without_jacobian_term": ("dS = P * (dP - Dr[:, None])", "dS = P * dP"),
    "bwd_dk_unscaled": ("dKb = scale * (dS.T @ Qb)", "dKb = dS.T @ Qb"),
    "bwd_ignores_window": ("vis = visible(Qb.shape[0], Kb.shape[0], window, kl)",
                           "vis = visible(Qb.shape[0], Kb.shape[0], kept_tiles=kl)"),
    "bwd_ignores_block_lists": ("vis = visible(Qb.shape[0], Kb.shape[0], window, kl)",
                                "vis = visible(Qb.shape[0], Kb.shape[0], window)"),
}


def _mutant(old, new):
    src = open(omasks.__file__).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle.masks_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "oracle_masks_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_masks_pins_catch_planted_mistake(name):
    mod = _mutant(*MUTANTS[name])
    failed = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(mod)
            except (AssertionError, ValueError, IndexError, FloatingPointError):
                failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {name}"
