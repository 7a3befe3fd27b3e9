"""Pins of the split-KV decoding oracle (oracle/decode.py) to facts outside itself.

* Square shapes reduce to the forward oracle, itself pinned in test_oracle_pins.py.
* One query, no mask: a scalar brute force with math.exp / math.fsum.
* Bottom-right alignment, closed form: with K = 0 every visible score is 0, so query
  i averages V over keys 0 .. Nk-Nq+i and LSE_i = ln(Nk-Nq+i+1).
* The last query sees every key, causal or not.
* The combine is the algebraic identity of the "Flash Attention" wiki's
  "Flash-Decoding" section: merging parts over any partition of the keys gives the
  unsplit result; one part is returned unchanged; an empty (-inf) part has no weight;
  parts with huge statistics stay finite (the max is subtracted first).
Each planted mistake in MUTANTS must fail at least one pin.
"""
from __future__ import annotations

import math
import types

import numpy as np
import pytest
import torch

import oracle
import oracle.decode as oracle_decode
from workloads import randn


def _case(seed, B=1, Hq=4, Hkv=2, Nq=5, Nk=37, d=8):
    q = randn(seed, (B, Hq, Nq, d), torch.float32)
    k = randn(seed + 1, (B, Hkv, Nk, d), torch.float32)
    v = randn(seed + 2, (B, Hkv, Nk, d), torch.float32)
    return q, k, v


def pin_square_is_forward(mod):
    q, k, v = _case(11, Nq=40, Nk=40)
    for causal in (False, True):
        O, L = mod.attention_fwd_kv(q, k, v, causal, 0.3)
        O2, L2 = oracle.attention_fwd(q, k, v, causal, 0.3)
        assert np.allclose(O, O2, atol=1e-13, rtol=0) and np.allclose(L, L2, atol=1e-13, rtol=0)


def pin_one_query_brute_force(mod):
    q, k, v = _case(12, B=1, Hq=2, Hkv=1, Nq=1, Nk=7, d=3)
    O, L = mod.attention_fwd_kv(q, k, v, False, 0.7)
    Q, K, V = q.double().numpy(), k.double().numpy(), v.double().numpy()
    for h in range(2):
        s = [0.7 * math.fsum(Q[0, h, 0, c] * K[0, 0, j, c] for c in range(3)) for j in range(7)]
        e = [math.exp(x) for x in s]
        tot = math.fsum(e)
        assert abs(L[0, h, 0] - math.log(tot)) < 1e-13
        for c in range(3):
            ref = math.fsum(e[j] * V[0, 0, j, c] for j in range(7)) / tot
            assert abs(O[0, h, 0, c] - ref) < 1e-13


def pin_bottom_right_closed_form(mod):
    q, _, v = _case(13, Nq=6, Nk=20)
    k = torch.zeros(1, 2, 20, 8)
    O, L = mod.attention_fwd_kv(q, k, v, True, 0.5)
    V = v.double().numpy()
    for h in range(4):
        for i in range(6):
            n = 20 - 6 + i + 1
            assert abs(L[0, h, i] - math.log(n)) < 1e-13
            assert np.allclose(O[0, h, i], V[0, h // 2, :n].mean(axis=0), atol=1e-13, rtol=0)


def pin_last_query_sees_all(mod):
    q, k, v = _case(14, Nq=9, Nk=50)
    Oc, Lc = mod.attention_fwd_kv(q, k, v, True, 0.4)
    On, Ln = mod.attention_fwd_kv(q, k, v, False, 0.4)
    assert np.allclose(Oc[:, :, -1], On[:, :, -1], atol=1e-14, rtol=0)
    assert np.allclose(Lc[:, :, -1], Ln[:, :, -1], atol=1e-14, rtol=0)
    assert not np.allclose(Lc[:, :, 0], Ln[:, :, 0])


def _merge_case(mod, cuts, causal):
    q, k, v = _case(15, Nq=8, Nk=37)
    parts = [mod.attention_fwd_kv(q, k, v, causal, 0.35, (a, b)) for a, b in zip(cuts[:-1], cuts[1:])]
    Op = np.stack([p[0] for p in parts], axis=-2)
    Lp = np.stack([p[1] for p in parts], axis=-1)
    O, L = mod.lse_combine(Op, Lp)
    Of, Lf = mod.attention_fwd_kv(q, k, v, causal, 0.35)
    assert np.allclose(O, Of, atol=1e-12, rtol=0) and np.allclose(L, Lf, atol=1e-12, rtol=0)


def pin_combine_of_partition_is_whole(mod):
    for causal in (False, True):
        for cuts in ((0, 13, 37), (0, 1, 2, 36, 37), (0, 20, 20, 37), (0, 30, 33, 37)):
            _merge_case(mod, cuts, causal)


def pin_combine_identities(mod):
    g = np.random.default_rng(16)
    Op = g.standard_normal((3, 4, 6))
    Lp = g.standard_normal((3, 4))
    O1, L1 = mod.lse_combine(Op[:, :1], Lp[:, :1])
    assert np.allclose(O1, Op[:, 0], atol=1e-15) and np.allclose(L1, Lp[:, 0], atol=1e-15)
    Lz = Lp.copy()
    Lz[:, 2] = -np.inf
    Oa, La = mod.lse_combine(Op, Lz)
    Ob, Lb = mod.lse_combine(Op[:, [0, 1, 3]], Lp[:, [0, 1, 3]])
    assert np.allclose(Oa, Ob, atol=1e-14) and np.allclose(La, Lb, atol=1e-14)
    perm = [2, 0, 3, 1]
    Oc, Lc = mod.lse_combine(Op[:, perm], Lp[:, perm])
    Od, Ld = mod.lse_combine(Op, Lp)
    assert np.allclose(Oc, Od, atol=1e-14) and np.allclose(Lc, Ld, atol=1e-14)
    # huge statistics: weights e^0 and e^1 relative to the max, result exact and finite
    Oh, Lh = mod.lse_combine(np.array([[[1.0, 0.0], [0.0, 1.0]]]), np.array([[800.0, 801.0]]))
    e = math.exp(-1.0)
    assert np.allclose(Oh, [[e / (1 + e), 1 / (1 + e)]], atol=1e-15)
    assert abs(Lh[0] - (801.0 + math.log(1 + e))) < 1e-12
    # all parts empty
    Oe, Le = mod.lse_combine(np.ones((1, 2, 3)), np.full((1, 2), -np.inf))
    assert np.all(Oe == 0) and np.all(np.isneginf(Le))


PINS = [pin_square_is_forward, pin_one_query_brute_force, pin_bottom_right_closed_form,
        pin_last_query_sees_all, pin_combine_of_partition_is_whole, pin_combine_identities]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_decode_oracle_pins(pin):
    pin(oracle_decode)


MUTANTS = {
    "top_left_causal_alignment": ("pos = Nk - Nq + np.arange(Nq)", "pos = np.arange(Nq)"),
    "causal_masks_diagonal": ("S[pos[:, None] < keys[None, :]]", "S[pos[:, None] <= keys[None, :]]"),
    "combine_not_normalised": ("num / np.where(any_part, den, 1.0)[..., None]", "num"),
    "combine_lse_without_max": ("Msafe + np.log(np.where(any_part, den, 1.0))", "np.log(np.where(any_part, den, 1.0))"),
    "combine_without_max_shift": ("w = np.exp(Lp - Msafe[..., None])", "w = np.exp(Lp)"),
    "key_range_inclusive": ("keys = np.arange(lo, hi)", "keys = np.arange(lo, hi + 1)[: hi - lo]; hi = hi + (hi < Nk)"),
    "partial_lse_log2": ("LSE[b, h, ok] = m[ok] + np.log(l[ok])", "LSE[b, h, ok] = m[ok] + np.log2(l[ok])"),
}


def _mutant(old, new):
    src = open(oracle_decode.__file__).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_decode_mutant")
    exec(compile(src.replace(old, new), "oracle_decode_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_decode_pins_catch_planted_mistake(name):
    mod = _mutant(*MUTANTS[name])
    failed = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(mod)
            except (AssertionError, ValueError, IndexError, FloatingPointError):
                failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {name}"
