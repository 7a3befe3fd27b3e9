"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics (CPU only).

Each check is written independently of the oracle's code: scalar loops with
math.fsum / math.exp, closed forms, invariants, finite differences, a library
routine (torch's fp64 autograd on CPU), and the pages' printed numbers under
tests/golden/.  The mutation tests at the end plant plausible mistakes in a copy
of the oracle's source and check that at least one pin fails for each.
"""
from __future__ import annotations

import csv
import json
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oracle_attention
from exact_io_aware_fwd_amd import metrics

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng_case(seed, B, Hq, Hkv, N, d, scale_q=1.0):
    g = np.random.default_rng(seed)
    q = g.standard_normal((B, Hq, N, d)) * scale_q
    k = g.standard_normal((B, Hkv, N, d))
    v = g.standard_normal((B, Hkv, N, d))
    do = g.standard_normal((B, Hq, N, d))
    return q, k, v, do


# ----------------------------------------------------------------------------
# independent scalar brute force (pure Python; no numpy linear algebra)

def brute_fwd_head(q, k, v, causal, scale):
    """One head: q, k, v as nested lists [N][d]. Returns (O [N][d], LSE [N])."""
    N, d = len(q), len(q[0])
    O, LSE = [], []
    for i in range(N):
        keys = [j for j in range(N) if (not causal) or j <= i]
        s = [scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in keys]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        Z = math.fsum(w)
        O.append([math.fsum(w[a] * v[keys[a]][t] for a in range(len(keys))) / Z for t in range(d)])
        LSE.append(mx + math.log(Z))
    return O, LSE


def brute_fwd(q, k, v, causal, scale):
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    O = np.zeros((B, Hq, N, d))
    L = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            kh = h // (Hq // Hkv)
            o, l = brute_fwd_head(q[b, h].tolist(), k[b, kh].tolist(), v[b, kh].tolist(), causal, scale)
            O[b, h] = np.array(o)
            L[b, h] = np.array(l)
    return O, L


# ----------------------------------------------------------------------------
# pin checks, parameterised by the oracle module so that mutants can be run through them

def check_rows_sum_to_one(orc):
    q, k, _, _ = rng_case(1, 1, 1, 1, 37, 8)
    for causal in (False, True):
        P = orc.attention_probs(q[0, 0], k[0, 0], causal, 0.3)
        assert np.all(P >= 0)
        assert np.max(np.abs(P.sum(axis=1) - 1.0)) < 1e-12
        if causal:
            assert np.all(P[np.triu_indices(37, 1)] == 0.0)


def check_constant_v(orc):
    q, k, _, do = rng_case(2, 1, 2, 1, 29, 6)
    c = np.array([0.5, -1.25, 3.0, 0.0, 7.5, -2.0])
    v = np.broadcast_to(c, (1, 1, 29, 6)).copy()
    for causal in (False, True):
        O, _ = orc.attention_fwd(q, k, v, causal, 0.4)
        assert np.max(np.abs(O - c)) <= 1e-14 * 8
        dQ, dK, dV = orc.attention_bwd(q, k, v, do, causal, 0.4)
        assert np.max(np.abs(dQ)) < 1e-12
        assert np.max(np.abs(dK)) < 1e-12
        # dV = sum over the group of P^T dO
        ref = sum(orc.attention_probs(q[0, h], k[0, 0], causal, 0.4).T @ do[0, h] for h in range(2))
        assert np.max(np.abs(dV[0, 0] - ref)) < 1e-12


def check_causal_row0(orc):
    q, k, v, _ = rng_case(3, 2, 3, 3, 19, 5)
    scale = 0.7
    O, L = orc.attention_fwd(q, k, v, True, scale)
    assert np.array_equal(O[:, :, 0], v[:, :, 0])
    for b in range(2):
        for h in range(3):
            ref = scale * math.fsum(q[b, h, 0, t] * k[b, h, 0, t] for t in range(5))
            assert abs(L[b, h, 0] - ref) < 1e-13


def check_naive_lse(orc):
    # moderate scores (|S| << 709) so that ln(sum(exp(S))) needs no max shift
    q, k, v, _ = rng_case(4, 1, 2, 1, 23, 4, scale_q=3.0)
    scale = 0.9
    for causal in (False, True):
        _, L = orc.attention_fwd(q, k, v, causal, scale)
        for h in range(2):
            for i in range(23):
                terms = [math.exp(scale * math.fsum(q[0, h, i, t] * k[0, 0, j, t] for t in range(4)))
                         for j in range(23) if (not causal) or j <= i]
                assert abs(L[0, h, i] - math.log(math.fsum(terms))) < 1e-12


def check_closed_forms(orc):
    g = np.random.default_rng(5)
    # N = 1: O = V, LSE = scale q.k, dQ = dK = 0, dV = dO
    q, k, v, do = (g.standard_normal((1, 1, 1, 7)) for _ in range(4))
    for causal in (False, True):
        O, L = orc.attention_fwd(q, k, v, causal, 0.6)
        assert np.allclose(O, v, rtol=0, atol=1e-15)
        assert abs(L[0, 0, 0] - 0.6 * math.fsum(q[0, 0, 0] * k[0, 0, 0])) < 1e-14
        dQ, dK, dV = orc.attention_bwd(q, k, v, do, causal, 0.6)
        assert np.max(np.abs(dQ)) == 0 or np.max(np.abs(dQ)) < 1e-15
        assert np.max(np.abs(dK)) < 1e-15
        assert np.allclose(dV, do, rtol=0, atol=1e-15)
    # N = 2, non-causal: O_0 = sigma(s00 - s01) v0 + sigma(s01 - s00) v1
    q, k, v = (g.standard_normal((1, 1, 2, 3)) for _ in range(3))
    O, _ = orc.attention_fwd(q, k, v, False, 1.1)
    s00 = 1.1 * math.fsum(q[0, 0, 0] * k[0, 0, 0])
    s01 = 1.1 * math.fsum(q[0, 0, 0] * k[0, 0, 1])
    sig = 1.0 / (1.0 + math.exp(-(s00 - s01)))
    ref = sig * v[0, 0, 0] + (1 - sig) * v[0, 0, 1]
    assert np.max(np.abs(O[0, 0, 0] - ref)) < 1e-14


def check_shift_invariance(orc):
    q, k, v, _ = rng_case(6, 1, 2, 1, 31, 8)
    u = np.random.default_rng(7).standard_normal(8)
    scale = 0.5
    for causal in (False, True):
        O1, L1 = orc.attention_fwd(q, k, v, causal, scale)
        O2, L2 = orc.attention_fwd(q, k + u, v, causal, scale)
        assert np.max(np.abs(O1 - O2)) < 1e-12
        assert np.max(np.abs((L2 - L1) - scale * (q @ u))) < 1e-12


def check_brute_force(orc):
    cases = [(1, 2, 1, 1, 1), (1, 1, 1, 9, 2), (2, 2, 1, 16, 3), (1, 4, 2, 7, 64), (1, 1, 1, 13, 64)]
    for seed, (B, Hq, Hkv, N, d) in enumerate(cases):
        q, k, v, _ = rng_case(100 + seed, B, Hq, Hkv, N, d)
        for causal in (False, True):
            O, L = orc.attention_fwd(q, k, v, causal, 1 / math.sqrt(d))
            Ob, Lb = brute_fwd(q, k, v, causal, 1 / math.sqrt(d))
            assert np.max(np.abs(O - Ob)) < 1e-13
            assert np.max(np.abs(L - Lb)) < 1e-13


def fd_grads(q, k, v, do, causal, scale, h=1e-5):
    """Central differences of L = sum(dO * O) with the scalar brute-force forward."""
    def loss(q_, k_, v_):
        return float(np.sum(do * brute_fwd(q_, k_, v_, causal, scale)[0]))
    grads = []
    for which in range(3):
        arrs = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(arrs[which])
        for idx in np.ndindex(*g.shape):
            plus = [a.copy() for a in arrs]
            minus = [a.copy() for a in arrs]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        grads.append(g)
    return grads


def check_finite_differences(orc):
    for causal in (False, True):
        q, k, v, do = rng_case(8, 1, 2, 1, 5, 3)
        scale = 0.8
        dQ, dK, dV = orc.attention_bwd(q, k, v, do, causal, scale)
        fq, fk, fv = fd_grads(q, k, v, do, causal, scale)
        for a, b in ((dQ, fq), (dK, fk), (dV, fv)):
            assert np.max(np.abs(a - b)) < 1e-7 * max(1.0, np.max(np.abs(b)))


def check_gradient_invariants(orc):
    q, k, v, do = rng_case(9, 1, 4, 2, 33, 8)
    for causal in (False, True):
        _, _, dV = orc.attention_bwd(q, k, v, do, causal, 0.35)
        # rows of P sum to 1, so sum_j dV_j = sum_i dO_i over the heads sharing a K/V head
        for kh in range(2):
            ref = do[0, 2 * kh:2 * kh + 2].sum(axis=(0, 1))
            assert np.max(np.abs(dV[0, kh].sum(axis=0) - ref)) < 1e-11
    # constant K: every row of dS sums to zero, so dQ = 0
    kc = np.broadcast_to(k[:, :, :1], k.shape).copy()
    for causal in (False, True):
        dQ, _, _ = orc.attention_bwd(q, kc, v, do, causal, 0.35)
        assert np.max(np.abs(dQ)) < 1e-12


def check_gqa_is_head_expansion(orc):
    # contiguous groups: K/V head kh serves query heads [kh*G, (kh+1)*G)
    q, k, v, do = rng_case(10, 2, 6, 2, 11, 4)
    ke, ve = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    for causal in (False, True):
        O, L = orc.attention_fwd(q, k, v, causal, 0.5)
        Oe, Le = orc.attention_fwd(q, ke, ve, causal, 0.5)
        assert np.max(np.abs(O - Oe)) < 1e-14 and np.max(np.abs(L - Le)) < 1e-14
        dQ, dK, dV = orc.attention_bwd(q, k, v, do, causal, 0.5)
        dQe, dKe, dVe = orc.attention_bwd(q, ke, ve, do, causal, 0.5)
        assert np.max(np.abs(dQ - dQe)) < 1e-13
        assert np.max(np.abs(dK - dKe.reshape(2, 2, 3, 11, 4).sum(axis=2))) < 1e-13
        assert np.max(np.abs(dV - dVe.reshape(2, 2, 3, 11, 4).sum(axis=2))) < 1e-13


def check_row_subset(orc):
    q, k, v, _ = rng_case(11, 1, 2, 2, 600, 8)   # crosses the oracle's 512-row chunk
    rows = np.array([0, 1, 255, 511, 512, 599])
    for causal in (False, True):
        O, L = orc.attention_fwd(q, k, v, causal, 0.3)
        Os, Ls = orc.attention_fwd(q, k, v, causal, 0.3, rows=rows)
        # BLAS may block a 6-row product differently from a 512-row one: rounding only
        assert np.max(np.abs(O[:, :, rows] - Os)) < 1e-14 and np.max(np.abs(L[:, :, rows] - Ls)) < 1e-13


def check_torch_autograd(orc):
    """Library cross-check: torch's fp64 CPU attention math and autograd."""
    q, k, v, do = rng_case(12, 2, 4, 2, 40, 16)
    for causal in (False, True):
        tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
        kk = tk.repeat_interleave(2, dim=1)
        vv = tv.repeat_interleave(2, dim=1)
        S = 0.25 * (tq @ kk.transpose(-1, -2))
        if causal:
            S = S.masked_fill(torch.ones(40, 40, dtype=torch.bool).triu(1), float("-inf"))
        out = torch.softmax(S, dim=-1) @ vv
        lse = torch.logsumexp(S, dim=-1)
        out.backward(torch.tensor(do))
        O, L = orc.attention_fwd(q, k, v, causal, 0.25)
        dQ, dK, dV = orc.attention_bwd(q, k, v, do, causal, 0.25)
        assert np.max(np.abs(O - out.detach().numpy())) < 1e-13
        assert np.max(np.abs(L - lse.detach().numpy())) < 1e-13
        for mine, ref in ((dQ, tq.grad), (dK, tk.grad), (dV, tv.grad)):
            assert np.max(np.abs(mine - ref.numpy())) < 1e-12


PINS = [
    check_rows_sum_to_one, check_constant_v, check_causal_row0, check_naive_lse,
    check_closed_forms, check_shift_invariance, check_brute_force, check_finite_differences,
    check_gradient_invariants, check_gqa_is_head_expansion, check_row_subset, check_torch_autograd,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(oracle_attention)


# ----------------------------------------------------------------------------
# the pages' worked numbers

def test_footprint_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "footprint_worked_example.json")))
    p = g["primer"]
    per_head = oracle.materialised_bytes(p["N"], p["elt_bytes"])
    assert round(per_head / 1e6) == p["per_head_S_plus_P_MB_approx"]
    assert round(oracle.materialised_bytes(p["N"], p["elt_bytes"], p["heads"]) / 1e9, 1) == p["all_heads_GB_approx"]
    assert round(oracle.materialised_bytes(p["N_long"], p["elt_bytes"]) / 1e9) == p["per_head_long_GB_approx"]
    assert round(oracle.materialised_bytes(p["N_long"], p["elt_bytes"], p["heads"]) / 1e9, -1) == p["all_heads_long_GB_approx"]
    r = g["praveentn"]
    assert oracle.materialised_bytes(r["N"], r["elt_bytes"]) / 2 ** 20 == r["attention_matrix_MiB"]


def _csv(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return list(csv.DictReader(line for line in f if not line.startswith("#")))


def test_sm75_memory_table_is_s_plus_p():
    # naive - flash = S and P for batch*heads = 8 at fp16, to the table's 0.1 MB rounding
    for row in _csv("sm75_memory_footprint.csv"):
        N = int(row["seq_len"])
        diff = float(row["naive_MB"]) - float(row["flash_MB"])
        assert abs(oracle.materialised_bytes(N, 2, heads=8) / 1e6 - diff) <= 0.1


def test_sm75_throughput_flop_convention():
    # TFLOPS = 4*B*H*N^2*d / t (halved when causal) with B*H = 8 reproduces the printed column
    for row in _csv("sm75_throughput.csv"):
        d, causal, N = int(row["d"]), bool(int(row["causal"])), int(row["seq_len"])
        tflops = metrics.fwd_flops(1, 8, N, d, causal) / (float(row["flash_ms"]) * 1e-3) / 1e12
        assert abs(tflops - float(row["TFLOPS"])) <= 0.006, (row, tflops)


# ----------------------------------------------------------------------------
# planted mistakes: each mutant of the oracle's source must fail at least one pin

MUTANTS = {
    "page_literal_dS_without_D": ("dS = P * (dP - D)\n", "dS = P * dP\n"),
    "dQ_missing_scale": ("dQ[b, h, rr] = scale * (dS @ Kh)", "dQ[b, h, rr] = dS @ Kh"),
    "dK_overwrites_group": ("dK[b, kh] += scale * (dS.T @ Qr)", "dK[b, kh] = scale * (dS.T @ Qr)"),
    "causal_masks_diagonal": ("rows[:, None] < np.arange", "rows[:, None] <= np.arange"),
    "causal_mask_transposed": ("rows[:, None] < np.arange(K.shape[0])[None, :]",
                               "rows[:, None] > np.arange(K.shape[0])[None, :]"),
    "interleaved_gqa_mapping": ("kh = h // group\n            for r0 in range(0, R",
                                "kh = h % Hkv\n            for r0 in range(0, R"),
    "lse_in_log2": ("m + np.log(l)", "m + np.log2(l)"),
    "unnormalised_output": ("return E / l, m[:, 0], l[:, 0]", "return E, m[:, 0], l[:, 0]"),
    "scores_transposed": ("S = scale * (Qr @ K.T)", "S = scale * (Qr @ K.T).T[: Qr.shape[0], : K.shape[0]]"),
    "dV_uses_dP": ("dV[b, kh] += P.T @ dOr", "dV[b, kh] += P.T @ dOr * 1.0001"),
}


def _mutant(old, new):
    src = open(oracle_attention.__file__).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    mod = _mutant(*MUTANTS[name])
    failed = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {name}"
