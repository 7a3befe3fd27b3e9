"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the fp64 oracle at the stated tolerances.

Tolerances (element by element over the compared tensor):
  O    : max |O - O_ref| / max |O_ref|   <= 2e-3 (fp16), 1.5e-2 (bf16)
  LSE  : max |LSE - LSE_ref|             <= 1e-4
  dQ, dK, dV : ||x - x_ref||_2 / ||x_ref||_2 <= 1e-2
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import exact_io_aware_fwd_amd as fa

O_TOL = {torch.float16: 2e-3, torch.bfloat16: 1.5e-2}
LSE_TOL = 1e-4
GRAD_TOL = 1e-2


def round_to(x: np.ndarray, dtype) -> np.ndarray:
    """Round fp64 values to `dtype` (RNE, through torch's CPU cast) and back to fp64."""
    return torch.from_numpy(np.ascontiguousarray(x)).float().to(dtype).double().numpy()


def lowprec_bwd_baseline(q, k, v, do, causal, scale):
    """Gradients with the backward's documented rounding points and otherwise exact arithmetic.

    O enters as the input dtype (it is the forward's output), and P and dS are rounded to
    the input dtype before the products that use them.  Its error against the oracle is
    the floor this precision design can reach; the Primer's proposed verification (section
    on Turing checks) bounds a kernel's error by about twice such a baseline's.
    """
    dt = q.dtype
    Q, K, V, dO = (t.double().numpy() for t in (q, k, v, do))
    B, Hq, N, d = Q.shape
    G = Hq // K.shape[1]
    O, L = oracle.attention_fwd(q, k, v, causal, scale)
    Ob = round_to(O, dt)
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    for b in range(B):
        for h in range(Hq):
            kh = h // G
            S = scale * Q[b, h] @ K[b, kh].T
            if causal:
                S[np.triu_indices(N, 1)] = -np.inf
            P = np.exp(S - L[b, h][:, None])
            dS = P * (dO[b, h] @ V[b, kh].T - (dO[b, h] * Ob[b, h]).sum(1)[:, None])
            dV[b, kh] += round_to(P, dt).T @ dO[b, h]
            dK[b, kh] += scale * round_to(dS, dt).T @ Q[b, h]
            dQ[b, h] = scale * round_to(dS, dt) @ K[b, kh]
    return dQ, dK, dV


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(*ts):
    return [t.to("cuda:0").contiguous() for t in ts]


def o_err(o, o_ref):
    o = o.double().cpu().numpy() if hasattr(o, "cpu") else o
    return float(np.max(np.abs(o - o_ref)) / max(np.max(np.abs(o_ref)), 1e-30))


def lse_err(l, l_ref):
    l = l.double().cpu().numpy() if hasattr(l, "cpu") else l
    return float(np.max(np.abs(l - l_ref)))


def rel_l2(x, x_ref):
    x = x.double().cpu().numpy() if hasattr(x, "cpu") else x
    return float(np.linalg.norm((x - x_ref).ravel()) / max(np.linalg.norm(x_ref.ravel()), 1e-30))


def check_fwd(q, k, v, causal, scale, rows=None, label=""):
    """Run fa.fwd on cuda:0 and compare with the oracle (all rows or the sampled `rows`)."""
    say(f"[fwd] {label} q={tuple(q.shape)} k={tuple(k.shape)} {q.dtype} causal={causal} rows={'all' if rows is None else len(rows)}")
    qd, kd, vd = to_dev(q, k, v)
    o, lse = fa.fwd(qd, kd, vd, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_fwd(q, k, v, causal, scale, rows=rows)
    o_c, l_c = o.cpu(), lse.cpu()
    if rows is not None:
        o_c, l_c = o_c[:, :, rows], l_c[:, :, rows]
    eo, el = o_err(o_c, O_ref), lse_err(l_c, L_ref)
    assert np.isfinite(eo) and np.isfinite(el)
    assert eo <= O_TOL[q.dtype], f"O error {eo:.3e} > {O_TOL[q.dtype]}"
    assert el <= LSE_TOL, f"LSE error {el:.3e} > {LSE_TOL}"
    return eo, el
