"""Materialising softmax attention in float64 — the oracle (test infrastructure only).

Every function here is the textbook definition, evaluated row chunk by row chunk
so that memory stays bounded; nothing is tiled over keys, fused or reordered
beyond that.  Sources (page title, then the part of the page):

* "FlashAttention Primer: IO-Aware Attention, from FA1 to FA4", section "Why
  attention is quadratic": S = Q K^T / sqrt(d), P = row-softmax(S), O = P V.
  The scale is an argument here; callers pass 1/sqrt(d) as the float32 value the
  kernel receives, so both sides use the same number.
* "Flash Attention" (wiki), section "Online softmax": masks are applied before the
  exponentials; a causal mask sets future-position scores to minus infinity.
  Reading taken: key j is visible to query i iff j <= i (equal query and key
  lengths; non-square causal is outside this path).
* "FlashAttention Primer", section "Backward pass: recomputation instead of
  storage": the forward saves O and one per-row log-sum-exp.  Reading taken: the
  statistic is LSE_i = ln sum_j exp(S_ij) of the scaled, masked scores, natural log.
* Same section, backward formulas.  The page's dS omits the softmax-Jacobian term
  and the 1/sqrt(d) factor; the true gradient of L(O) for S = scale * Q K^T is
      dV = P^T dO,  dP = dO V^T,  D_i = sum_k dO_ik O_ik,  dS = P * (dP - D),
      dQ = scale * dS K,  dK = scale * dS^T Q,
  which is what this oracle computes (the finite-difference pin in the tests fails
  the page's literal formula).
* Grouped/multi-query attention ("Flash Attention" wiki, section
  "FlashAttention-2"): several query heads share one K/V head.  Reading taken:
  contiguous groups, K/V head = hq // (Hq // Hkv); dK and dV of a K/V head sum
  over its query heads.

Pins (tests/test_oracle_pins.py): rows of P sum to 1, constant V, causal row 0,
the naive log-sum-exp, closed forms at N=1 and N=2, shift invariance, an
independent scalar brute force on tiny inputs, central finite differences of the
gradients, gradient invariants, and the worked footprint examples.
"""
from __future__ import annotations

import numpy as np

_CHUNK = 512


def to_f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or a CPU torch tensor (fp16/bf16/fp32/fp64) to float64."""
    if hasattr(x, "detach"):          # torch tensor; bf16 has no numpy dtype, so go through torch
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError("k, v must be [B, Hkv, N, d] matching q")
    Hkv = k.shape[1]
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, N, d


def _scores(Qr: np.ndarray, K: np.ndarray, rows: np.ndarray, causal: bool, scale: float) -> np.ndarray:
    """S rows = scale * Q_rows K^T with future keys set to -inf when causal."""
    S = scale * (Qr @ K.T)
    if causal:
        S[rows[:, None] < np.arange(K.shape[0])[None, :]] = -np.inf
    return S


def _softmax_rows(S: np.ndarray):
    """Row softmax with the max subtracted first; returns (P, row max, row sum of exp)."""
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    return E / l, m[:, 0], l[:, 0]


def attention_probs(q_head, k_head, causal: bool, scale: float) -> np.ndarray:
    """P = row-softmax(scale * q k^T) for one head, [N, N] float64 (small N only)."""
    Q = to_f64(q_head)
    K = to_f64(k_head)
    S = _scores(Q, K, np.arange(Q.shape[0]), causal, float(scale))
    return _softmax_rows(S)[0]


def attention_fwd(q, k, v, causal: bool, scale: float, rows=None):
    """O = softmax(scale * Q K^T [masked]) V and LSE, float64.

    q: [B, Hq, N, d]; k, v: [B, Hkv, N, d] (any float dtype; upcast exactly).
    rows: optional 1-D integer array of query positions; then O is
    [B, Hq, len(rows), d] and LSE is [B, Hq, len(rows)].
    Returns (O, LSE) with LSE in natural-log units.
    """
    Q, K, V = to_f64(q), to_f64(k), to_f64(v)
    B, Hq, Hkv, N, d = _check_shapes(Q, K, V)
    scale = float(scale)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    group = Hq // Hkv
    O = np.zeros((B, Hq, R, d))
    LSE = np.zeros((B, Hq, R))
    for b in range(B):
        for h in range(Hq):
            kh = h // group
            for r0 in range(0, R, _CHUNK):
                rr = rows[r0:r0 + _CHUNK]
                S = _scores(Q[b, h, rr], K[b, kh], rr, causal, scale)
                P, m, l = _softmax_rows(S)
                O[b, h, r0:r0 + len(rr)] = P @ V[b, kh]
                LSE[b, h, r0:r0 + len(rr)] = m + np.log(l)
    return O, LSE


def attention_bwd(q, k, v, do, causal: bool, scale: float):
    """(dQ, dK, dV) of L = sum(dO * O) for O = attention_fwd(q, k, v), float64.

    dK and dV are [B, Hkv, N, d] and sum over the query heads sharing a K/V head.
    O and P are recomputed here in float64 (the oracle keeps nothing from a GPU run).
    """
    Q, K, V, dO = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    B, Hq, Hkv, N, d = _check_shapes(Q, K, V)
    if dO.shape != Q.shape:
        raise ValueError("do must have the shape of q")
    scale = float(scale)
    group = Hq // Hkv
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    allrows = np.arange(N)
    for b in range(B):
        for h in range(Hq):
            kh = h // group
            Kh, Vh = K[b, kh], V[b, kh]
            for r0 in range(0, N, _CHUNK):
                rr = allrows[r0:r0 + _CHUNK]
                Qr, dOr = Q[b, h, rr], dO[b, h, rr]
                P = _softmax_rows(_scores(Qr, Kh, rr, causal, scale))[0]
                Or = P @ Vh
                dV[b, kh] += P.T @ dOr
                dP = dOr @ Vh.T
                D = (dOr * Or).sum(axis=1, keepdims=True)
                dS = P * (dP - D)
                dQ[b, h, rr] = scale * (dS @ Kh)
                dK[b, kh] += scale * (dS.T @ Qr)
    return dQ, dK, dV


def materialised_bytes(N: int, elt_bytes: int, heads: int = 1) -> int:
    """HBM bytes a materialising schedule holds for S and P: 2 * N^2 * elt_bytes per head.

    "FlashAttention Primer", section "Why attention is quadratic", worked example:
    both N x N matrices are stored at the input precision.
    """
    return 2 * N * N * elt_bytes * heads
