"""Attention of a few new queries against a long key/value sequence, and the
log-sum-exp combine of partial results, in float64 — the oracle for split-KV
decoding (test infrastructure only).

Sources (page title, then the part of the page):

* "Flash Attention" (wiki), section "Training and autoregressive decoding": in
  one-token decoding the query length can be one while the cached key/value
  sequence is long.
* Same page, section "Flash-Decoding": the key/value sequence is split into chunks,
  attention is computed per chunk, and the partial outputs are combined using
  their log-sum-exp statistics (per-split attention, per-split statistics, a small
  reduction).
* "FlashAttention Primer: IO-Aware Attention, from FA1 to FA4", section "Why
  attention is quadratic" for S, P, O; the natural-log LSE as in
  :mod:`oracle.attention`.

Readings taken where the pages are silent:

* Alignment of a query block shorter than the key sequence: the Nq queries are the
  last Nq positions, so query i sits at position Nk - Nq + i and, under a causal
  mask, sees keys j <= Nk - Nq + i (for Nq == Nk this is the square causal mask).
* A part in which a query sees no key contributes nothing: its output is 0 and its
  statistic -inf, and the combine gives it weight 0.

The combine is the exact identity behind the method: with partial results
(O_s, L_s) over disjoint key sets, O = sum_s exp(L_s - M) O_s / sum_s exp(L_s - M)
and L = M + ln sum_s exp(L_s - M) for M = max_s L_s.

Pins: tests/test_oracle_decode_pins.py.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def attention_fwd_kv(q, k, v, causal: bool, scale: float, key_range=None):
    """(O, LSE) of queries q [B, Hq, Nq, d] against keys/values [B, Hkv, Nk, d].

    key_range = (lo, hi) restricts the keys to lo <= j < hi (a split); rows that
    see no key there get O = 0 and LSE = -inf.  LSE is in natural-log units.
    """
    Q, K, V = _f64(q), _f64(k), _f64(v)
    B, Hq, Nq, d = Q.shape
    _, Hkv, Nk, _ = K.shape
    if K.shape != V.shape or K.shape[0] != B or K.shape[3] != d or Hq % Hkv != 0:
        raise ValueError("shapes must be q [B,Hq,Nq,d], k = v [B,Hkv,Nk,d], Hq % Hkv == 0")
    if causal and Nq > Nk:
        raise ValueError("causal needs Nq <= Nk")
    lo, hi = (0, Nk) if key_range is None else (int(key_range[0]), int(key_range[1]))
    lo, hi = max(lo, 0), min(hi, Nk)
    group = Hq // Hkv
    pos = Nk - Nq + np.arange(Nq)                  # absolute position of each query
    keys = np.arange(lo, hi)
    O = np.zeros((B, Hq, Nq, d))
    LSE = np.full((B, Hq, Nq), -np.inf)
    if hi <= lo:
        return O, LSE
    for b in range(B):
        for h in range(Hq):
            kh = h // group
            S = float(scale) * (Q[b, h] @ K[b, kh, lo:hi].T)
            if causal:
                S[pos[:, None] < keys[None, :]] = -np.inf
            seen = np.isfinite(S).any(axis=1)
            m = np.where(seen, S.max(axis=1), 0.0)
            E = np.exp(S - m[:, None])
            l = E.sum(axis=1)
            ok = seen & (l > 0)
            O[b, h, ok] = (E[ok] / l[ok, None]) @ V[b, kh, lo:hi]
            LSE[b, h, ok] = m[ok] + np.log(l[ok])
    return O, LSE


def lse_combine(o_parts, lse_parts):
    """Merge partial results over disjoint key sets: o_parts [..., S, d], lse_parts [..., S].

    Returns (O [..., d], LSE [...]).  Rows whose parts are all -inf get O = 0, LSE = -inf.
    """
    Op, Lp = _f64(o_parts), _f64(lse_parts)
    if Op.shape[:-1] != Lp.shape:
        raise ValueError("o_parts must be lse_parts' shape plus a trailing d")
    M = Lp.max(axis=-1)
    any_part = np.isfinite(M)
    Msafe = np.where(any_part, M, 0.0)
    w = np.exp(Lp - Msafe[..., None])                 # exp(-inf) = 0 for empty parts
    den = w.sum(axis=-1)
    num = (w[..., None] * Op).sum(axis=-2)
    O = np.where(any_part[..., None], num / np.where(any_part, den, 1.0)[..., None], 0.0)
    LSE = np.where(any_part, Msafe + np.log(np.where(any_part, den, 1.0)), -np.inf)
    return O, LSE
