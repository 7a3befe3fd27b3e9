"""Exact attention under the mask family — variable-length (packed) batches, queries
shorter or longer than keys, sliding windows and block-sparse tile lists — in float64:
the oracle (test infrastructure only).

Sources (page title, then the part of the page):

* "FlashAttention Primer: IO-Aware Attention, from FA1 to FA4", section "FlashAttention-2:
  better work partitioning": the release line added variable-length (unpadded) entry
  points and sliding-window attention; section "FlashAttention-1: tiling plus online
  softmax": block-sparse attention computes exactly on the kept blocks; section
  "Hardware, dtype, determinism, and padding caveats": variable-length sequences are
  handled without padding through cumulative sequence lengths (cu_seqlens).
* "Flash Attention" (wiki), section "Block-sparse FlashAttention": masked score blocks are
  skipped, so work and IO scale with the kept blocks, and the result is exact for the
  mask it defines; section "Specialized kernels have boundaries": query and key lengths
  can differ, so causal-window conventions must be stated; section "Numerical
  validation": masks, variable-length batches and fully masked rows deserve tests.
* Softmax attention itself: "FlashAttention Primer", section "Why attention is quadratic";
  masked scores are minus infinity before the exponentials ("Flash Attention" (wiki),
  section "Online softmax").

Readings taken where the pages are silent (listed with the others in the design notes):

* Packed layout: with cumulative lengths cu_q, cu_k (B+1 entries each), sequence b owns
  query rows cu_q[b] .. cu_q[b+1]-1 and key rows cu_k[b] .. cu_k[b+1]-1; tensors are
  head-major [H, total, d] (LSE [H, total]).  Without them every sequence has Nq queries
  and Nk keys in [B, H, N, d] tensors.
* Alignment: within a sequence of Lq queries and Lk keys, query i sits at key position
  p_i = i + Lk - Lq (the queries are the last Lq positions; Lq = Lk is the square case).
* Window (left, right): key j is visible to query i iff left < 0 or j >= p_i - left, and
  right < 0 or j <= p_i + right.  (-1, -1) is full attention, (-1, 0) causal.
* Block-sparse list: the queries of a sequence are cut into blocks of 256 and the keys
  into tiles of 64; for each (sequence, head or all heads, query block) the caller lists
  the key tiles to visit; a score outside the listed tiles is masked.
* A query that sees no key gets O = 0 and LSE = -inf.
* Gradients ("FlashAttention Primer", section "Backward pass: recomputation instead of
  storage", with the full softmax Jacobian as in :mod:`oracle.attention`; the same mask,
  block lists included, as the forward): for every visible pair, P = exp(S - LSE), dV += P^T dO, dP = dO V^T, D_i = sum_k dO_ik O_ik,
  dS = P * (dP - D), dQ = scale dS K, dK += scale dS^T Q; masked pairs and rows without
  keys contribute nothing; dK and dV of a K/V head sum over its query heads.

Pins: tests/test_oracle_masks_pins.py.
"""
from __future__ import annotations

import numpy as np

from .attention import to_f64

QBLOCK = 256      # queries per block of a block-sparse list
KTILE = 64        # keys per tile of a block-sparse list


def visible(Lq: int, Lk: int, window=(-1, -1), kept_tiles=None, rows=None) -> np.ndarray:
    """[Lq, Lk] bool (or [len(rows), Lk]): key j visible to query i (alignment, window,
    listed tiles)."""
    left, right = window
    i = (np.arange(Lq) if rows is None else np.asarray(rows))[:, None]
    j = np.arange(Lk)[None, :]
    p = i + (Lk - Lq)
    vis = np.ones((i.shape[0], Lk), dtype=bool)
    if left >= 0:
        vis &= j >= p - left
    if right >= 0:
        vis &= j <= p + right
    if kept_tiles is not None:             # kept_tiles[qb] = collection of key-tile indices
        tile_ok = np.zeros((-(-Lq // QBLOCK), -(-Lk // KTILE)), dtype=bool)
        for qb, tiles in enumerate(kept_tiles):
            for t in tiles:
                if 0 <= t < tile_ok.shape[1]:
                    tile_ok[qb, t] = True
        vis &= tile_ok[i // QBLOCK, (np.arange(Lk) // KTILE)[None, :]]
    return vis


def _head_lists(block_lists, b: int, h: int):
    """Key-tile lists (one per query block) of query head h of sequence b, or None."""
    if block_lists is None:
        return None
    hm = block_lists[b]
    return hm[0] if len(hm) == 1 else hm[h]


def _attend(Q, K, V, vis, scale):
    """Rows of softmax(scale Q K^T masked by vis) V and their LSE; empty rows -> 0, -inf."""
    Lq, d = Q.shape
    O = np.zeros((Lq, V.shape[1]))
    L = np.full(Lq, -np.inf)
    if K.shape[0] == 0:
        return O, L
    S = scale * (Q @ K.T)
    S = np.where(vis, S, -np.inf)
    ok = vis.any(axis=1)
    if ok.any():
        m = S[ok].max(axis=1, keepdims=True)
        E = np.exp(S[ok] - m)
        l = E.sum(axis=1)
        O[ok] = (E @ V) / l[:, None]
        L[ok] = m[:, 0] + np.log(l)
    return O, L


def attention_fwd_masked(q, k, v, scale: float, cu_seqlens_q=None, cu_seqlens_k=None, window=(-1, -1),
                         block_lists=None, rows=None):
    """(O, LSE) in float64 under the mask family.

    Fixed lengths: q [B, Hq, Nq, d], k/v [B, Hkv, Nk, d] -> O [B, Hq, Nq, d], LSE [B, Hq, Nq].
    Packed: cu_seqlens_q/k given; q [Hq, total_q, d], k/v [Hkv, total_k, d] ->
    O [Hq, total_q, d], LSE [Hq, total_q].
    block_lists: None, or a nested list [B][Hm][query block] -> key-tile indices with
    Hm = 1 (shared by all heads) or Hq.
    rows (fixed lengths only): optional query indices to evaluate; O and LSE then hold
    only those rows.
    """
    Q, K, V = to_f64(q), to_f64(k), to_f64(v)
    scale = float(scale)
    packed = cu_seqlens_q is not None
    if packed != (cu_seqlens_k is not None):
        raise ValueError("give both cumulative length arrays or neither")
    if packed:
        cq = np.asarray(cu_seqlens_q, dtype=np.int64)
        ck = np.asarray(cu_seqlens_k, dtype=np.int64)
        B = len(cq) - 1
        Hq, Hkv = Q.shape[0], K.shape[0]
        if rows is not None:
            raise ValueError("rows applies to fixed lengths only")
    else:
        B, Hq, Nq, _ = Q.shape
        Hkv, Nk = K.shape[1], K.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    O = np.zeros(Q.shape if rows is None else (B, Hq, len(rows), Q.shape[-1]))
    L = np.full(O.shape[:-1], -np.inf)
    for b in range(B):
        for h in range(Hq):
            kl = _head_lists(block_lists, b, h)
            if packed:
                qs, qe, ks, ke = cq[b], cq[b + 1], ck[b], ck[b + 1]
                vis = visible(qe - qs, ke - ks, window, kl)
                O[h, qs:qe], L[h, qs:qe] = _attend(Q[h, qs:qe], K[h // G, ks:ke], V[h // G, ks:ke], vis, scale)
            else:
                r = np.arange(Nq) if rows is None else np.asarray(rows)
                vis = visible(Nq, Nk, window, kl, r)
                O[b, h], L[b, h] = _attend(Q[b, h, r], K[b, h // G], V[b, h // G], vis, scale)
    return O, L


def visible_pairs(Lqs, Lks, window=(-1, -1), block_lists_one_head=None) -> int:
    """Number of visible (query, key) pairs of one head over sequences of the given lengths."""
    n = 0
    for b, (lq, lk) in enumerate(zip(Lqs, Lks)):
        kl = None if block_lists_one_head is None else block_lists_one_head[b]
        n += int(visible(int(lq), int(lk), window, kl).sum())
    return n


def attention_bwd_masked(q, k, v, do, scale: float, cu_seqlens_q=None, cu_seqlens_k=None, window=(-1, -1),
                         block_lists=None):
    """(dQ, dK, dV) in float64 of L(O) for O = attention_fwd_masked(q, k, v, ...) with the
    same lengths, window and block lists, and dO = dL/dO.  Layouts as in
    attention_fwd_masked."""
    Q, K, V, dO = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    scale = float(scale)
    O, LSE = attention_fwd_masked(Q, K, V, scale, cu_seqlens_q, cu_seqlens_k, window, block_lists)
    packed = cu_seqlens_q is not None
    if packed:
        cq = np.asarray(cu_seqlens_q, dtype=np.int64)
        ck = np.asarray(cu_seqlens_k, dtype=np.int64)
        B, Hq, Hkv = len(cq) - 1, Q.shape[0], K.shape[0]
    else:
        B, Hq, Nq, _ = Q.shape
        Hkv, Nk = K.shape[1], K.shape[2]
    G = Hq // Hkv
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    for b in range(B):
        for h in range(Hq):
            kl = _head_lists(block_lists, b, h)
            if packed:
                sq, sk = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
                Qb, Kb, Vb, dOb, Ob, Lb = Q[h, sq], K[h // G, sk], V[h // G, sk], dO[h, sq], O[h, sq], LSE[h, sq]
            else:
                Qb, Kb, Vb, dOb, Ob, Lb = Q[b, h], K[b, h // G], V[b, h // G], dO[b, h], O[b, h], LSE[b, h]
            vis = visible(Qb.shape[0], Kb.shape[0], window, kl)
            ok = np.isfinite(Lb)
            S = scale * (Qb @ Kb.T)
            P = np.where(vis & ok[:, None], np.exp(S - np.where(ok, Lb, 0.0)[:, None]), 0.0)
            dVb = P.T @ dOb
            dP = dOb @ Vb.T
            Dr = (dOb * Ob).sum(axis=1)
            dS = P * (dP - Dr[:, None])
            dQb = scale * (dS @ Kb)
            dKb = scale * (dS.T @ Qb)
            if packed:
                dQ[h, sq] = dQb
                dK[h // G, sk] += dKb
                dV[h // G, sk] += dVb
            else:
                dQ[b, h] = dQb
                dK[b, h // G] += dKb
                dV[b, h // G] += dVb
    return dQ, dK, dV
