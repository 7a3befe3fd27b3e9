"""GPU parity of the forward's online softmax where the reference has to move.

`fwd_unit_kernel` forms P from the reference as it stands and rescales only when a lane's
probabilities over a 32-key unit sum past 2^8, or when the lane has no reference yet
(Primer, "FlashAttention-4": conditional rescaling; Wiki, "Online softmax").  Random
N(0, 1) inputs almost never take that slow path after the first unit.  These inputs do:

* rising scores: every key's score grows with its position, by about 8 (log2 units) per
  unit, so nearly every unit of every row moves the reference;
* a jump: one late key whose score is ~95 (d = 64) to ~190 (d = 128, log2 units) above the
  rest, so 2^(s c - m) comes out huge or, past 128, infinite before the rescale (the slow
  path must catch it and form P again);
* falling scores: the first unit holds each row's maximum and every later unit underflows
  towards zero under the stale reference.

Each case runs fa_fwd, and the key-split route of fa_fwd_splitkv (two and three splits,
each split starting from no reference), against the fp64 oracle at the usual tolerances:
O max error / max |O_ref| <= 2e-3 (fp16), 1.5e-2 (bf16); LSE max abs <= 1e-4.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import exact_io_aware_fwd_amd as fa
from tests.gpu_util import LSE_TOL, O_TOL, lse_err, o_err, say, to_dev

pytestmark = pytest.mark.gpu


def _signs(seed: int, d: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    return np.where(g.random(d) < 0.5, -1.0, 1.0)


def _case(kind: str, B: int, Hq: int, Hkv: int, N: int, d: int, dt, seed: int):
    """q, k, v (CPU, dtype dt): N(0, 1) plus a component along one +-1 direction w per head."""
    q = workloads.randn(seed, (B, Hq, N, d), torch.float32).double().numpy()
    k = workloads.randn(seed + 1, (B, Hkv, N, d), torch.float32).double().numpy()
    v = workloads.randn(seed + 2, (B, Hkv, N, d), dt)
    w = _signs(seed + 3, d)
    pos = np.arange(N, dtype=np.float64)
    # score of the aligned component: scale * a_q * a_k * d = a_q * a_k * sqrt(d)
    if kind == "rising":      # a_q a_k sqrt(d) grows by ~5.5 (x log2 e = ~8) per 32 keys
        a_q = 1.0
        a_k = pos * (5.5 / 32) / math.sqrt(d)
    elif kind == "jump":      # key 5N/6 scores ~65 (d = 64) to ~135 (d = 128) above the others
        a_q = 2.0
        a_k = np.zeros(N)
        a_k[(5 * N) // 6] = 6.0 if d == 128 else 4.0
    elif kind == "falling":   # the first keys highest, then ~8 (log2) lower per unit, floor 0
        a_q = 1.0
        a_k = np.maximum(0.0, 12 * 32 - pos) * (5.5 / 32) / math.sqrt(d)
    else:
        raise ValueError(kind)
    q = q * 0.5 + a_q * w
    k = k * 0.5 + a_k[None, None, :, None] * w
    to = lambda x: torch.from_numpy(x.astype(np.float32)).to(dt)
    return to(q), to(k), v


CASES = [
    (kind, B, Hq, Hkv, N, d, dt)
    for kind in ("rising", "jump", "falling")
    for (B, Hq, Hkv, N, d, dt) in ((1, 4, 2, 777, 128, torch.bfloat16), (2, 2, 1, 640, 64, torch.float16),
                                   (1, 8, 8, 1031, 128, torch.float16))
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-B{c[1]}Hq{c[2]}Hkv{c[3]}N{c[4]}d{c[5]}"
                                                      f"{'f16' if c[6] == torch.float16 else 'bf16'}")
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_reference_moves(case, causal):
    kind, B, Hq, Hkv, N, d, dt = case
    q, k, v = _case(kind, B, Hq, Hkv, N, d, dt, 9900 + N + d)
    scale = 1 / math.sqrt(d)
    say(f"[fwd softmax] {kind} B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} {dt} causal={causal}")
    O_ref, L_ref = oracle.attention_fwd(q, k, v, causal, scale)
    assert np.isfinite(L_ref).all()
    qd, kd, vd = to_dev(q, k, v)
    runs = {"fa_fwd": fa.fwd(qd, kd, vd, causal=causal, softmax_scale=scale)}
    for s in (2, 3):   # key splits, each starting from no reference (fp32 partials: a workspace)
        assert fa.splitkv_workspace_size(B, Hq, Hkv, N, N, d, dt, s) > 0
        runs[f"{s} key splits"] = fa.fwd_splitkv(qd, kd, vd, causal=causal, softmax_scale=scale, num_splits=s)
    torch.cuda.synchronize()
    for name, (o, lse) in runs.items():
        eo, el = o_err(o.cpu(), O_ref), lse_err(lse.cpu(), L_ref)
        say(f"    {name}: O {eo:.2e} LSE {el:.2e} (LSE range {L_ref.min():.1f} .. {L_ref.max():.1f})")
        assert eo <= O_TOL[dt] and el <= LSE_TOL, (name, eo, el)


def test_jump_past_the_exponent_range_hits_every_row():
    """The jump key's score minus the stale reference exceeds 128 (log2), the range of fp32's
    exponential, for every row that sees it: those rows must come out as that key's V and
    its score as the LSE, to fp32 accuracy of the softmax."""
    B, Hq, Hkv, N, d, dt = 1, 2, 1, 512, 128, torch.bfloat16
    q, k, v = _case("jump", B, Hq, Hkv, N, d, dt, 9950)
    scale = 1 / math.sqrt(d)
    jk = (5 * N) // 6
    S = scale * q.double()[0] @ k.double()[0, 0].T              # [Hq, N, N]
    others = torch.cat([S[..., :jk], S[..., jk + 1:]], dim=-1).amax(dim=-1)
    assert torch.all((S[..., jk] - others) * math.log2(math.e) > 128)
    qd, kd, vd = to_dev(q, k, v)
    o, lse = fa.fwd(qd, kd, vd, causal=True, softmax_scale=scale)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_fwd(q, k, v, True, scale)
    assert o_err(o.cpu(), O_ref) <= O_TOL[dt] and lse_err(lse.cpu(), L_ref) <= LSE_TOL
    # rows at and after the jump key: O is that key's V (bf16-rounded), LSE its score
    assert torch.equal(o[0, :, jk:].cpu(), v[0, 0, jk].expand(Hq, N - jk, d))


@pytest.mark.parametrize("N", [960, 1000], ids=["jump-in-odd-unit", "jump-in-even-unit"])
def test_small_grid_merge_with_a_jump(N):
    """On a small grid each 32 queries' keys are split between two waves by 32-key unit
    parity and the two partial results merged at the end; the jump key (5N/6) lands in an
    odd unit for N = 960 and an even one for N = 1000, so either wave holds the term that
    dominates and the other's part must vanish in the merge: O of the rows that see the
    jump is that key's V exactly, and all rows match the oracle."""
    B, Hq, Hkv, d, dt = 1, 2, 1, 128, torch.bfloat16
    jk = (5 * N) // 6
    assert (jk // 32) % 2 == (1 if N == 960 else 0)
    q, k, v = _case("jump", B, Hq, Hkv, N, d, dt, 9960 + N)
    scale = 1 / math.sqrt(d)
    S = scale * q.double()[0] @ k.double()[0, 0].T
    others = torch.cat([S[..., :jk], S[..., jk + 1:]], dim=-1).amax(dim=-1)
    assert torch.all((S[..., jk] - others) * math.log2(math.e) > 128)
    say(f"[fwd softmax] small-grid merge, jump key {jk} (unit {jk // 32}) N={N}")
    qd, kd, vd = to_dev(q, k, v)
    for causal in (True, False):
        o, lse = fa.fwd(qd, kd, vd, causal=causal, softmax_scale=scale)
        torch.cuda.synchronize()
        O_ref, L_ref = oracle.attention_fwd(q, k, v, causal, scale)
        assert o_err(o.cpu(), O_ref) <= O_TOL[dt] and lse_err(lse.cpu(), L_ref) <= LSE_TOL
        rows = slice(jk, None) if causal else slice(None)
        n = o[0, :, rows].shape[1]
        assert torch.equal(o[0, :, rows].cpu(), v[0, 0, jk].expand(Hq, n, d))
