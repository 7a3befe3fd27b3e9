"""GPU parity of the FP8 path (fa_fp8_quantize_rows, fa_fp8_quantize_v, fa_fwd_fp8)
against the fp64 oracle in oracle/fp8.py.

Quantisation is compared bit for bit: every code (a code of zero compares equal to
its negative) and every scale.  The value-tile layout is undone with the documented
key permutation before the comparison.

The forward pass is compared with the oracle's exact attention over the dequantised
operands.  Its tolerance is derived from the two approximations the kernel makes
(a derivation, not a fit):
  * P is rounded to e4m3 for the product with V.  With p_j = exp(S_j - max S) <= 1,
    l = sum_j p_j, pb_j = p_j / l and e_j = max(2^-4 p_j, 2^-10) for every visible key
    (half an e4m3 ulp: relative 2^-4 for normal values, absolute 2^-10 below 2^-6; the
    kernel's probabilities are p_j times 2^delta with delta >= 0, which only lowers
    both), this moves O_ic by at most sum_j e_j |V_jc| / l.
  * The FP8 matrix product does not sum its 64 products exactly: on MI355X its result
    is off by up to about 2^-12 of the sum of the magnitudes of the products and the
    accumulator input (measured over random e4m3 operands spanning the whole range;
    EPS = 2^-11 is used).  A score (two products for d = 128, one for d = 64, the first
    result being the second's accumulator input) is then off by at most
    delta_ij = 2 EPS A_ij with A_ij = scale sum_k |Q_ik K_jk|, which moves LSE_i by at
    most sum_j pb_j delta_ij and O_ic by at most sum_j pb_j delta_ij |V_jc - O_ic| (to
    first order); the value products, one per 64 keys accumulated into O, add at most
    EPS U_i (1 + 2^-4) sum_j pb_j |V_jc| over U_i units.
  * Per element: |O - O_ref| <= the sum of these + 2^-8 |O_ref| (bf16 output)
    + 1e-6 max|O_ref|.
  * In aggregate: rms(O - O_ref) <= sqrt(mean(sum_j e_j^2 V_jc^2 / l^2)) (independent
    roundings each bounded by e_j) + rms of the score and accumulation terms (the latter
    with sqrt(U_i) for U_i) + the rms of the bf16 rounding.
  * LSE: |LSE_i - LSE_ref_i| <= sum_j pb_j delta_ij + 2e-5 (fp32 exponentials and sums;
    the row sums use the unrounded fp32 P).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as ofp8
import workloads
from tests.gpu_util import say, to_dev
import exact_io_aware_fwd_amd as fa

pytestmark = pytest.mark.gpu

EPS = 2.0 ** -11     # accumulation error bound of the FP8 matrix product (see above and the test below)


def _perm():
    """Position p of a value tile -> key within the tile (p = 32h + 16t + 4a + b -> 32t + 8a + 4h + b)."""
    p = np.arange(64)
    h, t, a, b = p // 32, (p // 16) % 2, (p // 4) % 4, p % 4
    return 32 * t + 8 * a + 4 * h + b


def _same_codes(got: np.ndarray, want: np.ndarray) -> bool:
    got = np.where((got & 0x7F) == 0, 0, got)
    want = np.where((want & 0x7F) == 0, 0, want)
    return np.array_equal(got, want)


def _v_rows(codes_t: np.ndarray, N: int) -> np.ndarray:
    """Value tiles [B,H,nkb,d,64] -> row codes [B,H,N,d] (and check the padding is code 0)."""
    B, H, nkb, d, _ = codes_t.shape
    rows = np.zeros((B, H, nkb * 64, d), dtype=np.uint8)
    perm = _perm()
    for kt in range(nkb):
        rows[:, :, 64 * kt + perm, :] = np.transpose(codes_t[:, :, kt], (0, 1, 3, 2))
    assert np.all(rows[:, :, N:] == 0), "keys past N must be code 0"
    return rows[:, :, :N]


def _signs(seed, d):
    return workloads.random_signs(seed, d)


QUANT_CASES = [
    # (B, H, N, d, dtype, block_rows, with_signs)
    (1, 2, 256, 128, torch.bfloat16, 64, True),
    (2, 3, 1000, 128, torch.bfloat16, 128, True),
    (1, 2, 777, 64, torch.float16, 256, True),
    (1, 1, 1, 64, torch.bfloat16, 64, True),
    (1, 2, 300, 128, torch.float16, 64, False),
    (2, 1, 65, 64, torch.bfloat16, 128, False),
]


@pytest.mark.parametrize("case", QUANT_CASES, ids=lambda c: f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}{str(c[4])[6:]}_blk{c[5]}_{'rot' if c[6] else 'plain'}")
def test_quantize_rows_bit_exact(case):
    B, H, N, d, dt, blk, rot = case
    x = workloads.randn_outliers(9100 + N, (B, H, N, d), 1e-3, 16.0, dt)
    s = _signs(9200 + d, d) if rot else None
    say(f"[fp8 quant rows] {case}")
    codes, scales = fa.fp8_quantize(to_dev(x)[0], blk, None if s is None else torch.from_numpy(s).cuda())
    torch.cuda.synchronize()
    want_c, want_s = ofp8.quantize(x, blk, s)
    assert np.array_equal(scales.cpu().double().numpy(), want_s)
    assert _same_codes(codes.cpu().numpy(), want_c)


@pytest.mark.parametrize("case", [c for c in QUANT_CASES if not c[6]] + [(1, 2, 1000, 128, torch.bfloat16, 256, False),
                                                                        (1, 1, 64, 128, torch.bfloat16, 64, False)],
                         ids=lambda c: f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}_blk{c[5]}")
def test_quantize_v_bit_exact(case):
    B, H, N, d, dt, blk, _ = case
    x = workloads.randn_outliers(9300 + N, (B, H, N, d), 1e-3, 16.0, dt)
    say(f"[fp8 quant v] {case}")
    codes, scales = fa.fp8_quantize_v(to_dev(x)[0], blk)
    torch.cuda.synchronize()
    want_c, want_s = ofp8.quantize(x, blk, None)
    assert np.array_equal(scales.cpu().double().numpy(), want_s)
    assert _same_codes(_v_rows(codes.cpu().numpy(), N), want_c)


def _bounds(Qh, Kh, Vh, O_ref, causal, scale, rows):
    """Per-element worst-case bound and rms bound of the kernel's O error, and the
    per-row LSE bound, for query rows `rows` (see the module docstring)."""
    B, Hq, N, d = Qh.shape
    G = Hq // Kh.shape[1]
    R = len(rows)
    nchunk = d // 64
    worst = np.zeros((B, Hq, R, d))
    ms_p = np.zeros((B, Hq, R, d))        # squared P-rounding term (independent roundings)
    ms_acc = np.zeros((B, Hq, R, d))      # squared score/accumulation terms, random-walk form
    lse_b = np.zeros((B, Hq, R))
    units = (rows // 64 + 1) if causal else np.full(R, -(-N // 64))
    for b in range(B):
        for h in range(Hq):
            Q, K, V = Qh[b, h, rows], Kh[b, h // G], Vh[b, h // G]
            S = scale * Q @ K.T
            A = scale * np.abs(Q) @ np.abs(K).T
            if causal:
                vis = rows[:, None] >= np.arange(N)[None, :]
                S[~vis] = -np.inf
                A[~vis] = 0.0
            p = np.exp(S - S.max(axis=1, keepdims=True))
            l = p.sum(axis=1, keepdims=True)
            pb = p / l
            e = np.where(p > 0, np.maximum(2.0 ** -4 * p, 2.0 ** -10), 0.0)
            delta = nchunk * EPS * A
            t_round = (e @ np.abs(V)) / l
            t_score = np.zeros((R, d))
            w = pb * delta
            for r0 in range(0, R, 64):            # sum_j w_rj |V_jc - O_rc|, 64 rows at a time
                dev = np.abs(V[None, :, :] - O_ref[b, h, r0:r0 + 64][:, None, :])
                t_score[r0:r0 + 64] = np.einsum("rj,rjc->rc", w[r0:r0 + 64], dev)
            t_acc = EPS * (1 + 2.0 ** -4) * (pb @ np.abs(V))
            worst[b, h] = t_round + t_score + units[:, None] * t_acc
            ms_p[b, h] = ((e * e) @ (V * V)) / (l * l)
            ms_acc[b, h] = (t_score + np.sqrt(units)[:, None] * t_acc) ** 2
            lse_b[b, h] = (pb * delta).sum(axis=1)
    rms_bound = np.sqrt(np.mean(ms_p)) + np.sqrt(np.mean(ms_acc))
    return worst, rms_bound, lse_b


def _compare(o_c, l_c, q, k, v, s, causal, scale, bq, bkv, rows):
    """Check GPU O/LSE rows against the oracle for one problem (q, k, v CPU tensors)."""
    Qh, Kh, Vh = ofp8.quantized_operands(q, k, v, s, bq, bkv)
    O_ref, L_ref = oracle.attention_fwd(Qh, Kh, Vh, causal, scale, rows=rows)   # = ofp8.attention_fwd_fp8
    assert np.all(np.isfinite(o_c)) and np.all(np.isfinite(l_c))
    worst, rms_b, lse_b = _bounds(Qh, Kh, Vh, O_ref, causal, scale, rows)
    err = np.abs(o_c - O_ref)
    bound = worst + 2.0 ** -8 * np.abs(O_ref) + 1e-6 * np.max(np.abs(O_ref))
    assert np.all(err <= bound), f"O outside the rounding bound: worst excess {np.max(err - bound):.3e}"
    rms = float(np.sqrt(np.mean(err ** 2)))
    rms_bound = float(rms_b + 2.0 ** -8 * np.sqrt(np.mean(O_ref ** 2)) / np.sqrt(3))
    el = np.abs(l_c - L_ref)
    say(f"    rms {rms:.3e} (bound {rms_bound:.3e}), max err {np.max(err):.3e}, "
        f"lse {np.max(el):.2e} (bound {np.min(lse_b) + 2e-5:.2e} .. {np.max(lse_b) + 2e-5:.2e})")
    assert rms <= rms_bound, f"O rms error {rms:.3e} > {rms_bound:.3e}"
    assert np.all(el <= lse_b + 2e-5), f"LSE error {np.max(el - lse_b):.3e} above its bound"
    return rms, float(np.max(el))


def _run_gpu(q, k, v, s, causal, scale, bq, bkv):
    qd, kd, vd = to_dev(q, k, v)
    sd = None if s is None else torch.from_numpy(s).cuda()
    ops = fa.fp8_prepare(qd, kd, vd, sd, bq, bkv)
    o, lse = fa.fwd_fp8(*ops, causal=causal, softmax_scale=scale, block_q=bq, block_kv=bkv)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


def check_fp8_fwd(q, k, v, s, causal, scale, bq=64, bkv=64, label=""):
    B, Hq, N, d = q.shape
    say(f"[fp8 fwd] {label} q={tuple(q.shape)} k={tuple(k.shape)} causal={causal} blocks=({bq},{bkv})")
    o, lse = _run_gpu(q, k, v, s, causal, scale, bq, bkv)
    return _compare(o, lse, q, k, v, s, causal, scale, bq, bkv, np.arange(N))


@pytest.mark.parametrize("name", ["fp8_mha8_n1024_d128", "fp8_h4_n1000_d64"])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_fwd_workloads(name, causal):
    w = workloads.FP8_WORKLOADS[name]
    if causal not in w.causal:
        pytest.skip("not a setting of this workload")
    q, k, v, s = workloads.make_fp8_inputs(w)
    check_fp8_fwd(q, k, v, s, causal, w.scale, w.block_q, w.block_kv, label=name)


SHAPES = [
    # (B, Hq, Hkv, N, d, causal, bq, bkv, signs)
    (1, 1, 1, 1, 128, False, 64, 64, True),
    (1, 2, 1, 63, 64, True, 64, 64, True),
    (1, 2, 2, 65, 128, True, 128, 64, True),
    (2, 4, 1, 200, 128, False, 64, 128, True),
    (1, 2, 2, 513, 64, True, 256, 256, False),
    (1, 8, 2, 300, 128, True, 64, 64, False),
    (1, 1, 1, 2048, 128, True, 64, 64, True),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda c: "B{}Hq{}Hkv{}N{}d{}{}_q{}kv{}_{}".format(
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "", c[6], c[7], "rot" if c[8] else "plain"))
def test_fp8_fwd_shapes(shape):
    B, Hq, Hkv, N, d, causal, bq, bkv, rot = shape
    q = workloads.randn_outliers(9400 + N, (B, Hq, N, d), 1e-3, 16.0)
    k = workloads.randn_outliers(9401 + N, (B, Hkv, N, d), 1e-3, 16.0)
    v = workloads.randn_outliers(9402 + N, (B, Hkv, N, d), 1e-3, 16.0)
    s = _signs(9403, d) if rot else None
    check_fp8_fwd(q, k, v, s, causal, float(np.float32(1 / np.sqrt(d))), bq, bkv)


def test_fp8_fwd_headline_sampled_rows():
    """The grouped-query N=8192 shape at full size, in the launch configuration the
    benchmark times, on sampled heads and rows (first, last, block edges, random).
    Heads are independent problems (quantisation blocks never span heads), so the
    oracle runs on each sampled (batch, head) with its K/V head alone."""
    w = workloads.FP8_WORKLOADS[workloads.FP8_HEADLINE]
    q, k, v, s = workloads.make_fp8_inputs(w)
    say(f"[fp8 fwd] {w.name} full size, sampled heads and rows")
    o, lse = _run_gpu(q, k, v, s, True, w.scale, w.block_q, w.block_kv)
    g = np.random.Generator(np.random.PCG64(5))
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 255, 256, 4095, 8191], g.integers(0, w.N, 16)]))
    G = w.Hq // w.Hkv
    for b, h in ((0, 0), (1, 13), (1, 31)):
        sl = slice(h // G, h // G + 1)
        _compare(o[b:b + 1, h:h + 1, rows], lse[b:b + 1, h:h + 1, rows], q[b:b + 1, h:h + 1], k[b:b + 1, sl],
                 v[b:b + 1, sl], s, True, w.scale, w.block_q, w.block_kv, rows)


def test_fp8_fwd_deterministic():
    q = workloads.randn_outliers(9500, (1, 4, 700, 128), 1e-3, 16.0)
    k = workloads.randn_outliers(9501, (1, 2, 700, 128), 1e-3, 16.0)
    v = workloads.randn_outliers(9502, (1, 2, 700, 128), 1e-3, 16.0)
    s = torch.from_numpy(_signs(9503, 128)).cuda()
    say("[fp8 fwd] determinism")
    ops = fa.fp8_prepare(*to_dev(q, k, v), s)
    o1, l1 = fa.fwd_fp8(*ops, causal=True)
    o2, l2 = fa.fwd_fp8(*ops, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fp8_exact_inputs_match_exact_attention():
    """Operands that are e4m3 values times block powers of two go through quantisation
    unchanged, so the kernel differs from exact attention only by its P rounding."""
    g = np.random.Generator(np.random.PCG64(9600))
    vals = ofp8.e4m3_values()[:127]
    B, H, N, d = 1, 2, 256, 64
    out = []
    for _ in range(3):
        C = vals[g.integers(0, 127, (B, H, N, d))] * np.where(g.random((B, H, N, d)) < 0.5, -1.0, 1.0)
        C[..., ::64, 0] = 448.0
        C = C / 256.0
        out.append(torch.from_numpy(C).to(torch.bfloat16))   # 4-bit significands: exact in bf16
    q, k, v = out
    say("[fp8 fwd] exact operands")
    ops = fa.fp8_prepare(*to_dev(q, k, v), None)
    for t, want in ((ops[3], 2.0 ** -8), (ops[4], 2.0 ** -8), (ops[5], 2.0 ** -8)):
        assert torch.all(t == want)
    check_fp8_fwd(q, k, v, None, True, 0.125, label="exact operands")
    O, L = oracle.attention_fwd(q, k, v, True, 0.125)
    O2, L2 = ofp8.attention_fwd_fp8(q, k, v, None, True, 0.125)
    assert np.max(np.abs(O - O2)) < 1e-12 and np.max(np.abs(L - L2)) < 1e-12


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_score_product_error_within_half_eps(d):
    """The measurement behind EPS.  With one key and one query per head, the forward's LSE
    is the score itself, S = scale * q.k, formed by the scaled FP8 matrix product (one
    64-deep product at d = 64; at d = 128 two, the first result being the second's
    accumulator input), so |LSE - S_exact| is that product's accumulation error.  The
    operands are block-quantised values whose magnitudes span 2^-8 .. 2^8 (every e4m3
    binade, subnormals included) with random signs (sums with heavy cancellation), 4096
    heads per case.  Each product is held to EPS / 2 of the magnitudes it sums (its
    products and its accumulator input), the per-product error the derivation above
    doubles for its margin; fp32 rounding of LSE = ln 2 * (S log2 e) is allowed on top."""
    B, H = 64, 64
    g = np.random.Generator(np.random.PCG64(9800 + d))

    def draw():
        mag = np.exp2(g.uniform(-8.0, 8.0, (B, H, 1, d)))
        sign = np.where(g.random((B, H, 1, d)) < 0.5, -1.0, 1.0)
        return torch.from_numpy((mag * sign).astype(np.float32)).to(torch.bfloat16)

    q, k = draw(), draw()
    v = workloads.randn(9810 + d, (B, H, 1, d), torch.bfloat16)
    scale = float(np.float32(1 / np.sqrt(d)))
    say(f"[fp8 fwd] score product error, d={d}, {B * H} single-key heads")
    _, lse = _run_gpu(q, k, v, None, True, scale, 64, 64)
    Qh, Kh, _ = ofp8.quantized_operands(q, k, v, None, 64, 64)
    prod = scale * Qh[:, :, 0, :] * Kh[:, :, 0, :]                 # [B, H, d], exact in float64
    S = prod.sum(axis=-1)
    a1 = np.abs(prod[..., :64]).sum(axis=-1)
    a2 = np.abs(prod[..., 64:]).sum(axis=-1)
    # per product EPS/2 of (its products + its accumulator input, |first result| <= a1)
    bound = EPS / 2 * (a1 + a2 + (a1 if d == 128 else 0.0)) + 8 * 2.0 ** -24 * np.abs(S) + 1e-30
    err = np.abs(lse[:, :, 0] - S)
    rel = err / (a1 + a2)
    say(f"    max |LSE - S| / sum|products| = {rel.max():.3e} (2^{np.log2(max(rel.max(), 1e-30)):.2f}); "
        f"mean {rel.mean():.3e}; per-product bound EPS/2 = 2^{np.log2(EPS / 2):.0f}")
    assert np.all(np.isfinite(lse)), "non-finite LSE"
    assert np.all(err <= bound), f"accumulation error above EPS/2 per product: worst {np.max(err / bound):.3f}x"
