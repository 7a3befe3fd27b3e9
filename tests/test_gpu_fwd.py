"""GPU parity of the forward pass (fa_fwd through the C ABI) against the fp64 oracle."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import exact_io_aware_fwd_amd as fa
from tests.gpu_util import O_TOL, LSE_TOL, check_fwd, lse_err, o_err, say, to_dev

pytestmark = pytest.mark.gpu

DTYPES = [torch.float16, torch.bfloat16]


# ---- tiny and ragged sequence lengths: whole output vs the oracle -------------------------
@pytest.mark.parametrize("dtype", DTYPES, ids=["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 2, 3, 7, 16, 17, 63, 64, 65, 127, 129, 255, 257, 300])
def test_small_and_ragged(N, d, dtype):
    q, k, v = workloads.random_case(10 * N + d, 1, 4, 2, N, d, dtype)
    for causal in (False, True):
        check_fwd(q, k, v, causal, 1 / math.sqrt(d), label=f"N={N} d={d}")


@pytest.mark.parametrize("case", [
    # (B, Hq, Hkv, N, d, dtype): tails past several tiles, MQA, GQA, batch > 1
    (2, 3, 3, 1000, 64, torch.float16),
    (1, 8, 1, 1000, 128, torch.bfloat16),
    (3, 6, 2, 777, 128, torch.float16),
    (1, 2, 2, 2049, 128, torch.bfloat16),
    (2, 16, 8, 512, 64, torch.bfloat16),
], ids=lambda c: f"B{c[0]}Hq{c[1]}Hkv{c[2]}N{c[3]}d{c[4]}")
def test_multi_tile_tails(case):
    B, Hq, Hkv, N, d, dt = case
    q, k, v = workloads.random_case(7 + N, B, Hq, Hkv, N, d, dt)
    for causal in (False, True):
        check_fwd(q, k, v, causal, 1 / math.sqrt(d), label="tail")


# ---- the named workloads ----------------------------------------------------------------
def _sample_rows(N, seed):
    g = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 63, 64, 255, 256, 511, N // 2, N - 2, N - 1]
    rnd = g.choice(N, size=12, replace=False).tolist()
    return np.array(sorted(set(r for r in fixed + rnd if 0 <= r < N)))


@pytest.mark.parametrize("name", ["single_head_n256_d64_fp16", "mha8_n1024_d64_fp16"])
def test_workload_full(name):
    w = workloads.WORKLOADS[name]
    q, k, v = workloads.make_inputs(w)
    for causal in w.causal:
        check_fwd(q, k, v, causal, w.scale, label=name)


@pytest.mark.parametrize("name", ["b4_h32_n4096_d128_bf16_causal_qx8", "gqa_b2_hq32_hkv8_n8192_d128_bf16_causal",
                                  "fwd_bwd_h16_n4096_d128_bf16_causal"])
def test_workload_sampled_rows(name):
    """Full-size launch; the oracle computes a sample of rows in every head."""
    w = workloads.WORKLOADS[name]
    q, k, v = workloads.make_inputs(w)[:3]
    for causal in w.causal:
        check_fwd(q, k, v, causal, w.scale, rows=_sample_rows(w.N, 99), label=name)


# ---- invariants -------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", DTYPES, ids=["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_constant_v_gives_v(d, dtype):
    q, k, _ = workloads.random_case(5, 2, 4, 2, 333, d, dtype)
    c = workloads.randn(77, (d,), dtype)
    v = c.expand(2, 2, 333, d).contiguous()
    for causal in (False, True):
        qd, kd, vd = to_dev(q, k, v)
        o, _ = fa.fwd(qd, kd, vd, causal=causal)
        # each row is a convex combination of identical rows.  P is rounded to the input dtype
        # before P V while l sums the fp32 P, so besides the output rounding the weights may
        # sum to 1 within the dtype's rounding: allow two units of roundoff of max|c|
        err = (o.float().cpu() - c.float()).abs().max().item()
        assert err <= c.float().abs().max().item() * (2 ** -7 if dtype == torch.bfloat16 else 2 ** -10)


@pytest.mark.parametrize("d", [64, 128])
def test_causal_row0(d):
    q, k, v = workloads.random_case(6, 1, 4, 4, 200, d, torch.bfloat16)
    qd, kd, vd = to_dev(q, k, v)
    scale = 1 / math.sqrt(d)
    o, lse = fa.fwd(qd, kd, vd, causal=True, softmax_scale=scale)
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])
    ref = float(np.float32(scale)) * (q[:, :, 0].double() * k[:, :, 0].double()).sum(-1)
    assert (lse[:, :, 0].cpu().double() - ref).abs().max().item() <= LSE_TOL


def test_gqa_head_mapping():
    """K/V heads hold distinct constants in V: every query head's output names its K/V head."""
    B, Hq, Hkv, N, d = 2, 12, 3, 130, 64
    q, k, _ = workloads.random_case(8, B, Hq, Hkv, N, d, torch.float16)
    v = torch.arange(B * Hkv, dtype=torch.float16).view(B, Hkv, 1, 1).expand(B, Hkv, N, d).contiguous()
    qd, kd, vd = to_dev(q, k, v)
    o, _ = fa.fwd(qd, kd, vd, causal=False)
    o = o.float().cpu()
    for b in range(B):
        for h in range(Hq):
            assert torch.all(o[b, h] == float(b * Hkv + h // (Hq // Hkv))), (b, h)


def small_grid_split(B, Hq, N, d, causal):
    """The launch rule of fa_fwd at d = 128: grids of at most 256 blocks of 128 rows (512
    when causal) run the key-split workgroups (8 waves, two per 32 queries)."""
    return d == 128 and B * Hq * -(-N // 128) <= (512 if causal else 256)


@pytest.mark.parametrize("causal,hq", [(False, 85), (True, 170)])
def test_small_grid_key_split_threshold(causal, hq):
    """One more query head takes the grid past the small-grid line: the smaller call runs
    the key-split workgroups (each 32 queries' two waves take alternate 32-key units and
    merge their partial results, "FlashAttention Primer", "FlashAttention-1"), the larger
    one wave per 32 queries.  The two sum in different orders, so the heads they share
    agree to rounding, not bit for bit; the oracle checks the first and last head of each."""
    N, d = 300, 128
    assert small_grid_split(1, hq, N, d, causal) and not small_grid_split(1, hq + 1, N, d, causal)
    q, k, v = workloads.random_case(31 + hq, 1, hq + 1, 1, N, d, torch.bfloat16)
    scale = 1 / math.sqrt(d)
    say(f"[fwd] small-grid key split: Hq={hq} vs {hq + 1} (MQA) N={N} causal={causal}")
    qd, kd, vd = to_dev(q, k, v)
    o_small, l_small = fa.fwd(qd[:, :hq].contiguous(), kd, vd, causal=causal, softmax_scale=scale)
    o_big, l_big = fa.fwd(qd, kd, vd, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    for o, l, heads in ((o_small, l_small, (0, hq - 1)), (o_big, l_big, (0, hq))):
        for h in heads:
            O_ref, L_ref = oracle.attention_fwd(q[:, h:h + 1], k, v, causal, scale)
            eo, el = o_err(o[:, h:h + 1].cpu(), O_ref), lse_err(l[:, h:h + 1].cpu(), L_ref)
            say(f"    Hq={o.shape[1]} head {h}: O {eo:.2e} LSE {el:.2e}")
            assert eo <= O_TOL[torch.bfloat16] and el <= LSE_TOL
    ref = o_big[:, :hq].float()
    assert (o_small.float() - ref).abs().max().item() <= O_TOL[torch.bfloat16] * ref.abs().max().item()
    assert (l_small - l_big[:, :hq]).abs().max().item() <= LSE_TOL


@pytest.mark.parametrize("causal,hq", [(False, 64), (True, 128)])
def test_key_split_grid_does_not_change_bits(causal, hq):
    """Inside the small-grid region every row takes the same steps whatever the grid, so
    one more query head leaves the heads both calls share bit for bit the same."""
    N, d = 300, 128
    assert small_grid_split(1, hq, N, d, causal) and small_grid_split(1, hq + 1, N, d, causal)
    q, k, v = workloads.random_case(41 + hq, 1, hq + 1, 1, N, d, torch.float16)
    scale = 1 / math.sqrt(d)
    say(f"[fwd] key-split grid: Hq={hq} vs {hq + 1} (MQA) N={N} causal={causal}")
    qd, kd, vd = to_dev(q, k, v)
    o_small, l_small = fa.fwd(qd[:, :hq].contiguous(), kd, vd, causal=causal, softmax_scale=scale)
    o_big, l_big = fa.fwd(qd, kd, vd, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o_small, o_big[:, :hq]) and torch.equal(l_small, l_big[:, :hq])
    O_ref, L_ref = oracle.attention_fwd(q[:, hq:hq + 1], k, v, causal, scale)
    assert o_err(o_big[:, hq:hq + 1].cpu(), O_ref) <= O_TOL[torch.float16]
    assert lse_err(l_big[:, hq:hq + 1].cpu(), L_ref) <= LSE_TOL


def small_grid_waves_d64(B, Hq, N, causal):
    """The launch rule of fa_fwd at d = 64: 4 waves on 64 rows while the 64-row grid has at
    most 512 blocks, 6 on 96 rows for causal grids of up to 1024, else none (8-wave grid)."""
    nb = B * Hq * -(-N // 64)
    return 4 if nb <= 512 else 6 if causal and nb <= 1024 else 0


@pytest.mark.parametrize("case", [
    # (B, Hq, Hkv, N, dtype, causal, waves per workgroup the rule picks)
    (1, 12, 4, 3000, torch.float16, True, 6),
    (2, 4, 1, 2049, torch.bfloat16, True, 4),
    (1, 16, 16, 1111, torch.bfloat16, False, 4),
    (1, 3, 3, 4100, torch.float16, False, 4),
], ids=lambda c: f"B{c[0]}Hq{c[1]}Hkv{c[2]}N{c[3]}{'f16' if c[4] == torch.float16 else 'bf16'}"
                 f"{'causal' if c[5] else 'full'}-{c[6]}w")
def test_small_grid_key_split_d64(case):
    """d = 64 small grids run the same two-waves-per-32-queries workgroups (64 or 96 rows):
    whole tensors against the oracle, ragged tails, GQA/MQA."""
    B, Hq, Hkv, N, dt, causal, nw = case
    assert small_grid_waves_d64(B, Hq, N, causal) == nw
    q, k, v = workloads.random_case(5100 + N + Hq, B, Hq, Hkv, N, 64, dt)
    check_fwd(q, k, v, causal, 0.125, label=f"d=64 key-split {nw} waves")


def test_forward_is_bitwise_deterministic():
    w = workloads.WORKLOADS["b4_h32_n4096_d128_bf16_causal_qx8"]
    q, k, v = to_dev(*workloads.random_case(9, 2, 8, 2, 2048, 128, torch.bfloat16))
    o1, l1 = fa.fwd(q, k, v, causal=True)
    o2, l2 = fa.fwd(q, k, v, causal=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    del w


@pytest.mark.parametrize("d,dt,N", [(128, torch.bfloat16, 1000), (64, torch.float16, 777), (128, torch.float16, 4100)])
def test_forward_writes_every_output_element(d, dt, N):
    """O and LSE prefilled with NaN: after fa_fwd every element is finite and matches the
    oracle on sampled rows (each lane's 16-byte pieces of O, swapped between the two
    half-waves, must land on the row's every column)."""
    B, Hq, Hkv = 2, 4, 2
    q, k, v = workloads.random_case(700 + N + d, B, Hq, Hkv, N, d, dt)
    qd, kd, vd = to_dev(q, k, v)
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device="cuda:0")
    for causal in (False, True):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        fa.fwd(qd, kd, vd, causal=causal, out=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all() and torch.isfinite(lse).all()
        rows = np.array([0, 1, 31, 32, 63, 200, N // 2, N - 2, N - 1])
        O_ref, L_ref = oracle.attention_fwd(q, k, v, causal, 1 / math.sqrt(d), rows=rows)
        assert o_err(o[:, :, rows].cpu(), O_ref) <= O_TOL[dt]
        assert lse_err(lse[:, :, rows].cpu(), L_ref) <= LSE_TOL


def test_forward_allocates_nothing():
    """fa_fwd allocates no device memory: torch's allocator sees only O and LSE."""
    q, k, v = to_dev(*workloads.random_case(10, 1, 8, 8, 1024, 128, torch.bfloat16))
    o = torch.empty_like(q)
    lse = torch.empty(1, 8, 1024, dtype=torch.float32, device="cuda:0")
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(3):
        fa.fwd(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0


def test_empty_inputs():
    q = torch.empty(0, 2, 16, 64, dtype=torch.float16, device="cuda:0")
    o, lse = fa.fwd(q, q[:, :1], q[:, :1])
    assert o.shape == q.shape and lse.shape == (0, 2, 16)
    q = torch.empty(1, 2, 0, 64, dtype=torch.float16, device="cuda:0")
    o, lse = fa.fwd(q, q, q, causal=True)
    assert o.numel() == 0 and lse.numel() == 0


def test_rejects_unsupported_on_gpu():
    q = torch.zeros(1, 1, 8, 96, dtype=torch.float16, device="cuda:0")
    with pytest.raises(fa.FaError) as e:
        fa.fwd(q, q, q)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
