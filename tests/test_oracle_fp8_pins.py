"""Pins of the FP8 oracle (oracle/fp8.py) to facts outside itself.

* The e4m3 code table equals torch's float8_e4m3fn decoding of all 256 bit patterns,
  and rounding equals torch's float32 -> float8_e4m3fn cast (an independent library
  routine) on every midpoint, its neighbours and random values over the whole range.
* The Hadamard matrix equals the closed form H[i, j] = (-1)^popcount(i & j) and
  H H^T = d I; the transform is orthogonal (dot products and norms are kept) and
  maps a one-hot outlier onto d entries of equal magnitude.
* Block scales: the block maximum lands in (224, 448] after scaling, every code is
  within half a unit in the last place, and a block's scale depends on that block only.
* The stated rounding point: a value just above a midpoint that float32 rounds onto
  the midpoint is decided by ties-to-even.
* Special case that reduces to exact attention: operands that are e4m3 values times
  powers of two in the transformed domain are quantised without error, so the FP8
  oracle equals the exact forward oracle.
* The pages' qualitative claim: on inputs with outliers the random-sign Hadamard
  transform lowers the error of FP8 attention against exact attention, and per-block
  scales lower it when one block holds the large values.
Each planted mistake in MUTANTS must fail at least one pin.
"""
from __future__ import annotations

import math
import types
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as oracle_fp8
from workloads import randn


def _torch_e4m3(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_table_matches_torch(mod):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    t = mod.e4m3_values()
    assert np.array_equal(np.isnan(t), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(t[ok], ref[ok])


def pin_rounding_matches_torch(mod):
    vals = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    mids = 0.5 * (vals[:-1] + vals[1:])                       # exact in float32
    m32 = mids.astype(np.float32)
    xs = [vals, mids, np.nextafter(m32, np.float32(np.inf)), np.nextafter(m32, np.float32(0))]
    g = np.random.Generator(np.random.PCG64(77))
    xs.append((np.exp2(g.uniform(-12, 8.8, 20000)) * g.uniform(1, 2, 20000)).astype(np.float32))
    x = np.concatenate([np.asarray(a, dtype=np.float64) for a in xs])
    x = np.minimum(x, 448.0).astype(np.float32).astype(np.float64)
    x = np.concatenate([x, -x])
    got = mod.e4m3_encode(x)
    want = _torch_e4m3(x)
    zero = (got & 0x7F) == 0
    assert np.array_equal(zero, (want & 0x7F) == 0)
    assert np.array_equal(got[~zero], want[~zero])


def pin_hadamard_closed_form(mod):
    for d in (1, 2, 8, 64, 128):
        H = mod.hadamard(d)
        i, j = np.meshgrid(np.arange(d), np.arange(d), indexing="ij")
        pc = np.vectorize(lambda a: bin(int(a)).count("1"))(i & j)
        assert np.array_equal(H, np.where(pc % 2 == 0, 1.0, -1.0))
        assert np.array_equal(H @ H.T, d * np.eye(d))


def pin_transform_orthogonal(mod):
    for d in (64, 128):
        g = np.random.Generator(np.random.PCG64(d))
        s = g.integers(0, 2, d) * 2.0 - 1.0
        q = randn(5, (3, 7, d), torch.bfloat16)
        k = randn(6, (3, 9, d), torch.bfloat16)
        Qt, Kt = mod.incoherent(q, s), mod.incoherent(k, s)
        Q, K = q.double().numpy(), k.double().numpy()
        ref = Q @ np.swapaxes(K, -1, -2)
        got = Qt @ np.swapaxes(Kt, -1, -2)
        assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))
        assert np.allclose(np.linalg.norm(Qt, axis=-1), np.linalg.norm(Q, axis=-1), rtol=1e-13, atol=0)
        # a lone outlier is spread evenly: (A e_j) diag(s) H / sqrt(d) has |entries| = A / sqrt(d)
        x = np.zeros((1, d))
        x[0, d // 3] = 40.0
        assert np.allclose(np.abs(mod.incoherent(x, s)), 40.0 / math.sqrt(d), rtol=1e-15, atol=0)


def pin_inv_sqrt(mod):
    getcontext().prec = 60
    for d in (4, 32, 64, 128, 256):
        c = mod.inv_sqrt(d)
        x = Decimal(1) / Decimal(d).sqrt()
        err = [abs(Decimal(float(t)) - x) for t in (c, np.nextafter(c, 0), np.nextafter(c, 1))]
        assert err[0] < err[1] and err[0] < err[2]       # the float64 value nearest 1/sqrt(d)


def pin_block_scales(mod):
    g = np.random.Generator(np.random.PCG64(3))
    x = g.standard_normal((2, 300, 16)) * np.exp2(g.integers(-20, 20, (2, 300, 1)))
    x[1, 64:128] = 0.0                                        # an all-zero block
    codes, scales = mod.quantize(x, 64)
    assert scales.shape == (2, 5)
    e = np.log2(scales)
    assert np.array_equal(e, np.round(e))                     # powers of two
    x32 = x.astype(np.float32).astype(np.float64)
    vals = mod.e4m3_decode(codes)
    for b in range(2):
        for blk in range(5):
            r = slice(64 * blk, min(64 * blk + 64, 300))
            amax = np.max(np.abs(x32[b, r]))
            if amax == 0:
                assert scales[b, blk] == 1.0 and np.all((codes[b, r] & 0x7F) == 0)
                continue
            assert 224.0 < amax / scales[b, blk] <= 448.0
            y = x32[b, r] / scales[b, blk]
            v = vals[b, r]
            # half an ulp: 2^-4 relative for normal codes, 2^-10 absolute below 2^-6
            bound = np.where(np.abs(y) >= 2.0 ** -6, 2.0 ** -4 * np.abs(y) * (1 + 1e-12), 2.0 ** -10)
            assert np.all(np.abs(v - y) <= bound)
    # a block's scale depends on that block alone
    x2 = x.copy()
    x2[0, 130, 3] = 1e3 * np.max(np.abs(x[0, 128:192]))
    _, s2 = mod.quantize(x2, 64)
    changed = s2 != scales
    assert changed[0, 2] and changed.sum() == 1


def pin_fp32_rounding_point(mod):
    # 1.0625 is the midpoint of 1.0 (code 0x38) and 1.125 (0x39); 1.0625 + 2^-40 rounds to
    # 1.0625 in float32 and the tie then goes to the even code.  448 fixes the scale at 1.
    x = np.array([[[1.0625 + 2.0 ** -40, 448.0, -1.0625 - 2.0 ** -40]]])
    codes, scales = mod.quantize(x, 1)
    assert scales[0, 0] == 1.0
    assert list(codes[0, 0]) == [0x38, 0x7E, 0xB8]


def _exact_operands(mod, seed, d, B=1, H=2, N=150):
    """Q, K, V whose transformed (Q, K) or plain (V) values are e4m3 values times one power of
    two per 64-row block, with each block's magnitude reaching (224, 448] * 2^e."""
    g = np.random.Generator(np.random.PCG64(seed))
    s = g.integers(0, 2, d) * 2.0 - 1.0
    vals = mod.e4m3_values()[:127]
    out = []
    for t in range(3):
        C = vals[g.integers(0, 127, (B, H, N, d))] * np.where(g.random((B, H, N, d)) < 0.5, -1.0, 1.0)
        C[..., ::64, 0] = 448.0                              # fix each block's maximum
        e = g.integers(-3, 3, (B, H, -(-N // 64)))
        C = C * np.repeat(np.exp2(e), 64, axis=-1)[..., :N, None] / 64.0
        if t < 2:   # undo M = diag(s) H / sqrt(d): x = C M^T = C H diag(s) / sqrt(d)  (d = 64: exact)
            out.append((C @ mod.hadamard(d).T) * s / math.sqrt(d))
        else:
            out.append(C)
    return out, s


def pin_exact_special_case(mod):
    (q, k, v), s = _exact_operands(mod, 21, 64)
    Qh, Kh, Vh = mod.quantized_operands(q, k, v, s, 64, 64)
    assert np.array_equal(Qh, mod.incoherent(q, s)) and np.array_equal(Vh, v)
    for causal in (False, True):
        O, L = mod.attention_fwd_fp8(q, k, v, s, causal, 0.05, 64, 64)
        O2, L2 = oracle.attention_fwd(q, k, v, causal, 0.05)
        assert np.max(np.abs(O - O2)) <= 1e-12 * np.max(np.abs(O2))
        assert np.max(np.abs(L - L2)) <= 1e-11


def _outlier_inputs(seed, shape, frac, mult):
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(size=shape, dtype=np.float32)
    x[g.random(size=shape, dtype=np.float32) < frac] *= mult
    return torch.from_numpy(x).to(torch.bfloat16)


def pin_error_claims(mod):
    B, H, N, d = 1, 2, 256, 64
    q, k, v = (_outlier_inputs(40 + i, (B, H, N, d), 1e-2, 16.0) for i in range(3))
    s = np.random.Generator(np.random.PCG64(41)).integers(0, 2, d) * 2.0 - 1.0
    sc = 0.125
    O, _ = oracle.attention_fwd(q, k, v, False, sc)

    def rms(signs, bq, bkv, qq=q, kk=k, vv=v, ref=O):
        O2, _ = mod.attention_fwd_fp8(qq, kk, vv, signs, False, sc, bq, bkv)
        return float(np.sqrt(np.mean((O2 - ref) ** 2)))

    per_tensor = rms(None, N, N)
    rotated = rms(s, N, N)
    assert per_tensor > 1.5 * rotated            # the transform lowers the error on outlier inputs
    # without outliers it neither helps nor hurts much
    q0, k0, v0 = (randn(50 + i, (B, H, N, d), torch.bfloat16) for i in range(3))
    O0, _ = oracle.attention_fwd(q0, k0, v0, False, sc)
    r0, r1 = rms(None, N, N, q0, k0, v0, O0), rms(s, N, N, q0, k0, v0, O0)
    assert 0.7 < r0 / r1 < 1.4
    # per-block scales help when one block holds the large values: V rows 192..255 scaled by
    # 2^14 and a causal mask, so queries 0..191 see only the ordinary blocks
    big = v0.clone()
    big[:, :, 192:] *= 16384.0
    Ob, _ = oracle.attention_fwd(q0, k0, big, True, sc)
    err = {}
    for bkv in (64, N):
        O2, _ = mod.attention_fwd_fp8(q0, k0, big, s, True, sc, 64, bkv)
        err[bkv] = float(np.sqrt(np.mean((O2 - Ob)[:, :, :192] ** 2)))
    assert err[N] > 2.0 * err[64]


PINS = [pin_table_matches_torch, pin_rounding_matches_torch, pin_hadamard_closed_form, pin_transform_orthogonal,
        pin_inv_sqrt, pin_block_scales, pin_fp32_rounding_point, pin_exact_special_case, pin_error_claims]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_fp8_oracle_pins(pin):
    pin(oracle_fp8)


MUTANTS = {
    "ties_away_from_zero": ("n = np.rint(a / step)", "n = np.floor(a / step + 0.5)"),
    "subnormal_spacing_2e_minus_10": ("np.rint(r * 2.0 ** 9)", "np.rint(r * 2.0 ** 10)"),
    "fnuz_bias_8": ("2.0 ** (exp.astype(np.float64) - 7)", "2.0 ** (exp.astype(np.float64) - 8)"),
    "hadamard_other_sign": ("H = np.block([[H, H], [H, -H]])", "H = np.block([[H, H], [-H, H]])"),
    "normalised_by_1_over_d": ("return ((X * s) @ hadamard(d)) * inv_sqrt(d)", "return ((X * s) @ hadamard(d)) / d"),
    "signs_dropped": ("return ((X * s) @ hadamard(d)) * inv_sqrt(d)", "return (X @ hadamard(d)) * inv_sqrt(d)"),
    "exponent_one_low": ("e = np.where(pos, e, 0)", "e = np.where(pos, e - 1, 0)"),
    "no_fp32_rounding_point": ("X = X.astype(np.float32).astype(np.float64)", "X = X"),
    "scale_per_column": ("s = np.repeat(np.asarray(scales, dtype=np.float64), block_rows, axis=-1)[..., :N]\n    return vals * s[..., None]",
                         "s = np.repeat(np.asarray(scales, dtype=np.float64), block_rows, axis=-1)[..., :N]\n    return vals * s[..., :1, None]"),
    "v_transformed_too": ("Vh = dequantize(*quantize(v, block_kv, None), block_kv)",
                          "Vh = dequantize(*quantize(v, block_kv, signs), block_kv)"),
    "sqrt2_double_rounded": ("else math.ldexp(math.sqrt(2.0), -(k + 1) // 2)", "else 1.0 / math.sqrt(d)"),
}


def _mutant(old, new):
    src = open(oracle_fp8.__file__).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle.fp8_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "oracle_fp8_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_fp8_pins_catch_planted_mistake(name):
    mod = _mutant(*MUTANTS[name])
    failed = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(mod)
            except (AssertionError, ValueError, IndexError, FloatingPointError):
                failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {name}"
