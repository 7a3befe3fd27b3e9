"""FP8 (e4m3) forward attention with per-block scales and incoherent processing,
in float64 — the oracle (test infrastructure only).

Sources (page title, then the part of the page):

* "Flash Attention" (wiki), section "FlashAttention-3": the low-precision path
  combines block quantization with an incoherent-processing transform made of
  random signs and a Hadamard transform; the same orthogonal transform is applied
  to the queries and to the keys, which leaves their dot products unchanged in
  exact arithmetic and spreads outliers over all coordinates.  The page contrasts
  it with a baseline that quantizes each tensor with one scale.
* "FlashAttention Primer: IO-Aware Attention, from FA1 to FA4", section
  "FlashAttention-3: Hopper asynchrony and FP8": scores are quantized in blocks and
  a random rotation is applied before quantization.
* "FlashAttention" (explainer), section "What Hopper bought FlashAttention-3":
  accuracy of the FP8 path is kept by per-block scaling.
* Attention itself is :func:`oracle.attention.attention_fwd` on the dequantised
  operands.

Readings taken where the pages are silent (each is listed with the others in the
design notes):

* Format: e4m3 with the "fn" conventions — sign bit, 4 exponent bits with bias 7,
  3 mantissa bits, subnormals when the exponent field is 0, no infinities, the two
  all-ones codes are NaN, largest finite magnitude 448.  Rounding is to nearest,
  ties to the even code; a negative value that rounds to zero keeps its sign.
* Transform: M = diag(sigma) H_d / sqrt(d) with sigma a vector of d random signs
  (an input) and H_d the Sylvester Hadamard matrix of order d (d a power of two),
  so M is orthogonal.  Q and K are multiplied by M on the right; V is not
  transformed.  The product x diag(sigma) H_d is a signed sum of the inputs and is
  formed exactly in float64 (half-precision inputs); 1/sqrt(d) is applied as one
  float64 multiplication by the float64 value nearest 1/sqrt(d).
* Blocks: a block is `block_rows` consecutive rows (positions) of one head, all d
  columns; the last block of a head may be short.
* Scale: the transformed values are rounded to float32; each block gets the
  power-of-two scale 2^e with e the smallest integer such that the block's largest
  magnitude is at most 448 * 2^e (e = 0 for an all-zero block; e is clamped to
  [-127, 127]).  Codes are e4m3(x / 2^e); the division by a power of two is exact,
  so each code is decided by one rounding of a float32 value.
* The attention is exact (float64) attention of the dequantised operands
  scale_block * value(code) with the caller's softmax scale.  The probabilities
  are not rounded here: a kernel that feeds them to an FP8 product rounds them,
  and that rounding is what its tolerance covers.

Parity pins: tests/test_oracle_fp8_pins.py.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import attention_fwd, to_f64

E4M3_MAX = 448.0
E_MIN, E_MAX = -127, 127


def e4m3_values() -> np.ndarray:
    """Values of the 256 e4m3 codes (NaN for 0x7f and 0xff), decoded field by field."""
    codes = np.arange(256)
    sign = np.where(codes >> 7, -1.0, 1.0)
    exp = (codes >> 3) & 0xF
    man = codes & 0x7
    mag = np.where(exp == 0, man / 8.0 * 2.0 ** -6, (1.0 + man / 8.0) * 2.0 ** (exp.astype(np.float64) - 7))
    mag = np.where((exp == 0xF) & (man == 0x7), np.nan, mag)
    return sign * mag


_TABLE = e4m3_values()


def e4m3_encode(x) -> np.ndarray:
    """Round float64 values with |x| <= 448 to the nearest e4m3 code (ties to even).

    The e4m3 values in [2^E, 2^(E+1)) (E >= -6) are spaced 2^(E-3) apart, and those
    below 2^-6 are the multiples of 2^-9; |x| divided by its spacing (exact: a power of
    two) is rounded to the nearest integer, ties to the even one, which is the value's
    significand in units of the spacing, so its parity is the code's last bit.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode needs finite values with |x| <= 448")
    a = np.abs(x)
    _, e = np.frexp(a)                                  # a = m 2^e, m in [0.5, 1)
    E = np.maximum(e - 1, -6)                           # binade of a; the subnormals share 2^-6's spacing
    step = np.ldexp(1.0, E - 3)
    n = np.rint(a / step)                               # round half to even
    r = n * step                                        # the chosen e4m3 magnitude
    _, er = np.frexp(r)
    Er = er - 1
    normal = r >= 2.0 ** -6
    man = np.where(normal, np.rint(np.ldexp(r, -Er) * 8) - 8, np.rint(r * 2.0 ** 9))
    code = np.where(normal, (Er + 7) * 8 + man, man).astype(np.int64)
    code = code | np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.int64)]


def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (entries +-1): H_1 = [1], H_2n = [[H, H], [H, -H]]."""
    if d < 1 or d & (d - 1):
        raise ValueError("Hadamard order must be a power of two")
    H = np.ones((1, 1))
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    return H


def inv_sqrt(d: int) -> float:
    """The float64 value nearest 1/sqrt(d) for d a power of two: 2^(-k/2) for even k = log2 d,
    else the float64 value nearest sqrt(2) times 2^(-(k+1)/2) (scaling by 2^j commutes with rounding)."""
    k = d.bit_length() - 1
    if d != 1 << k:
        raise ValueError("d must be a power of two")
    return math.ldexp(1.0, -k // 2) if k % 2 == 0 else math.ldexp(math.sqrt(2.0), -(k + 1) // 2)


def incoherent(x, signs) -> np.ndarray:
    """x M with M = diag(signs) H_d / sqrt(d), along the last axis, float64."""
    X = to_f64(x)
    d = X.shape[-1]
    s = np.asarray(signs, dtype=np.float64)
    if s.shape != (d,) or not np.all(np.abs(s) == 1.0):
        raise ValueError("signs must be d values of +-1")
    return ((X * s) @ hadamard(d)) * inv_sqrt(d)


def block_exponents(amax: np.ndarray) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e (0 where amax == 0), clamped to [-127, 127]."""
    amax = np.asarray(amax, dtype=np.float64)
    pos = amax > 0
    e = np.zeros(amax.shape, dtype=np.int64)
    safe = np.where(pos, amax, E4M3_MAX)
    e = np.ceil(np.log2(safe / E4M3_MAX)).astype(np.int64)
    e = np.where(safe > E4M3_MAX * np.ldexp(1.0, e), e + 1, e)       # log2 may be one off either way
    e = np.where(safe <= E4M3_MAX * np.ldexp(1.0, e - 1), e - 1, e)
    e = np.where(pos, e, 0)
    return np.clip(e, E_MIN, E_MAX)


def quantize(x, block_rows: int, signs=None):
    """Block quantisation of x [..., N, d] (optionally transformed first).

    Returns (codes uint8 [..., N, d], scales float64 [..., ceil(N / block_rows)]),
    scales being powers of two.
    """
    if block_rows < 1:
        raise ValueError("block_rows must be positive")
    X = incoherent(x, signs) if signs is not None else to_f64(x)
    X = X.astype(np.float32).astype(np.float64)          # the rounding point before quantisation
    N = X.shape[-2]
    nb = -(-N // block_rows)
    pad = nb * block_rows - N
    A = np.abs(X)
    if pad:
        A = np.concatenate([A, np.zeros(A.shape[:-2] + (pad, A.shape[-1]))], axis=-2)
    amax = A.reshape(A.shape[:-2] + (nb, block_rows * A.shape[-1])).max(axis=-1)
    e = block_exponents(amax)
    per_row = np.repeat(e, block_rows, axis=-1)[..., :N]
    codes = e4m3_encode(np.ldexp(X, -per_row[..., None]))
    return codes, np.ldexp(1.0, e)


def dequantize(codes, scales, block_rows: int) -> np.ndarray:
    """scale of the row's block times the value of each code, float64."""
    vals = e4m3_decode(codes)
    N = vals.shape[-2]
    s = np.repeat(np.asarray(scales, dtype=np.float64), block_rows, axis=-1)[..., :N]
    return vals * s[..., None]


def quantized_operands(q, k, v, signs, block_q: int, block_kv: int):
    """Dequantised (Q-hat, K-hat, V-hat): Q and K transformed and block-quantised, V block-quantised.

    signs=None skips the transform (block quantisation alone).
    """
    Qh = dequantize(*quantize(q, block_q, signs), block_q)
    Kh = dequantize(*quantize(k, block_kv, signs), block_kv)
    Vh = dequantize(*quantize(v, block_kv, None), block_kv)
    return Qh, Kh, Vh


def attention_fwd_fp8(q, k, v, signs, causal: bool, scale: float, block_q: int = 64, block_kv: int = 64,
                      rows=None):
    """(O, LSE) of exact attention over the dequantised FP8 operands, float64."""
    Qh, Kh, Vh = quantized_operands(q, k, v, signs, block_q, block_kv)
    return attention_fwd(Qh, Kh, Vh, causal, scale, rows=rows)
