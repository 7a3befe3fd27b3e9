"""Work and traffic conventions used to turn kernel times into throughput.

FLOP convention: the forward pass counts its two N x N x d matrix products,
4 * B * Hq * N^2 * d, halved when causal ("FlashAttention Primer", section
"Why attention is quadratic", gives the two products; the flash-attention-sm75
README's "Performance" tables reproduce with exactly this count at batch*heads = 8).
The backward pass counts five such products (recomputed Q K^T, P^T dO, dO V^T,
dS K, dS^T Q): 10 * B * Hq * N^2 * d, halved when causal.  The pages give no
backward convention; this is the reading used throughout.

Bytes: the compulsory HBM traffic of the forward pass is reading Q, K, V once and
writing O and the fp32 log-sum-exp once.  Split-KV decoding is bound by that traffic
(every cached K/V byte is read once per call; the arithmetic is small), so it is
measured in bytes per second against the HBM peak.
"""
from __future__ import annotations

# MI355X (gfx950) published dense peaks.
MFMA_BF16_TFLOPS = 2516.6          # 256 CUs x 4096 flop/clk/CU x 2.4 GHz
MFMA_FP8_TFLOPS = 5033.2           # 256 CUs x 8192 flop/clk/CU x 2.4 GHz (dense)
HBM_GBPS = 8000.0


def fwd_flops(B: int, Hq: int, N: int, d: int, causal: bool) -> float:
    f = 4.0 * B * Hq * N * N * d
    return f / 2 if causal else f


def bwd_flops(B: int, Hq: int, N: int, d: int, causal: bool) -> float:
    f = 10.0 * B * Hq * N * N * d
    return f / 2 if causal else f


def fwd_bytes(B: int, Hq: int, Hkv: int, N: int, d: int, elt_bytes: int) -> float:
    """Compulsory forward traffic: Q, K, V read once; O and fp32 LSE written once."""
    return (2.0 * B * Hq + 2.0 * B * Hkv) * N * d * elt_bytes + 4.0 * B * Hq * N


def bwd_bytes(B: int, Hq: int, Hkv: int, N: int, d: int, elt_bytes: int) -> float:
    """Compulsory backward traffic: Q, O, dO, dQ (Hq heads), K, V, dK, dV (Hkv heads), LSE."""
    return (4.0 * B * Hq + 4.0 * B * Hkv) * N * d * elt_bytes + 4.0 * B * Hq * N


def decode_bytes(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, elt_bytes: int) -> float:
    """Compulsory split-KV traffic: K, V (Nk rows) and Q read once, O and fp32 LSE written once."""
    return 2.0 * B * Hkv * Nk * d * elt_bytes + 2.0 * B * Hq * Nq * d * elt_bytes + 4.0 * B * Hq * Nq


def fp8_quant_bytes(B: int, Hq: int, Hkv: int, N: int, d: int, elt_bytes: int, block_q: int, block_kv: int) -> float:
    """Compulsory traffic of quantising Q, K and V: each input read once, one code byte per
    element and one fp32 scale per block written (value tiles padded to 64 keys)."""
    nkb = -(-N // 64) * 64
    return ((B * Hq + 2.0 * B * Hkv) * N * d * elt_bytes + (B * Hq + B * Hkv) * N * d + B * Hkv * nkb * d
            + 4.0 * (B * Hq * -(-N // block_q) + 2 * B * Hkv * -(-N // block_kv)))
