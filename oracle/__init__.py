"""fp64 CPU oracle for exact softmax attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
this package: only the test suite, the smoke check in ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` use it.  It shares no code with the HIP path.

It is the plain, materialising definition of scaled dot-product attention written
out in numpy float64 (see :mod:`oracle.attention` for the passages each function
follows), plus the footprint arithmetic of the pages' worked example, and the
few-queries / long-key-sequence case with the log-sum-exp combine of split-KV
decoding (:mod:`oracle.decode`), and the FP8 path with per-block scales and the
random-sign Hadamard transform (:mod:`oracle.fp8`), and the mask family: packed
variable-length batches, unequal query/key lengths, sliding windows and block-sparse
tile lists (:mod:`oracle.masks`).
"""
from .attention import (
    attention_fwd,
    attention_bwd,
    attention_probs,
    materialised_bytes,
    to_f64,
)
from .decode import attention_fwd_kv, lse_combine
from .fp8 import attention_fwd_fp8, quantize as fp8_quantize, dequantize as fp8_dequantize
from .masks import attention_fwd_masked, visible_pairs

__all__ = [
    "attention_fwd",
    "attention_bwd",
    "attention_probs",
    "materialised_bytes",
    "to_f64",
    "attention_fwd_kv",
    "lse_combine",
    "attention_fwd_fp8",
    "fp8_quantize",
    "fp8_dequantize",
    "attention_fwd_masked",
    "visible_pairs",
]
