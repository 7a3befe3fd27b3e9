"""Thin Python binding of the C ABI in include/fa.h (argument marshalling only).

torch supplies device memory and the current stream; every step of the attention
computation runs in the HIP kernels of libfa.so.  There is no fallback: if the
library is missing or a call fails, an exception is raised.

torch is imported before libfa.so is loaded so that the library binds to the
HIP runtime torch already has in the process (both carry the same soname).
"""
from __future__ import annotations

import ctypes
import math
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "fa.h")

FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3
FA_F16, FA_BF16 = 0, 1

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_string(status)}: {detail}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libfa.so (built in-tree by exact_io_aware_fwd_amd.build) and declare its prototypes."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -m exact_io_aware_fwd_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    L.fa_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                         ctypes.c_int, ctypes.c_int, ctypes.c_float, _vp]
    L.fa_fwd.restype = ctypes.c_int
    L.fa_bwd_workspace_size.argtypes = [_i64, _i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int]
    L.fa_bwd_workspace_size.restype = ctypes.c_size_t
    L.fa_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                         _i64, _i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, ctypes.c_float, _vp]
    L.fa_bwd.restype = ctypes.c_int
    L.fa_bwd_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                 ctypes.c_int, ctypes.c_int, ctypes.c_float, _vp]
    L.fa_bwd_noalloc.restype = ctypes.c_int
    L.fa_fwd_splitkv.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _i64, _i64, _i64, _i64, _i64, _i64,
                                 ctypes.c_int, ctypes.c_int, ctypes.c_float, _i64, _vp]
    L.fa_fwd_splitkv.restype = ctypes.c_int
    L.fa_fwd_splitkv_workspace_size.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_int, _i64]
    L.fa_fwd_splitkv_workspace_size.restype = ctypes.c_size_t
    L.fa_fwd_splitkv_num_splits.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64]
    L.fa_fwd_splitkv_num_splits.restype = _i64
    L.fa_lse_combine.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, ctypes.c_int, _vp]
    L.fa_lse_combine.restype = ctypes.c_int
    L.fa_fwd_masked.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_int,
                                _vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _i64, ctypes.c_float, _vp]
    L.fa_fwd_masked.restype = ctypes.c_int
    L.fa_bwd_masked_workspace_size.argtypes = [_i64, _i64, _i64, _i64, _i64, ctypes.c_int]
    L.fa_bwd_masked_workspace_size.restype = ctypes.c_size_t
    L.fa_bwd_masked.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _i64, _i64, _i64,
                                _i64, _i64, _i64, ctypes.c_int, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _i64,
                                ctypes.c_float, _vp]
    L.fa_bwd_masked.restype = ctypes.c_int
    L.fa_fp8_v_codes_bytes.argtypes = [_i64, _i64, _i64, _i64]
    L.fa_fp8_v_codes_bytes.restype = ctypes.c_size_t
    L.fa_fp8_quantize_rows.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_int, _i64, _vp]
    L.fa_fp8_quantize_rows.restype = ctypes.c_int
    L.fa_fp8_quantize_v.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_int, _i64, _vp]
    L.fa_fp8_quantize_v.restype = ctypes.c_int
    L.fa_fwd_fp8.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                             ctypes.c_int, ctypes.c_float, _vp]
    L.fa_fwd_fp8.restype = ctypes.c_int
    L.fa_status_string.argtypes = [ctypes.c_int]
    L.fa_status_string.restype = ctypes.c_char_p
    L.fa_last_error.argtypes = []
    L.fa_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def declared_symbols() -> list[str]:
    """Names of the functions include/fa.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(fa_[a-z_0-9]+)\s*\(", text, re.M)))


def status_string(status: int) -> str:
    return load().fa_status_string(status).decode()


def last_error() -> str:
    return load().fa_last_error().decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return FA_F16
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float16 or bfloat16)")


def _check(t: torch.Tensor, name: str, device, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shapes(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"k, v must be [B, Hkv, N, d] matching q {tuple(q.shape)}; got {tuple(k.shape)}")
    return B, Hq, k.shape[1], N, d


def _raise(st: int):
    raise FaError(st, last_error())


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
        softmax_scale: float | None = None, out: torch.Tensor | None = None,
        lse: torch.Tensor | None = None):
    """O, LSE = attention(q, k, v) via fa_fwd on the current stream.

    q [B,Hq,N,d], k/v [B,Hkv,N,d] (fp16 or bf16, contiguous, same device);
    returns O [B,Hq,N,d] (q's dtype) and LSE [B,Hq,N] float32 (natural log).
    """
    L = load()
    B, Hq, Hkv, N, d = _shapes(q, k, v)
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, dev, q.dtype)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, Hq, N), dtype=torch.float32, device=dev) if lse is None else lse
    _check(o, "out", dev, q.dtype)
    _check(lse_t, "lse", dev, torch.float32)
    if o.shape != q.shape or lse_t.shape != (B, Hq, N):
        raise ValueError("out/lse have the wrong shape")
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = L.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse_t.data_ptr(),
                      B, Hq, Hkv, N, d, _dtype_code(q), int(bool(causal)), scale, stream)
    if st != FA_OK:
        _raise(st)
    return o, lse_t


def bwd_workspace_size(B: int, Hq: int, Hkv: int, N: int, d: int, dtype, causal: bool) -> int:
    code = FA_BF16 if dtype == torch.bfloat16 else FA_F16
    return int(load().fa_bwd_workspace_size(B, Hq, Hkv, N, d, code, int(bool(causal))))


def bwd(q, k, v, o, lse, do, causal: bool = False, softmax_scale: float | None = None,
        workspace: torch.Tensor | None = None):
    """dQ, dK, dV via fa_bwd on the current stream (workspace allocated by torch if not given)."""
    L = load()
    B, Hq, Hkv, N, d = _shapes(q, k, v)
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _check(t, n, dev, q.dtype)
    _check(lse, "lse", dev, torch.float32)
    if o.shape != q.shape or do.shape != q.shape or lse.shape != (B, Hq, N):
        raise ValueError("o/do/lse have the wrong shape")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    need = bwd_workspace_size(B, Hq, Hkv, N, d, q.dtype, causal)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev) if workspace is None else workspace
    _check(ws, "workspace", dev)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = L.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                      dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel(),
                      B, Hq, Hkv, N, d, _dtype_code(q), int(bool(causal)), scale, stream)
    if st != FA_OK:
        _raise(st)
    return dq, dk, dv


# Bytes of the static device scratch behind fa_bwd_noalloc (include/fa.h).
NOALLOC_SCRATCH_BYTES = 64 << 20


def bwd_noalloc(q, k, v, o, lse, do, causal: bool = False, softmax_scale: float | None = None, out=None):
    """dQ, dK, dV via fa_bwd_noalloc: fa_bwd with its workspace in the library's static
    device scratch (no workspace argument; calls that overlap on one GPU race).  `out`
    optionally gives preallocated (dq, dk, dv)."""
    L = load()
    B, Hq, Hkv, N, d = _shapes(q, k, v)
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _check(t, n, dev, q.dtype)
    _check(lse, "lse", dev, torch.float32)
    if o.shape != q.shape or do.shape != q.shape or lse.shape != (B, Hq, N):
        raise ValueError("o/do/lse have the wrong shape")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dq, dk, dv = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)) if out is None else out
    for t, ref, n in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        _check(t, n, dev, q.dtype)
        if t.shape != ref.shape:
            raise ValueError(f"{n} has the wrong shape")
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = L.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                              dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, N, d, _dtype_code(q),
                              int(bool(causal)), scale, stream)
    if st != FA_OK:
        _raise(st)
    return dq, dk, dv


def splitkv_workspace_size(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, dtype, num_splits: int = 0) -> int:
    code = FA_BF16 if dtype == torch.bfloat16 else FA_F16
    return int(load().fa_fwd_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, code, num_splits))


def splitkv_num_splits(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int) -> int:
    return int(load().fa_fwd_splitkv_num_splits(B, Hq, Hkv, Nq, Nk, d))


def fwd_splitkv(q, k, v, causal: bool = False, softmax_scale: float | None = None, num_splits: int = 0,
                workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                lse: torch.Tensor | None = None):
    """O, LSE of q [B,Hq,Nq,d] against k/v [B,Hkv,Nk,d] via fa_fwd_splitkv (split-KV decoding).

    Query i is at position Nk - Nq + i (causal: sees keys j <= Nk - Nq + i).
    """
    L = load()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, Nq, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"k, v must be [B, Hkv, Nk, d] matching q {tuple(q.shape)}; got {tuple(k.shape)}")
    Hkv, Nk = k.shape[1], k.shape[2]
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, dev, q.dtype)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev) if lse is None else lse
    _check(o, "out", dev, q.dtype)
    _check(lse_t, "lse", dev, torch.float32)
    need = splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, q.dtype, num_splits)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev) if workspace is None else workspace
    _check(ws, "workspace", dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = L.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse_t.data_ptr(),
                              ws.data_ptr(), ws.numel(), B, Hq, Hkv, Nq, Nk, d, _dtype_code(q),
                              int(bool(causal)), scale, int(num_splits), stream)
    if st != FA_OK:
        _raise(st)
    return o, lse_t


def lse_combine(o_parts: torch.Tensor, lse_parts: torch.Tensor, dtype=torch.bfloat16):
    """Merge partial results: o_parts [rows, S, d] fp32, lse_parts [rows, S] fp32 -> (O [rows, d], LSE [rows])."""
    L = load()
    if o_parts.dim() != 3 or lse_parts.dim() != 2 or o_parts.shape[:2] != lse_parts.shape:
        raise ValueError("o_parts must be [rows, S, d] and lse_parts [rows, S]")
    rows, S, d = o_parts.shape
    dev = o_parts.device
    _check(o_parts, "o_parts", dev, torch.float32)
    _check(lse_parts, "lse_parts", dev, torch.float32)
    o = torch.empty((rows, d), dtype=dtype, device=dev)
    lse = torch.empty((rows,), dtype=torch.float32, device=dev)
    code = FA_BF16 if dtype == torch.bfloat16 else FA_F16
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = L.fa_lse_combine(o_parts.data_ptr(), lse_parts.data_ptr(), o.data_ptr(), lse.data_ptr(),
                              rows, S, d, code, stream)
    if st != FA_OK:
        _raise(st)
    return o, lse


def fp8_quantize(x: torch.Tensor, block_rows: int = 64, signs: torch.Tensor | None = None):
    """Block-quantise rows of x [B,H,N,d] (fp16/bf16) to e4m3 via fa_fp8_quantize_rows.

    signs: d float32 values of +-1 on x's device (the random-sign Hadamard transform is
    applied first), or None.  Returns (codes uint8 [B,H,N,d], scales float32
    [B,H,ceil(N/block_rows)]).
    """
    L = load()
    if x.dim() != 4:
        raise ValueError("x must be [B, H, N, d]")
    B, H, N, d = x.shape
    dev = x.device
    _check(x, "x", dev)
    if signs is not None:
        _check(signs, "signs", dev, torch.float32)
        if signs.shape != (d,):
            raise ValueError(f"signs must be [{d}]")
    codes = torch.empty((B, H, N, d), dtype=torch.uint8, device=dev)
    scales = torch.empty((B, H, -(-N // block_rows)), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = L.fa_fp8_quantize_rows(x.data_ptr(), None if signs is None else signs.data_ptr(), codes.data_ptr(),
                                    scales.data_ptr(), B, H, N, d, _dtype_code(x), block_rows, stream)
    if st != FA_OK:
        _raise(st)
    return codes, scales


def fp8_quantize_v(v: torch.Tensor, block_rows: int = 64):
    """Block-quantise values v [B,H,N,d] to e4m3 in the value-tile layout via fa_fp8_quantize_v.

    Returns (codes uint8 [B,H,ceil(N/64),d,64], scales float32 [B,H,ceil(N/block_rows)]).
    """
    L = load()
    if v.dim() != 4:
        raise ValueError("v must be [B, H, N, d]")
    B, H, N, d = v.shape
    dev = v.device
    _check(v, "v", dev)
    codes = torch.empty((B, H, -(-N // 64), d, 64), dtype=torch.uint8, device=dev)
    scales = torch.empty((B, H, -(-N // block_rows)), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = L.fa_fp8_quantize_v(v.data_ptr(), codes.data_ptr(), scales.data_ptr(), B, H, N, d, _dtype_code(v),
                                 block_rows, stream)
    if st != FA_OK:
        _raise(st)
    return codes, scales


def fwd_fp8(q8, k8, v8, q_scales, k_scales, v_scales, causal: bool = False, softmax_scale: float | None = None,
            block_q: int = 64, block_kv: int = 64, out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """O (bf16), LSE = FP8 attention over quantised operands via fa_fwd_fp8.

    q8 [B,Hq,N,d] and k8 [B,Hkv,N,d] from fp8_quantize, v8 [B,Hkv,ceil(N/64),d,64] from
    fp8_quantize_v, with their scales and block sizes.
    """
    L = load()
    if q8.dim() != 4 or k8.dim() != 4 or v8.dim() != 5:
        raise ValueError("q8, k8 must be [B, H, N, d] and v8 [B, H, ceil(N/64), d, 64]")
    B, Hq, N, d = q8.shape
    Hkv = k8.shape[1]
    if k8.shape != (B, Hkv, N, d) or v8.shape != (B, Hkv, -(-N // 64), d, 64):
        raise ValueError("k8 / v8 shapes do not match q8")
    dev = q8.device
    for t, n in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        _check(t, n, dev, torch.uint8)
    for t, n, blk, H in ((q_scales, "q_scales", block_q, Hq), (k_scales, "k_scales", block_kv, Hkv),
                         (v_scales, "v_scales", block_kv, Hkv)):
        _check(t, n, dev, torch.float32)
        if t.shape != (B, H, -(-N // blk)):
            raise ValueError(f"{n} must be [{B}, {H}, {-(-N // blk)}]")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    o = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=dev) if out is None else out
    lse_t = torch.empty((B, Hq, N), dtype=torch.float32, device=dev) if lse is None else lse
    _check(o, "out", dev, torch.bfloat16)
    _check(lse_t, "lse", dev, torch.float32)
    if o.shape != (B, Hq, N, d) or lse_t.shape != (B, Hq, N):
        raise ValueError("out/lse have the wrong shape")
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = L.fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), q_scales.data_ptr(), k_scales.data_ptr(),
                          v_scales.data_ptr(), o.data_ptr(), lse_t.data_ptr(), B, Hq, Hkv, N, d, block_q, block_kv,
                          int(bool(causal)), scale, stream)
    if st != FA_OK:
        _raise(st)
    return o, lse_t


def fp8_prepare(q, k, v, signs=None, block_q: int = 64, block_kv: int = 64):
    """Quantise q, k (transformed when signs is given) and v for fwd_fp8; returns the six operands."""
    q8, qs = fp8_quantize(q, block_q, signs)
    k8, ks = fp8_quantize(k, block_kv, signs)
    v8, vs = fp8_quantize_v(v, block_kv)
    return q8, k8, v8, qs, ks, vs


def block_lists_to_tensors(lists, maxq: int, maxk: int, device):
    """Nested block lists [B][Hm][query block] -> key tiles into (block_cnt, block_idx)
    int32 tensors of shapes [B, Hm, ceil(maxq/256)] and [B, Hm, ceil(maxq/256), ceil(maxk/64)]."""
    B, Hm = len(lists), len(lists[0])
    nqb, cap = -(-maxq // 256), -(-maxk // 64)
    cnt = torch.zeros((B, Hm, nqb), dtype=torch.int32)
    idx = torch.zeros((B, Hm, nqb, max(cap, 1)), dtype=torch.int32)
    for b in range(B):
        if len(lists[b]) != Hm:
            raise ValueError("every sequence needs the same number of head lists")
        for h in range(Hm):
            for qb, tiles in enumerate(lists[b][h][:nqb]):
                t = sorted(int(x) for x in tiles)[:cap]
                cnt[b, h, qb] = len(t)
                if t:
                    idx[b, h, qb, :len(t)] = torch.tensor(t, dtype=torch.int32)
    return cnt.to(device), idx.to(device)


def _check_lists(block_cnt, block_idx, B: int, mq: int, mk: int, dev) -> int:
    """Validate block-list tensors (as block_lists_to_tensors makes them); their head count."""
    if (block_cnt is None) != (block_idx is None):
        raise ValueError("give both block_cnt and block_idx, or neither")
    if block_idx is None:
        return 1
    _check(block_cnt, "block_cnt", dev, torch.int32)
    _check(block_idx, "block_idx", dev, torch.int32)
    bh = block_idx.shape[1]
    if block_cnt.dim() != 3 or block_idx.dim() != 4 or tuple(block_cnt.shape) != (B, bh, -(-mq // 256)) or \
            block_idx.shape[:3] != block_cnt.shape or block_idx.shape[3] != max(-(-mk // 64), 1):
        raise ValueError("block_cnt / block_idx have the wrong shape")
    return bh


def _masked_geometry(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, dev):
    """Sizes of a mask-family call, with the layout checks both passes make before the ABI:
    (B, Hq, Hkv, Nq, Nk, d, longest query length, longest key length, LSE shape)."""
    if cu_seqlens_q is not None:
        if q.dim() != 3 or k.dim() != 3 or v.dim() != 3 or k.shape != v.shape:
            raise ValueError("packed q, k, v must be [H, total, d] with k.shape == v.shape")
        Hq, Nq, d = q.shape
        Hkv, Nk = k.shape[0], k.shape[1]
        if k.shape[2] != d:
            raise ValueError("packed k, v must be [Hkv, total_k, d] matching q")
        B = cu_seqlens_q.numel() - 1
        if cu_seqlens_k is None or cu_seqlens_k.numel() != B + 1:
            raise ValueError("cu_seqlens_k must have B+1 entries like cu_seqlens_q")
        for t, n in ((cu_seqlens_q, "cu_seqlens_q"), (cu_seqlens_k, "cu_seqlens_k")):
            _check(t, n, dev, torch.int32)
        mq = Nq if max_seqlen_q is None else int(max_seqlen_q)
        mk = Nk if max_seqlen_k is None else int(max_seqlen_k)
        return B, Hq, Hkv, Nq, Nk, d, mq, mk, (Hq, Nq)
    if cu_seqlens_k is not None:
        raise ValueError("cu_seqlens_k given without cu_seqlens_q")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or k.shape != v.shape:
        raise ValueError("q, k, v must be [B, H, N, d] with k.shape == v.shape")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k, v must be [B, Hkv, Nk, d] matching q")
    return B, Hq, Hkv, Nq, Nk, d, Nq, Nk, (B, Hq, Nq)


def fwd_masked(q, k, v, window=(-1, -1), softmax_scale: float | None = None, cu_seqlens_q=None, cu_seqlens_k=None,
               max_seqlen_q: int | None = None, max_seqlen_k: int | None = None, block_cnt=None, block_idx=None,
               out=None, lse=None):
    """O, LSE under the mask family via fa_fwd_masked.

    Fixed lengths: q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d].  Packed: q [Hq,Nq,d], k/v [Hkv,Nk,d]
    with cu_seqlens_q/k int32 [B+1] GPU tensors (max_seqlen_* default to Nq, Nk).
    window = (left, right), -1 unbounded; (-1, 0) is causal (bottom-right aligned).
    block_cnt/block_idx: int32 GPU tensors from block_lists_to_tensors, or None.
    """
    L = load()
    dev = q.device
    B, Hq, Hkv, Nq, Nk, d, mq, mk, lse_shape = _masked_geometry(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                                                                max_seqlen_k, dev)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, dev, q.dtype)
    bh = _check_lists(block_cnt, block_idx, B, mq, mk, dev)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty(lse_shape, dtype=torch.float32, device=dev) if lse is None else lse
    _check(o, "out", dev, q.dtype)
    _check(lse_t, "lse", dev, torch.float32)
    if o.shape != q.shape or tuple(lse_t.shape) != lse_shape:
        raise ValueError("out/lse have the wrong shape")
    ptr = lambda t: None if t is None else t.data_ptr()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = L.fa_fwd_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse_t.data_ptr(), B, Hq, Hkv,
                             Nq, Nk, d, _dtype_code(q), ptr(cu_seqlens_q), ptr(cu_seqlens_k), mq, mk,
                             int(window[0]), int(window[1]), ptr(block_cnt), ptr(block_idx), bh, scale, stream)
    if st != FA_OK:
        _raise(st)
    return o, lse_t


def bwd_masked(q, k, v, o, lse, do, window=(-1, -1), softmax_scale: float | None = None, cu_seqlens_q=None,
               cu_seqlens_k=None, max_seqlen_q: int | None = None, max_seqlen_k: int | None = None,
               block_cnt=None, block_idx=None, workspace: torch.Tensor | None = None):
    """dQ, dK, dV under the mask family via fa_bwd_masked (layouts and block lists as in
    fwd_masked)."""
    L = load()
    dev = q.device
    B, Hq, Hkv, Nq, Nk, d, mq, mk, lse_shape = _masked_geometry(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                                                                max_seqlen_k, dev)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _check(t, n, dev, q.dtype)
    _check(lse, "lse", dev, torch.float32)
    if o.shape != q.shape or do.shape != q.shape or tuple(lse.shape) != lse_shape:
        raise ValueError("o and do must match q, and lse must be " + str(lse_shape))
    bh = _check_lists(block_cnt, block_idx, B, mq, mk, dev)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    need = L.fa_bwd_masked_workspace_size(B, Hq, Hkv, mq, mk, int(block_idx is not None))
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev) if workspace is None else workspace
    _check(ws, "workspace", dev)
    dq, dk, dv = torch.empty_like(q), torch.zeros_like(k), torch.zeros_like(v)
    ptr = lambda t: None if t is None else t.data_ptr()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = L.fa_bwd_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                             dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel(), B, Hq, Hkv, Nq,
                             Nk, d, _dtype_code(q), ptr(cu_seqlens_q), ptr(cu_seqlens_k), mq, mk, int(window[0]),
                             int(window[1]), ptr(block_cnt), ptr(block_idx), bh, scale, stream)
    if st != FA_OK:
        _raise(st)
    return dq, dk, dv
