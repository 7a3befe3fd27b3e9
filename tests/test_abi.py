"""C ABI checks that need no GPU: the library loads, exports what include/fa.h
declares, and rejects invalid arguments on the host before any HIP call.

Every call below fails validation (or has nothing to compute), so nothing is
launched; the pointer values are never dereferenced.
"""
from __future__ import annotations

import ctypes
import math
import subprocess

import pytest
import torch

from exact_io_aware_fwd_amd import binding
from tests.bwd_plan import dense_plan as _dense_plan

OK, INV, UNS = binding.FA_OK, binding.FA_ERR_INVALID_ARGUMENT, binding.FA_ERR_UNSUPPORTED
P = 0x10000          # an aligned fake device address (never dereferenced here)


@pytest.fixture(scope="module")
def L():
    return binding.load()


def test_exports_every_declared_symbol(L):
    names = binding.declared_symbols()
    assert set(names) == {"fa_fwd", "fa_bwd", "fa_bwd_workspace_size", "fa_status_string", "fa_last_error",
                          "fa_fwd_splitkv", "fa_fwd_splitkv_workspace_size", "fa_fwd_splitkv_num_splits",
                          "fa_lse_combine", "fa_fp8_v_codes_bytes", "fa_fp8_quantize_rows", "fa_fp8_quantize_v",
                          "fa_fwd_fp8", "fa_fwd_masked", "fa_bwd_masked",
                          "fa_bwd_masked_workspace_size", "fa_bwd_noalloc"}
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in names:
        assert n in exported, n
        assert hasattr(L, n)


def test_no_undefined_kernel_stubs():
    """Every kernel launched by the library has its host-side stub compiled in."""
    out = subprocess.run(["nm", "-D", binding.LIB_PATH], capture_output=True, text=True).stdout
    undefined = [l for l in out.splitlines() if " U " in l and "__device_stub__" in l]
    assert not undefined, undefined


def test_status_strings(L):
    assert binding.status_string(OK) == "FA_OK"
    assert binding.status_string(INV) == "FA_ERR_INVALID_ARGUMENT"
    assert binding.status_string(UNS) == "FA_ERR_UNSUPPORTED"
    assert binding.status_string(binding.FA_ERR_HIP) == "FA_ERR_HIP"
    assert binding.status_string(99) == "FA_ERR_UNKNOWN"


def fwd(L, q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=1, N=16, d=64, dtype=1, causal=0, scale=0.125):
    return L.fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, dtype, causal, scale, None)


def bwd(L, ws_bytes=1 << 20, B=1, Hq=2, Hkv=1, N=16, d=64, dtype=1, scale=0.125, **ptrs):
    p = {n: P for n in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv", "ws")}
    p.update(ptrs)
    return L.fa_bwd(p["q"], p["k"], p["v"], p["o"], p["lse"], p["do"], p["dq"], p["dk"], p["dv"], p["ws"],
                    ws_bytes, B, Hq, Hkv, N, d, dtype, 0, scale, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INV), (dict(k=None), INV), (dict(v=None), INV), (dict(o=None), INV), (dict(lse=None), INV),
    (dict(q=P + 8), INV), (dict(lse=P + 4), INV),
    (dict(B=-1), INV), (dict(N=-5), INV), (dict(Hq=0), INV), (dict(Hkv=0), INV),
    (dict(Hq=3, Hkv=2), INV), (dict(d=0), INV),
    (dict(d=96), UNS), (dict(d=256), UNS), (dict(d=32), UNS), (dict(dtype=7), UNS),
    (dict(scale=0.0), INV), (dict(scale=-0.125), INV), (dict(scale=math.nan), INV), (dict(scale=math.inf), INV),
    (dict(N=1 << 40), INV), (dict(B=1 << 33), INV),
])
def test_fwd_rejects(L, kw, expect):
    assert fwd(L, **kw) == expect
    assert binding.last_error() != ""


@pytest.mark.parametrize("kw", [dict(B=0), dict(N=0), dict(B=0, q=None, k=None, v=None, o=None, lse=None)])
def test_fwd_empty_is_noop(L, kw):
    assert fwd(L, **kw) == OK


@pytest.mark.parametrize("kw,expect", [
    (dict(do=None), INV), (dict(dq=None), INV), (dict(dk=None), INV), (dict(dv=None), INV), (dict(ws=None), INV),
    (dict(ws=P + 2), INV), (dict(ws_bytes=0), INV), (dict(Hq=4, Hkv=3), INV), (dict(d=80), UNS),
    (dict(scale=math.nan), INV),
])
def test_bwd_rejects(L, kw, expect):
    assert bwd(L, **kw) == expect
    assert binding.last_error() != ""


def test_bwd_workspace_too_small(L):
    need = L.fa_bwd_workspace_size(1, 2, 1, 16, 64, 1, 0)
    assert need >= 2 * 16 * 8
    assert bwd(L, ws_bytes=need - 1) == INV
    assert "workspace" in binding.last_error()


def test_workspace_size_values(L):
    # two fp32 row terms (LSE*log2e, -D) per query row, rows padded to 32 per head; with few
    # key blocks, then the partial dK/dV slots of the split key blocks from a 256-byte boundary
    for B, Hq, Hkv, N, d in ((1, 16, 16, 4096, 128), (2, 32, 8, 8192, 128), (1, 1, 1, 1, 64), (3, 6, 2, 1000, 64),
                             (1, 8, 1, 1000, 128), (1, 32, 8, 1024, 64), (1, 4, 4, 70000, 128)):
        for causal in (0, 1):
            got = L.fa_bwd_workspace_size(B, Hq, Hkv, N, d, 1, causal)
            rt = B * Hq * ((N + 31) // 32) * 32 * 8
            kb, k = _dense_plan(B, Hq, Hkv, N, causal)
            want = rt if k == 1 else -(-rt // 256) * 256 + B * Hkv * -(-N // kb) * k * 2 * kb * d * 4
            assert got == want, (B, Hq, Hkv, N, d, causal, got, want)
    assert _dense_plan(2, 32, 8, 8192, 1) == (256, 1) and _dense_plan(1, 8, 1, 1000, 1) == (128, 8)
    assert _dense_plan(1, 16, 16, 4096, 1) == (128, 1) and _dense_plan(1, 32, 8, 8192, 1) == (256, 2)
    assert _dense_plan(1, 16, 16, 1024, 1) == (128, 1) and _dense_plan(1, 16, 16, 2048, 1) == (128, 2)
    assert L.fa_bwd_workspace_size(1, 3, 2, 16, 64, 1, 0) == 0
    assert L.fa_bwd_workspace_size(1, 2, 1, 16, 96, 1, 0) == 0


def test_python_binding_validates_before_the_abi():
    import torch
    q = torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding.fwd(q, q, q)          # CPU tensors are refused before any call
    with pytest.raises(TypeError):
        binding._dtype_code(torch.zeros(1, dtype=torch.float32))


def test_bwd_noalloc_validates_on_the_host(L):
    """fa_bwd_noalloc checks its arguments as fa_bwd does, and refuses sizes whose workspace
    would not fit its 64 MiB static scratch, before any HIP call (so no device is touched)."""
    def call(B=1, Hq=2, Hkv=1, N=16, d=64, dtype=1, causal=0, scale=0.125, **ptrs):
        p = {n: ptrs.get(n, P) for n in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv")}
        return L.fa_bwd_noalloc(p["q"], p["k"], p["v"], p["o"], p["lse"], p["do"], p["dq"], p["dk"], p["dv"],
                                B, Hq, Hkv, N, d, dtype, causal, scale, None)
    assert call(B=0) == OK and call(N=0) == OK
    assert call(q=0) == INV and "q is NULL" in binding.last_error()
    assert call(dv=P + 8) == INV
    assert call(d=96) == UNS
    assert call(Hq=3, Hkv=2) == INV
    assert call(scale=float("nan")) == INV
    # 8 bytes of row terms per query row: 2^23 rows plus padding exceed 64 MiB
    B, Hq, N = 4, 64, 32768 + 32
    assert L.fa_bwd_workspace_size(B, Hq, 8, N, 128, 1, 1) > binding.NOALLOC_SCRATCH_BYTES
    assert call(B=B, Hq=Hq, Hkv=8, N=N, d=128, causal=1) == INV
    assert "static scratch" in binding.last_error()


def test_masked_bindings_check_layouts_before_the_abi():
    """Both mask-family bindings parse the layout (packed [H, total, d] with cumulative
    lengths, or [B, H, N, d]) before anything reaches the library, and refuse a workspace
    that is not a GPU tensor."""
    import torch
    q4 = torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16)
    q3 = torch.zeros(2, 16, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 2, 16)
    cu = torch.tensor([0, 16], dtype=torch.int32)
    for args in ((q4, q4, q4), (q3, q3, q3)):
        packed = args[0].dim() == 4      # the wrong layout for the cumulative-length argument
        kw = {"cu_seqlens_q": cu, "cu_seqlens_k": cu} if packed else {}
        with pytest.raises(ValueError):
            binding.fwd_masked(*args, **kw)
        with pytest.raises(ValueError):
            binding.bwd_masked(*args, args[0], lse, args[0], **kw)
    with pytest.raises(ValueError):      # k and v of different shapes
        binding.bwd_masked(q4, q4, torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16), q4, lse, q4)
    with pytest.raises(ValueError):      # cumulative key lengths of the wrong count
        binding.fwd_masked(q3, q3, q3, cu_seqlens_q=cu, cu_seqlens_k=torch.tensor([0, 8, 16], dtype=torch.int32))
    with pytest.raises(ValueError):      # the device check every workspace goes through
        binding._check(torch.zeros(64, dtype=torch.uint8), "workspace", torch.device("cuda:0"))


def splitkv(L, ws_bytes=1 << 24, B=1, Hq=8, Hkv=2, Nq=1, Nk=100, d=128, dtype=1, causal=0, scale=0.125, S=0,
            **ptrs):
    p = {n: P for n in ("q", "k", "v", "o", "lse", "ws")}
    p.update(ptrs)
    return L.fa_fwd_splitkv(p["q"], p["k"], p["v"], p["o"], p["lse"], p["ws"], ws_bytes,
                            B, Hq, Hkv, Nq, Nk, d, dtype, causal, scale, S, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INV), (dict(ws=None), INV), (dict(o=P + 4), INV), (dict(Nk=-1), INV), (dict(Nq=-1), INV),
    (dict(Hq=3), INV), (dict(Nk=0), INV), (dict(causal=1, Nq=8, Nk=4), INV), (dict(S=-2), INV),
    (dict(d=96), UNS), (dict(dtype=5), UNS), (dict(scale=0.0), INV), (dict(ws_bytes=64), INV),
    (dict(Nk=1 << 31), INV),
])
def test_splitkv_rejects(L, kw, expect):
    assert splitkv(L, **kw) == expect
    assert binding.last_error() != ""


@pytest.mark.parametrize("kw", [dict(B=0), dict(Nq=0), dict(Nq=0, Nk=0, q=None, ws=None)])
def test_splitkv_empty_is_noop(L, kw):
    assert splitkv(L, **kw) == OK


def test_splitkv_plan():
    # default splits: about 1024 waves over (batch, K/V head, 32-row group); each split a
    # multiple of 32 keys; a workgroup merges 4 splits, so the workspace holds
    # rows x (splits padded to 4) / 4 x (d + 1) floats
    assert binding.splitkv_num_splits(1, 64, 8, 1, 65536, 128) == 128
    assert binding.splitkv_num_splits(2, 32, 8, 4, 8192, 128) == 64
    assert binding.splitkv_num_splits(1, 8, 2, 1, 40, 64) == 2      # at most one split per 32 keys
    ws = binding.splitkv_workspace_size(1, 64, 8, 1, 65536, 128, torch.bfloat16)
    assert ws == 64 * 32 * 128 * 4 + 64 * 32 * 4
    assert binding.splitkv_workspace_size(1, 8, 2, 1, 40, 64, torch.bfloat16, 3) == 8 * 1 * 64 * 4 + 256
    assert binding.splitkv_workspace_size(1, 8, 3, 1, 40, 64, torch.bfloat16) == 0
    # as many queries as keys (>= 128): key splits per query block, one by default (no
    # workspace: the forward writes O and LSE itself); per row and split the fp32 part of O
    # and its LSE
    for shape in ((1, 32, 8, 1024, 1024), (1, 16, 16, 1024, 1024), (1, 1, 1, 128, 128), (1, 4, 2, 4096, 4096)):
        for d in (64, 128):
            assert binding.splitkv_num_splits(*shape, d) == 1
    assert binding.splitkv_workspace_size(1, 32, 8, 1024, 1024, 128, torch.bfloat16) == 0
    rows = 16 * 1024
    assert binding.splitkv_workspace_size(1, 16, 16, 1024, 1024, 64, torch.bfloat16) == 0
    assert binding.splitkv_workspace_size(1, 16, 16, 1024, 1024, 64, torch.bfloat16, 2) == rows * 2 * (64 + 1) * 4
    rows = 32 * 1024
    # an explicit count: 5 splits of 16 tiles -> ceil(16/5) = 4 tiles each, 4 splits used
    ws5 = binding.splitkv_workspace_size(1, 32, 8, 1024, 1024, 128, torch.bfloat16, 5)
    assert ws5 == rows * 4 * 128 * 4 + rows * 4 * 4


@pytest.mark.parametrize("args,expect", [
    ((P, P, P, P, -1, 2, 128, 1), INV), ((P, P, P, P, 4, 0, 128, 1), INV), ((P, P, P, P, 4, 2, 80, 1), UNS),
    ((None, P, P, P, 4, 2, 128, 1), INV), ((P, P, P + 2, P, 4, 2, 128, 1), INV), ((P, P, P, P, 0, 2, 128, 1), OK),
])
def test_lse_combine_validation(L, args, expect):
    assert L.fa_lse_combine(*args, None) == expect


def quant_rows(L, x=P, signs=P, codes=P, scales=P, B=1, H=2, N=100, d=128, dtype=1, blk=64):
    return L.fa_fp8_quantize_rows(x, signs, codes, scales, B, H, N, d, dtype, blk, None)


def quant_v(L, x=P, codes=P, scales=P, B=1, H=2, N=100, d=128, dtype=1, blk=64):
    return L.fa_fp8_quantize_v(x, codes, scales, B, H, N, d, dtype, blk, None)


def fwd_fp8(L, B=1, Hq=2, Hkv=1, N=100, d=128, bq=64, bkv=64, causal=0, scale=0.125, **ptrs):
    p = {n: P for n in ("q", "k", "v", "qs", "ks", "vs", "o", "lse")}
    p.update(ptrs)
    return L.fa_fwd_fp8(p["q"], p["k"], p["v"], p["qs"], p["ks"], p["vs"], p["o"], p["lse"], B, Hq, Hkv, N, d,
                        bq, bkv, causal, scale, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(x=None), INV), (dict(codes=P + 8), INV), (dict(scales=P + 2), INV), (dict(blk=32), INV),
    (dict(blk=96), INV), (dict(d=96), UNS), (dict(dtype=7), UNS), (dict(H=0), INV), (dict(N=-1), INV),
    (dict(N=1 << 31), INV),
])
def test_fp8_quantize_rejects(L, kw, expect):
    assert quant_rows(L, **kw) == expect
    assert binding.last_error() != ""
    kw.pop("signs", None)
    assert quant_v(L, **kw) == expect


def test_fp8_quantize_signs_optional_and_empty(L):
    # a NULL sign vector means no transform (it is not an error); empty inputs are no-ops
    assert quant_rows(L, N=0, signs=None) == OK
    assert quant_rows(L, B=0) == OK and quant_v(L, B=0) == OK
    assert quant_rows(L, signs=P + 2) == INV      # present but misaligned


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INV), (dict(vs=None), INV), (dict(o=P + 4), INV), (dict(bq=32), INV), (dict(bkv=512), INV),
    (dict(Hq=3, Hkv=2), INV), (dict(d=256), UNS), (dict(scale=-1.0), INV), (dict(N=-5), INV),
])
def test_fwd_fp8_rejects(L, kw, expect):
    assert fwd_fp8(L, **kw) == expect
    assert binding.last_error() != ""


def test_fwd_fp8_empty_and_sizes(L):
    assert fwd_fp8(L, N=0, q=None) == OK and fwd_fp8(L, B=0) == OK
    # value tiles: 64 keys x d bytes per tile, tiles rounded up
    assert L.fa_fp8_v_codes_bytes(2, 3, 100, 128) == 2 * 3 * 2 * 128 * 64
    assert L.fa_fp8_v_codes_bytes(1, 1, 64, 64) == 64 * 64
    assert L.fa_fp8_v_codes_bytes(1, 1, 0, 64) == 0


def masked(L, B=1, Hq=2, Hkv=1, Nq=100, Nk=120, d=128, dtype=1, cq=None, ck=None, mq=0, mk=0, wl=-1, wr=-1,
           bcnt=None, bidx=None, bh=1, scale=0.125, **ptrs):
    p = {n: P for n in ("q", "k", "v", "o", "lse")}
    p.update(ptrs)
    return L.fa_fwd_masked(p["q"], p["k"], p["v"], p["o"], p["lse"], B, Hq, Hkv, Nq, Nk, d, dtype, cq, ck, mq, mk,
                           wl, wr, bcnt, bidx, bh, scale, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INV), (dict(lse=P + 4), INV), (dict(Nk=-1), INV), (dict(Hq=3, Hkv=2), INV), (dict(d=80), UNS),
    (dict(cq=P), INV),                                      # one cu array without the other
    (dict(cq=P, ck=P, mq=101, mk=10), INV),                 # max length beyond the tensor rows
    (dict(cq=P + 2, ck=P, mq=10, mk=10), INV),              # misaligned
    (dict(wl=-2), INV), (dict(wr=-5), INV), (dict(bcnt=P), INV), (dict(bcnt=P, bidx=P, bh=3), INV),
    (dict(scale=float("nan")), INV),
])
def test_fwd_masked_rejects(L, kw, expect):
    assert masked(L, **kw) == expect
    assert binding.last_error() != ""


def test_fwd_masked_empty(L):
    assert masked(L, B=0) == OK and masked(L, Nq=0) == OK
    assert masked(L, cq=P, ck=P, mq=0, mk=5) == OK        # every sequence empty


def bwd_masked(L, ws_bytes=1 << 20, B=1, Hq=2, Hkv=1, Nq=100, Nk=120, d=128, dtype=1, cq=None, ck=None, mq=0, mk=0,
               wl=-1, wr=-1, bcnt=None, bidx=None, bh=1, scale=0.125, **ptrs):
    p = {n: P for n in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv", "ws")}
    p.update(ptrs)
    return L.fa_bwd_masked(p["q"], p["k"], p["v"], p["o"], p["lse"], p["do"], p["dq"], p["dk"], p["dv"], p["ws"],
                           ws_bytes, B, Hq, Hkv, Nq, Nk, d, dtype, cq, ck, mq, mk, wl, wr, bcnt, bidx, bh, scale, None)


# row terms of B=1, Hq=2, 100 queries: 2 heads x 4 blocks of 32 rows x 256 bytes
_RT = 2 * 4 * 256


@pytest.mark.parametrize("kw,expect", [
    (dict(dq=None), INV), (dict(ws=None), INV), (dict(ws_bytes=64), INV), (dict(cq=P), INV), (dict(wl=-3), INV),
    (dict(cq=P, ck=P, mq=500, mk=10), INV), (dict(d=96), UNS), (dict(Hq=3, Hkv=2), INV), (dict(scale=0.0), INV),
    (dict(bcnt=P), INV), (dict(bcnt=P, bidx=P, bh=3), INV), (dict(bcnt=P + 2, bidx=P), INV),
    (dict(bcnt=P, bidx=P, ws_bytes=_RT), INV),
])
def test_bwd_masked_rejects(L, kw, expect):
    assert bwd_masked(L, **kw) == expect
    assert binding.last_error() != ""


def test_bwd_masked_workspace_and_empty(L):
    # row terms per (sequence, head), padded to 32-row blocks: 256 bytes per block
    assert L.fa_bwd_masked_workspace_size(3, 4, 2, 100, 300, 0) == 3 * 4 * 4 * 256
    # with block lists: per (sequence, K/V head, 128-key block) a record of 2 + 3 * (Hq/Hkv) *
    # ceil(maxq/256) ints and a plan of 2 ints, a slot table of 1 + 2 * 512 ints, and 512 slots
    # of 2 x 128 x 128 floats; each region rounded up to 256 bytes
    up = lambda x: -(-x // 256) * 256
    nrec = 3 * 2 * 3
    assert L.fa_bwd_masked_workspace_size(3, 4, 2, 100, 300, 1) == \
        3 * 4 * 4 * 256 + up(nrec * (2 + 3 * 2 * 1) * 4) + up(nrec * 8) + up((1 + 2 * 512) * 4) + 512 * 2 * 128 * 128 * 4
    assert L.fa_bwd_masked_workspace_size(3, 4, 3, 100, 300, 1) == 0
    assert bwd_masked(L, B=0) == OK and bwd_masked(L, Nq=0) == OK
