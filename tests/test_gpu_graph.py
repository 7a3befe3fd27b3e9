"""The forward and backward captured in one HIP graph (torch.cuda.CUDAGraph on the
capture stream): the library allocates nothing and clears nothing with memsets, so its
launches record as plain kernel nodes.  Each case replays the graph several times; before
every replay the captured inputs are rewritten in place and the same calls run eagerly
(with synchronisations between), and every replay must equal the eager result bit for
bit: O, LSE, dQ, dK, dV.  The shapes cover the dK/dV pass with 64 and with 32 keys a
wave, unsplit and split with its reduction, and head size 64 in fp16.
"""
from __future__ import annotations

import pytest
import torch

import workloads
from tests.gpu_util import say
import exact_io_aware_fwd_amd as fa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,Hq,Hkv,N,d,dt,causal", [
    (4, 16, 16, 2100, 128, torch.bfloat16, True),   # 64 keys a wave, unsplit
    (1, 32, 8, 8192, 128, torch.bfloat16, True),    # 64 keys a wave, key blocks split in two + reduction
    (1, 16, 16, 2048, 128, torch.bfloat16, True),   # 32 keys a wave, split in two + reduction
    (1, 8, 2, 700, 64, torch.float16, False),       # d = 64, ragged tail
])
def test_fwd_bwd_graph_replays_equal_eager(B, Hq, Hkv, N, d, dt, causal):
    dev = torch.device("cuda:0")
    say(f"[graph] fwd+bwd captured: B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} {dt} causal={causal}")
    shapes = ((B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d), (B, Hq, N, d))
    q, k, v, do = (workloads.randn(700 + i, s, dt).to(dev) for i, s in enumerate(shapes))
    ws = torch.empty(max(fa.bwd_workspace_size(B, Hq, Hkv, N, d, dt, causal), 16), dtype=torch.uint8, device=dev)

    def step():
        o, lse = fa.fwd(q, k, v, causal=causal)
        return (o, lse) + fa.bwd(q, k, v, o, lse, do, causal=causal, workspace=ws)

    side = torch.cuda.Stream(dev)   # warm-up off the default stream, as capture requires
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = step()
    torch.cuda.synchronize()

    for r in range(3):
        for i, t in enumerate((q, k, v, do)):
            t.copy_(workloads.randn(800 + 10 * r + i, tuple(t.shape), dt).to(dev))
        torch.cuda.synchronize()
        eager = [t.clone() for t in step()]
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, x, y in zip(("O", "LSE", "dQ", "dK", "dV"), captured, eager):
            assert torch.equal(x, y), f"replay {r}: {name} differs from the eager call"
    del g


@pytest.mark.parametrize("name", ["mix_small_d64_bf16", "bsparse_b1_hq16_hkv4_n8192_d128_bf16"])
def test_masked_fwd_bwd_graph_replays_equal_eager(name):
    """The same for the mask family with block lists (packed sequences with a two-sided
    window; the N = 8192 block-sparse workload, whose long key blocks the dK/dV pass
    splits): the kernels that build the transposed lists and the chunk plan rewrite
    their workspace on every call, so no replay depends on what the previous one left."""
    dev = torch.device("cuda:0")
    w = workloads.MASK_WORKLOADS[name]
    say(f"[graph] masked fwd+bwd captured: {w.name}")
    q, k, v, cq, ck, lists = workloads.make_mask_inputs(w)
    q, k, v = (t.to(dev) for t in (q, k, v))
    do = workloads.randn(w.seeds[0] + 50, tuple(q.shape), q.dtype).to(dev)
    if w.packed:
        mq, mk = max(w.seqlens_q), max(w.seqlens_k)
        cqd, ckd = torch.from_numpy(cq).to(dev), torch.from_numpy(ck).to(dev)
    else:
        mq, mk, cqd, ckd = w.seqlens_q[0], w.seqlens_k[0], None, None
    bc, bi = fa.block_lists_to_tensors(lists, mq, mk, dev)
    ws = torch.empty(fa.binding.load().fa_bwd_masked_workspace_size(w.B, w.Hq, w.Hkv, mq, mk, 1),
                     dtype=torch.uint8, device=dev)

    def step():
        o, lse = fa.fwd_masked(q, k, v, w.window, w.scale, cqd, ckd, mq, mk, bc, bi)
        return (o, lse) + fa.bwd_masked(q, k, v, o, lse, do, w.window, w.scale, cqd, ckd, mq, mk, bc, bi,
                                        workspace=ws)

    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = step()
    torch.cuda.synchronize()

    for r in range(3):
        for i, t in enumerate((q, k, v, do)):
            t.copy_(workloads.randn(900 + 10 * r + i, tuple(t.shape), t.dtype).to(dev))
        torch.cuda.synchronize()
        eager = [t.clone() for t in step()]
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for nm, x, y in zip(("O", "LSE", "dQ", "dK", "dV"), captured, eager):
            assert torch.equal(x, y), f"replay {r}: {nm} differs from the eager call"
    del g
