"""Throughput of the attention hot path on one MI355X: fa_fwd + fa_bwd per step.

Workload: the grouped-query long-context case, B=2, Hq=32, Hkv=8, N=8192,
d=128, bf16, causal (the configuration the metric is quoted on).  A step is one
forward pass (O and LSE) followed by one backward pass (dQ, dK, dV) over one
batch of seeded synthetic inputs already resident in HBM.

Prints ONE JSON line.  `value` is fwd+bwd TFLOP/s with the algorithmic FLOP
count (forward 4*B*Hq*N^2*d, backward 10*B*Hq*N^2*d, both halved for causal).
`roofline` describes the kernel that takes most of the step; per-pass figures
are under `passes`.  `cpu_baseline` times the fp64 oracle on a bounded sample
of the same workload on the host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--fwd-only]
    python bench.py --decode [--steps K] ...    # split-KV decoding: GB/s against the HBM peak
    python bench.py --fp8 [--steps K] ...       # FP8 forward (quantise + attention): TFLOP/s
    python bench.py --masks [--steps K] ...     # mask-family forward (sliding window; varlen, block-sparse)
    python bench.py --sweep                     # fa_fwd / fa_bwd TFLOP/s over 128 shapes (markdown table)

Profiling helpers (rocprofv3 runs of this same script):
    python bench.py --copy-calibration          # a plain 1 GiB device copy, for HBM counters
    python bench.py --summarize DIR [--pmc]     # rocprofv3 CSV -> markdown summary on stdout
    python bench.py --record-traffic DIR ...    # FETCH/WRITE per dispatch -> profiles/traffic.json

`roofline.traffic` is filled from profiles/traffic.json only while the kernel sources
hash to the value recorded with the counters; otherwise it is null.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--fwd-only", action="store_true", help="time only the forward pass (profiling)")
    p.add_argument("--cpu-heads", type=int, default=12, help="query heads in the CPU-baseline sample")
    p.add_argument("--copy-calibration", action="store_true", help="run a plain 1 GiB device copy and exit")
    p.add_argument("--gemm-calibration", action="store_true",
                   help="time a plain bf16 8192^3 GEMM (vendor BLAS) and exit")
    p.add_argument("--summarize", metavar="DIR", help="summarize rocprofv3 CSV output under DIR and exit")
    p.add_argument("--pmc", action="store_true", help="with --summarize: counter CSVs instead of kernel trace")
    p.add_argument("--record-traffic", nargs=3, metavar=("KERNEL_DIR", "COPY_DIR", "KERNEL_SUBSTR"),
                   help="write profiles/traffic.json from FETCH_SIZE/WRITE_SIZE runs and exit "
                        "(SUBSTR may list alternatives separated by '|')")
    p.add_argument("--decode", action="store_true",
                   help="time the split-KV decoding forward instead (one JSON line, GB/s)")
    p.add_argument("--masks", action="store_true",
                   help="time the mask-family forward (sliding window headline; varlen and block-sparse alongside)")
    p.add_argument("--headline-only", action="store_true",
                   help="with --masks: skip the workloads timed alongside (profiling runs)")
    p.add_argument("--fp8", action="store_true",
                   help="time the FP8 forward (block quantisation with the Hadamard transform + attention)")
    p.add_argument("--sweep", action="store_true",
                   help="fa_fwd and fa_bwd TFLOP/s over a grid of shapes (bf16; markdown table) and exit")
    return p.parse_args()


# Sources whose text decides what a pass launches: its kernels, the shared device headers,
# and the host side that picks launch shapes and plans (fa_api.cpp, fa_internal.h).
_SHARED_SOURCES = ["exact_io_aware_fwd_amd/csrc/fa_device.h", "exact_io_aware_fwd_amd/csrc/fa_tiles.h",
                   "exact_io_aware_fwd_amd/csrc/fa_internal.h", "exact_io_aware_fwd_amd/csrc/fa_api.cpp"]
KERNEL_SOURCES = {
    "fwd": ["exact_io_aware_fwd_amd/csrc/fa_fwd.hip"] + _SHARED_SOURCES,
    "bwd": ["exact_io_aware_fwd_amd/csrc/fa_bwd.hip"] + _SHARED_SOURCES,
    "decode": ["exact_io_aware_fwd_amd/csrc/fa_decode.hip"] + _SHARED_SOURCES,
    "masks": ["exact_io_aware_fwd_amd/csrc/fa_fwd.hip"] + _SHARED_SOURCES,
    "fp8": ["exact_io_aware_fwd_amd/csrc/fa_fwd_fp8.hip", "exact_io_aware_fwd_amd/csrc/fa_fp8_quant.hip"]
           + _SHARED_SOURCES,
}
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
COPY_BYTES = 1 << 30


def warm_up(step, min_steps: int, min_seconds: float = 0.3) -> int:
    """Run `step` at least min_steps times and for at least min_seconds of GPU time (the
    clocks of an idle GPU take a while to ramp); returns the number of calls made."""
    import torch
    n, t0 = 0, time.perf_counter()
    while n < min_steps or time.perf_counter() - t0 < min_seconds:
        step()
        n += 1
        if n % 8 == 0 or n >= min_steps:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def copy_calibration():
    """A plain device-to-device copy of exactly 1 GiB, five times (for counter scaling)."""
    import torch
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "repeats": 5}))


def gemm_calibration():
    """A plain bf16 GEMM through torch (the vendor BLAS), 8192 x 8192 x 8192, timed with HIP
    events after 1 s of warm-up: the matrix-core rate a library product reaches on this part
    under the same power and clock limits as the attention kernels."""
    import torch
    from exact_io_aware_fwd_amd import metrics
    n = 8192
    g = torch.Generator(device="cuda:0").manual_seed(0)
    a = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16, generator=g)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 1.0:
        c = a @ b
        torch.cuda.synchronize()
    reps = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tf = 2 * n ** 3 / ms / 1e9
    print(json.dumps({"gemm": f"bf16 {n}x{n}x{n}", "ms": ms, "tflops": tf, "frac_of_peak": tf / metrics.MFMA_BF16_TFLOPS}))
    del c


def _read_csv(pattern):
    rows = []
    for f in sorted(glob.glob(pattern, recursive=True)):
        rows.extend(csv.DictReader(open(f)))
    return rows


def pmc_per_dispatch(directory):
    """{kernel name: {counter: mean value per dispatch}} from rocprofv3 --pmc CSV output."""
    tot = defaultdict(lambda: defaultdict(float))
    disp = defaultdict(set)
    for r in _read_csv(os.path.join(directory, "**", "*counter_collection.csv")):
        k = r["Kernel_Name"]
        tot[k][r["Counter_Name"]] += float(r["Counter_Value"])
        disp[(k, r["Counter_Name"])].add(r["Dispatch_Id"])
    return {k: {c: v / len(disp[(k, c)]) for c, v in cs.items()} for k, cs in tot.items()}


def summarize(directory, pmc):
    if pmc:
        for k, cs in pmc_per_dispatch(directory).items():
            print(f"### `{k}`\n\n| counter | per dispatch |\n|---|---|")
            for c, v in sorted(cs.items()):
                print(f"| {c} | {v:.6g} |")
            print()
        return
    rows = _read_csv(os.path.join(directory, "**", "*kernel_stats.csv"))
    print("| kernel | calls | total ns | average ns | min ns | max ns | % |\n|---|---|---|---|---|---|---|")
    for r in rows:
        print(f"| `{r['Name']}` | {r['Calls']} | {r['TotalDurationNs']} | {float(r['AverageNs']):.0f} | "
              f"{r['MinNs']} | {r['MaxNs']} | {float(r['Percentage']):.2f} |")


def traffic_kind(substr: str) -> str:
    """Which bench line a recorded kernel name (or '|'-separated names) belongs to."""
    # the mask family runs fwd_unit_kernel with its general mode on (fifth template argument)
    targs = substr[substr.find("<") + 1:substr.rfind(">")].split(", ") if "fwd_unit_kernel<" in substr else []
    return ("decode" if ("splitkv" in substr or "combine" in substr) else "fp8" if "fp8" in substr
            else "masks" if len(targs) >= 5 and targs[4] == "true" else "bwd" if "bwd" in substr else "fwd")


def record_traffic(kdir, cdir, substr):
    # every kernel whose name contains substr runs once per call of the pass: sum them
    alts = substr.split("|")
    kern = {k: v for k, v in pmc_per_dispatch(kdir).items() if any(a in k for a in alts)}
    copy = {k: v for k, v in pmc_per_dispatch(cdir).items() if "copy" in k.lower()}
    if not kern or not copy:
        raise SystemExit(f"expected kernels matching {substr!r} and a copy kernel; got {list(kern)}, {list(copy)}")
    kname = " + ".join(sorted(kern))
    kc = {c: sum(v.get(c, 0.0) for v in kern.values()) for c in ("FETCH_SIZE", "WRITE_SIZE")}
    cc = max(copy.values(), key=lambda c: c.get("FETCH_SIZE", 0) + c.get("WRITE_SIZE", 0))
    kib = COPY_BYTES / 1024
    fetch_factor = kib / cc["FETCH_SIZE"] if cc.get("FETCH_SIZE") else None
    write_factor = kib / cc["WRITE_SIZE"] if cc.get("WRITE_SIZE") else None
    kind = traffic_kind(substr)
    data = json.load(open(TRAFFIC_JSON)) if os.path.exists(TRAFFIC_JSON) else {}
    data[kind] = {"kernel": kname, "source_hash": source_hash(kind),
                  "fetch_kib": kc.get("FETCH_SIZE"), "write_kib": kc.get("WRITE_SIZE"),
                  "copy_fetch_factor": fetch_factor, "copy_write_factor": write_factor}
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    json.dump(data, open(TRAFFIC_JSON, "w"), indent=1)
    print(json.dumps(data[kind]))


def traffic_bytes(kind: str):
    """Per-launch HBM bytes from the recorded counters, if they match the current sources."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    rec = json.load(open(TRAFFIC_JSON)).get(kind)
    if not rec or rec.get("source_hash") != source_hash(kind):
        return None
    if None in (rec.get("fetch_kib"), rec.get("write_kib"), rec.get("copy_fetch_factor"), rec.get("copy_write_factor")):
        return None
    return 1024.0 * (rec["fetch_kib"] * rec["copy_fetch_factor"] + rec["write_kib"] * rec["copy_write_factor"])


def cpu_baseline(w, inputs, heads: int, fwd_only: bool, gpu_out=None):
    """The fp64 oracle on whole K/V groups of the workload: `heads` query heads of batch 0,
    all N rows, timed.  With `gpu_out` (o, lse[, dq, dk, dv] of the same inputs, CPU
    tensors), the oracle's results on that sample are also compared with the GPU's, at the
    parity tests' metrics: O max error / max|O_ref|, LSE max abs error, rel-L2 of dQ, dK, dV."""
    import numpy as np
    import oracle
    from exact_io_aware_fwd_amd import metrics
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    q, k, v, do = inputs
    G = w.Hq // w.Hkv
    heads = max(G, min(heads, w.Hq) // G * G)        # whole K/V groups of batch 0
    qs, ks, vs, dos = q[:1, :heads], k[:1, :heads // G], v[:1, :heads // G], do[:1, :heads]
    causal = True in w.causal
    t0 = time.perf_counter()
    O_ref, L_ref = oracle.attention_fwd(qs, ks, vs, causal, w.scale)
    flops = metrics.fwd_flops(1, heads, w.N, w.d, causal)
    grads = None
    if not fwd_only:
        grads = oracle.attention_bwd(qs, ks, vs, dos, causal, w.scale)
        flops += metrics.bwd_flops(1, heads, w.N, w.d, causal)
    dt = time.perf_counter() - t0
    rec = {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"batch 0, query heads 0-{heads - 1} with their K/V heads, all {w.N} rows, "
                  f"{'forward' if fwd_only else 'forward + backward'} in numpy float64 "
                  f"(materialising, full N^2 even when causal; credited the same algorithmic FLOPs); "
                  f"{dt:.1f} s",
        "seconds": dt,
    }
    if gpu_out is not None:
        def f64(t):
            return t.double().numpy()
        o, lse = f64(gpu_out[0][:1, :heads]), f64(gpu_out[1][:1, :heads])
        par = {"sample": f"batch 0, query heads 0-{heads - 1}",
               "o_max_rel": float(np.max(np.abs(o - O_ref)) / np.max(np.abs(O_ref))),
               "lse_max_abs": float(np.max(np.abs(lse - L_ref)))}
        if grads is not None and len(gpu_out) == 5:
            for name, x, r in zip(("dq", "dk", "dv"), (gpu_out[2][:1, :heads], gpu_out[3][:1, :heads // G],
                                                      gpu_out[4][:1, :heads // G]), grads):
                par[f"{name}_rel_l2"] = float(np.linalg.norm((f64(x) - r).ravel()) / np.linalg.norm(r.ravel()))
        tol = {"o_max_rel": 1.5e-2 if w.dtype == "bf16" else 2e-3, "lse_max_abs": 1e-4,
               "dq_rel_l2": 1e-2, "dk_rel_l2": 1e-2, "dv_rel_l2": 1e-2}
        par["within_tolerance"] = all(par[n] <= t for n, t in tol.items() if n in par)
        rec["parity"] = par
    return rec


def bench_decode(args):
    """Split-KV decoding on the long-cache decode workload: one JSON line in GB/s."""
    import torch
    import workloads
    import exact_io_aware_fwd_amd as fa
    from exact_io_aware_fwd_amd import metrics

    w = workloads.DECODE_WORKLOADS[args.workload or workloads.DECODE_HEADLINE]
    causal = True in w.causal
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cpu_inputs = workloads.make_decode_inputs(w)
    q, k, v = (t.to(dev) for t in cpu_inputs)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.binding.splitkv_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, q.dtype), dtype=torch.uint8,
                     device=dev)

    def step():
        fa.binding.fwd_splitkv(q, k, v, causal=causal, softmax_scale=w.scale, workspace=ws, out=o, lse=lse)

    nwarm = warm_up(step, max(args.warmup, 5))
    steps = max(args.steps, 50)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    nbytes = metrics.decode_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, q.element_size())
    gbps = nbytes / (ms * 1e-3) / 1e9
    rec = {
        "metric": "split-KV decoding attention: HBM GB/s and % of peak",
        "value": gbps, "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": nwarm,
        "ms_per_step": wall * 1e3 / steps, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {torch.bfloat16: "bf16", torch.float16: "fp16"}[q.dtype], "data": "synthetic (seeded iid N(0,1))",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": causal, "step": "fa_fwd_splitkv",
                   "num_splits": fa.binding.splitkv_num_splits(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d)},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": metrics.HBM_GBPS, "unit": "GB/s",
                     "frac": gbps / metrics.HBM_GBPS, "traffic": traffic_bytes("decode"),
                     "kernel": "splitkv_kernel + lse_combine_kernel", "avg_ms": ms, "algorithmic_bytes": nbytes},
    }
    if not args.no_cpu_baseline:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:  # pragma: no cover
            threads = len(os.sched_getaffinity(0))
        qs, ks, vs = cpu_inputs
        G = w.Hq // w.Hkv
        tc = time.perf_counter()
        reps = 0
        while time.perf_counter() - tc < 10.0:
            oracle.attention_fwd_kv(qs[:1, :G], ks[:1, :1], vs[:1, :1], causal, w.scale)
            reps += 1
        dt = time.perf_counter() - tc
        sb = metrics.decode_bytes(1, G, 1, w.Nq, w.Nk, w.d, q.element_size()) * reps
        rec["cpu_baseline"] = {"value": sb / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
                               "sample": f"batch 0, K/V head 0 with its {G} query heads, all {w.Nk} keys, "
                                         f"numpy float64, repeated {reps} times in {dt:.1f} s; "
                                         f"credited the same algorithmic bytes"}
    print(json.dumps(rec), flush=True)


def bench_fp8(args):
    """FP8 forward on the grouped-query N=8192 shape: one JSON line in TFLOP/s.

    A step quantises Q and K (random-sign Hadamard transform, per-block scales) and V,
    then runs the FP8 attention forward; `value` credits the forward's algorithmic FLOPs
    to the whole step.  The roofline line is the attention kernel against the dense
    FP8 matrix-core peak."""
    import torch
    import workloads
    import exact_io_aware_fwd_amd as fa
    from exact_io_aware_fwd_amd import metrics

    w = workloads.FP8_WORKLOADS[args.workload or workloads.FP8_HEADLINE]
    causal = True in w.causal
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cpu_inputs = workloads.make_fp8_inputs(w)
    q, k, v = (t.to(dev) for t in cpu_inputs[:3])
    signs = torch.from_numpy(cpu_inputs[3]).to(dev)
    o = torch.empty((w.B, w.Hq, w.N, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    ops = [None]

    def quantise():
        ops[0] = fa.fp8_prepare(q, k, v, signs, w.block_q, w.block_kv)

    def attend():
        fa.fwd_fp8(*ops[0], causal=causal, softmax_scale=w.scale, block_q=w.block_q, block_kv=w.block_kv,
                   out=o, lse=lse)

    nwarm = warm_up(lambda: (quantise(), attend()), max(args.warmup, 3))
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        quantise()
        ev[i][1].record(stream)
        attend()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    q_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    a_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    flops = metrics.fwd_flops(w.B, w.Hq, w.N, w.d, causal)
    step_ms = q_ms + a_ms
    value = flops / (step_ms * 1e-3) / 1e12
    achieved = flops / (a_ms * 1e-3) / 1e12
    qbytes = metrics.fp8_quant_bytes(w.B, w.Hq, w.Hkv, w.N, w.d, 2, w.block_q, w.block_kv)
    rec = {
        "metric": "FP8 attention forward TFLOPS and % of the FP8 matrix-core peak at N=8192 d=128 causal",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": nwarm,
        "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8 e4m3 operands, fp32 accumulation, bf16 output",
        "data": "synthetic (seeded N(0,1), 0.1% of entries x16; random signs)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d, "causal": causal,
                   "block_q": w.block_q, "block_kv": w.block_kv,
                   "step": "fa_fp8_quantize_rows (Q, K) + fa_fp8_quantize_v + fa_fwd_fp8"},
        "passes": {"quantise_ms": q_ms, "quantise_GBps": qbytes / (q_ms * 1e-3) / 1e9,
                   "attention_ms": a_ms, "attention_TFLOPs": achieved},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": metrics.MFMA_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / metrics.MFMA_FP8_TFLOPS, "traffic": traffic_bytes("fp8"),
                     "kernel": "fwd_fp8_kernel", "avg_ms": a_ms, "algorithmic_flops": flops},
    }
    if not args.no_cpu_baseline:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:  # pragma: no cover
            threads = len(os.sched_getaffinity(0))
        qc, kc, vc, sc = cpu_inputs
        G = w.Hq // w.Hkv
        heads = max(G, min(args.cpu_heads, w.Hq) // G * G)
        t1 = time.perf_counter()
        oracle.attention_fwd_fp8(qc[:1, :heads], kc[:1, :heads // G], vc[:1, :heads // G], sc, causal, w.scale,
                                 w.block_q, w.block_kv)
        dt = time.perf_counter() - t1
        sflops = metrics.fwd_flops(1, heads, w.N, w.d, causal)
        rec["cpu_baseline"] = {"value": sflops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                               "sample": f"batch 0, query heads 0-{heads - 1} with their K/V heads, all {w.N} rows: "
                                         f"quantisation and float64 attention of the dequantised operands "
                                         f"(full N^2 even when causal; credited the same algorithmic FLOPs); "
                                         f"{dt:.1f} s"}
    print(json.dumps(rec), flush=True)


def bench_masks(args):
    """Mask-family forward: one JSON line for the N=8192 sliding-window workload in
    TFLOP/s over the visible (query, key) pairs; its backward, and the forward and
    backward of the packed variable-length and the block-sparse workloads, are timed
    alongside (under `passes`)."""
    import numpy as np
    import torch
    import workloads
    import oracle.masks as om
    import exact_io_aware_fwd_amd as fa
    from exact_io_aware_fwd_amd import metrics

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    def prepare(w):
        q, k, v, cq, ck, lists = workloads.make_mask_inputs(w)
        qd, kd, vd = (t.to(dev) for t in (q, k, v))
        if w.packed:
            mq, mk = max(w.seqlens_q), max(w.seqlens_k)
            cqd, ckd = torch.from_numpy(cq).to(dev), torch.from_numpy(ck).to(dev)
        else:
            mq, mk, cqd, ckd = w.seqlens_q[0], w.seqlens_k[0], None, None
        bc, bi = fa.block_lists_to_tensors(lists, mq, mk, dev) if lists is not None else (None, None)
        o, lse = torch.empty_like(qd), torch.empty(qd.shape[:-1], dtype=torch.float32, device=dev)
        run = lambda: fa.fwd_masked(qd, kd, vd, w.window, w.scale, cqd, ckd, mq, mk, bc, bi, out=o, lse=lse)
        pairs = sum(om.visible_pairs([lq], [lk], w.window, None if lists is None else [lists[b][0]])
                    for b, (lq, lk) in enumerate(zip(w.seqlens_q, w.seqlens_k)))
        flops = 4.0 * w.d * w.Hq * pairs

        def backward():
            """The backward of the same problem (dO seeded), its workspace allocated once."""
            run()
            do = workloads.randn(w.seeds[0] + 50, tuple(qd.shape), qd.dtype).to(dev)
            ws = torch.empty(fa.binding.load().fa_bwd_masked_workspace_size(w.B, w.Hq, w.Hkv, mq, mk, int(bi is not None)),
                             dtype=torch.uint8, device=dev)
            return lambda: fa.bwd_masked(qd, kd, vd, o, lse, do, w.window, w.scale, cqd, ckd, mq, mk, bc, bi,
                                         workspace=ws)

        return run, flops, (q, k, v, cq, ck, lists), backward

    nwarms = []

    def timed(run, steps):
        nwarms.append(warm_up(run, max(args.warmup, 3)))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps, (time.perf_counter() - t0) * 1e3 / steps

    w = workloads.MASK_WORKLOADS[args.workload or workloads.MASK_HEADLINE]
    run, flops, cpu_inputs, backward = prepare(w)
    ms, wall_ms = timed(run, args.steps)
    achieved = flops / (ms * 1e-3) / 1e12
    passes = {}

    def time_backward(name, backward, f):
        # five products per visible pair against the forward's two
        mb, _ = timed(backward(), args.steps)
        passes[name + " backward"] = {"ms": mb, "TFLOPs": 2.5 * f / (mb * 1e-3) / 1e12, "visible_pair_flops": 2.5 * f}

    if not args.headline_only:
        time_backward(w.name, backward, flops)
    for name in workloads.MASK_WORKLOADS:
        if name == w.name or name.startswith("mix_") or args.headline_only:
            continue
        r2, f2, _, b2 = prepare(workloads.MASK_WORKLOADS[name])
        m2, _ = timed(r2, args.steps)
        passes[name] = {"ms": m2, "TFLOPs": f2 / (m2 * 1e-3) / 1e12, "visible_pair_flops": f2}
        time_backward(name, b2, f2)
    rec = {
        "metric": "mask-family attention forward TFLOPS (visible pairs) and % of the MFMA peak, sliding window at N=8192 d=128",
        "value": achieved, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": nwarms[0],
        "ms_per_step": wall_ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded iid N(0,1))",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.seqlens_q[0], "Nk": w.seqlens_k[0],
                   "d": w.d, "window": list(w.window), "step": "fa_fwd_masked",
                   "flops": "4 d x visible (query, key) pairs x heads"},
        "passes": passes,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": metrics.MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / metrics.MFMA_BF16_TFLOPS, "traffic": traffic_bytes("masks"),
                     "kernel": "fwd_unit_kernel<bf16, 128, false, 12, true, 1>", "avg_ms": ms, "algorithmic_flops": flops},
    }
    if not args.no_cpu_baseline:
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:  # pragma: no cover
            threads = len(os.sched_getaffinity(0))
        q, k, v, cq, ck, lists = cpu_inputs
        G = w.Hq // w.Hkv
        heads = max(G, min(args.cpu_heads, w.Hq) // G * G)
        t1 = time.perf_counter()
        om.attention_fwd_masked(q[:1, :heads], k[:1, :heads // G], v[:1, :heads // G], w.scale, window=w.window)
        dt = time.perf_counter() - t1
        sflops = flops / (w.B * w.Hq) * heads
        rec["cpu_baseline"] = {"value": sflops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                               "sample": f"batch 0, query heads 0-{heads - 1} with their K/V heads, all rows, "
                                         f"numpy float64 (materialising the full N x N scores and masking them; "
                                         f"credited the visible-pair FLOPs); {dt:.1f} s"}
    print(json.dumps(rec), flush=True)


def _fwd_kernel(B, Hq, N, d, causal):
    """The forward kernel fa_fwd launches for these sizes (its choice, restated for the
    label): 64-query waves at d = 128 once B * Hq * ceil(N / 512) reaches 512 (causal) or
    256; two waves per 32 queries on the smallest grids; else one 32-query wave each."""
    if d == 128 and B * Hq * -(-N // 512) >= (512 if causal else 256):
        return "fwd_unit2_kernel"
    small = (B * Hq * -(-N // 128) <= (512 if causal else 256) if d == 128
             else B * Hq * -(-N // 64) <= (1024 if causal else 512))
    return "fwd_unit_kernel (two waves per 32 queries)" if small else "fwd_unit_kernel"


def _dkdv_kernels(B, Hq, Hkv, N, causal):
    """The dK/dV launches fa_bwd makes for these sizes (its choice, restated for the label):
    records of 256 keys (64 a wave) or 128, split into chunks (and a reduction) when few;
    with the dQ pass (which also forms the row terms) the launch count of the backward."""
    steps, target = (Hq // Hkv) * -(-N // 32), 512 if causal else 256
    chunks = lambda r, m: max(min(target // r, 16, steps // m), 1)
    r256, r128 = B * Hkv * -(-N // 256), B * Hkv * -(-N // 128)
    name, k = (("bwd_dkdv64_kernel", chunks(r256, 256))
               if r256 >= target or r256 * chunks(r256, 256) >= r128 * chunks(r128, 32)
               else ("bwd_dkdv_kernel", chunks(r128, 32)))
    return (name + " + bwd_reduce_kernel", 3) if k > 1 else (name, 2)


def bench_sweep(args):
    """Forward and backward TFLOP/s (algorithmic FLOPs / time with HIP events on the launch
    stream, best of three rounds of 10 calls each, the rounds of the three calls interleaved so that
    each sees the same clocks) over d in {128, 64}, (B, Hq, Hkv) in
    {(1, 16, 16), (1, 32, 8), (2, 32, 8), (4, 32, 8)}, N from 1K to 16K (at most 1M query
    rows), causal or not; seeded N(0, 1) bf16 inputs, and fp16 ones at d = 128, N >= 4K.
    The forward is timed twice: fa_fwd, and fa_fwd_splitkv with as many queries as keys
    (the key-split route, default splits)."""
    import torch
    import workloads
    import exact_io_aware_fwd_amd as fa
    from exact_io_aware_fwd_amd import metrics

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    def best_ms(fns, reps=10, rounds=3):
        for fn in fns:
            fn()
        torch.cuda.synchronize()
        best = [float("inf")] * len(fns)
        for _ in range(rounds):
            for i, fn in enumerate(fns):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    fn()
                e1.record(stream)
                torch.cuda.synchronize()
                best[i] = min(best[i], e0.elapsed_time(e1) / reps)
        return best

    warm_until = time.perf_counter() + 0.3    # let the clocks ramp before the first shape
    print("| d | dtype | B | Hq/Hkv | N | causal | fa_fwd ms | fwd TFLOP/s | split-KV fwd ms (splits) | "
          "split TFLOP/s | fa_bwd ms | bwd TFLOP/s |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|", flush=True)
    for d in (128, 64):
        for (B, Hq, Hkv) in ((1, 16, 16), (1, 32, 8), (2, 32, 8), (4, 32, 8)):
            for N in (1024, 2048, 4096, 8192, 16384):
                if B * Hq * N > 2 * 32 * 16384:
                    continue
                # fp16 as well where the sm75 README's tables measure it at length (d = 128, N >= 4K)
                for dt in ((torch.bfloat16, torch.float16) if d == 128 and N >= 4096 else (torch.bfloat16,)):
                    q, k, v, do = (workloads.randn(1000 + i, (B, h, N, d), dt).to(dev)
                                   for i, h in enumerate((Hq, Hkv, Hkv, Hq)))
                    for causal in (True, False):
                        o = torch.empty_like(q)
                        lse = torch.empty(B, Hq, N, dtype=torch.float32, device=dev)
                        ws = torch.empty(max(fa.bwd_workspace_size(B, Hq, Hkv, N, d, q.dtype, causal), 16),
                                         dtype=torch.uint8, device=dev)
                        wss = torch.empty(max(fa.splitkv_workspace_size(B, Hq, Hkv, N, N, d, q.dtype), 16),
                                          dtype=torch.uint8, device=dev)
                        nsp = fa.splitkv_num_splits(B, Hq, Hkv, N, N, d)
                        fwd = lambda: fa.fwd(q, k, v, causal=causal, out=o, lse=lse)
                        while time.perf_counter() < warm_until:
                            fwd()
                            torch.cuda.synchronize()
                        # the backward reads the forward's O and LSE: fa_fwd and the key-split
                        # route write the same values (within rounding) into them
                        tf, ts, tb = best_ms([
                            fwd,
                            lambda: fa.fwd_splitkv(q, k, v, causal=causal, workspace=wss, out=o, lse=lse),
                            lambda: fa.bwd(q, k, v, o, lse, do, causal=causal, workspace=ws)])
                        ff = metrics.fwd_flops(B, Hq, N, d, causal)
                        fb = metrics.bwd_flops(B, Hq, N, d, causal)
                        name = {torch.bfloat16: "bf16", torch.float16: "fp16"}[dt]
                        print(f"| {d} | {name} | {B} | {Hq}/{Hkv} | {N} | {'yes' if causal else 'no'} | {tf:.4f} | "
                              f"{ff / tf / 1e9:.0f} | {ts:.4f} ({nsp}) | {ff / ts / 1e9:.0f} | {tb:.4f} | "
                              f"{fb / tb / 1e9:.0f} |", flush=True)
                    del q, k, v, do


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize, args.pmc)
        return
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.gemm_calibration:
        gemm_calibration()
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    if args.fp8:
        bench_fp8(args)
        return
    if args.masks:
        bench_masks(args)
        return
    if args.decode:
        bench_decode(args)
        return
    if args.sweep:
        bench_sweep(args)
        return

    import torch
    import workloads
    import exact_io_aware_fwd_amd as fa
    from exact_io_aware_fwd_amd import metrics

    w = workloads.WORKLOADS[args.workload or workloads.HEADLINE]
    causal = True in w.causal
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cpu_inputs = workloads.make_inputs(w)
    if len(cpu_inputs) == 3:
        cpu_inputs = cpu_inputs + (workloads.randn(w.seeds[2] + 1, (w.B, w.Hq, w.N, w.d), w.torch_dtype),)
    q, k, v, do = (t.to(dev) for t in cpu_inputs)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.bwd_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.d, q.dtype, causal), dtype=torch.uint8,
                     device=dev)

    def step():
        fa.fwd(q, k, v, causal=causal, softmax_scale=w.scale, out=o, lse=lse)
        if not args.fwd_only:
            fa.bwd(q, k, v, o, lse, do, causal=causal, softmax_scale=w.scale, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        fa.fwd(q, k, v, causal=causal, softmax_scale=w.scale, out=o, lse=lse)
        ev[i][1].record(stream)
        if not args.fwd_only:
            fa.bwd(q, k, v, o, lse, do, causal=causal, softmax_scale=w.scale, workspace=ws)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    fwd_t = sorted(e[0].elapsed_time(e[1]) for e in ev)
    bwd_t = sorted(e[1].elapsed_time(e[2]) for e in ev)
    fwd_ms, bwd_ms = sum(fwd_t) / args.steps, sum(bwd_t) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    f_fwd = metrics.fwd_flops(w.B, w.Hq, w.N, w.d, causal)
    f_bwd = 0.0 if args.fwd_only else metrics.bwd_flops(w.B, w.Hq, w.N, w.d, causal)
    peak = metrics.MFMA_BF16_TFLOPS
    value = (f_fwd + f_bwd) / (ms_per_step * 1e-3) / 1e12

    def med(t):
        return 0.5 * (t[(len(t) - 1) // 2] + t[len(t) // 2])

    # per pass: mean (the roofline figure), median and min of the per-step event times;
    # tflops and frac from the mean, tflops_median from the median
    passes = {"fwd": {"kernel": _fwd_kernel(w.B, w.Hq, w.N, w.d, causal), "launches": 1, "ms": fwd_ms,
                      "median_ms": med(fwd_t),
                      "min_ms": fwd_t[0], "tflops": f_fwd / (fwd_ms * 1e-3) / 1e12,
                      "tflops_median": f_fwd / (med(fwd_t) * 1e-3) / 1e12}}
    passes["fwd"]["frac"] = passes["fwd"]["tflops"] / peak
    if not args.fwd_only:
        dkdv, nl = _dkdv_kernels(w.B, w.Hq, w.Hkv, w.N, causal)
        passes["bwd"] = {"kernel": "bwd_dq_kernel + " + dkdv, "launches": nl,
                         "ms": bwd_ms, "median_ms": med(bwd_t), "min_ms": bwd_t[0],
                         "tflops": f_bwd / (bwd_ms * 1e-3) / 1e12,
                         "tflops_median": f_bwd / (med(bwd_t) * 1e-3) / 1e12}
        passes["bwd"]["frac"] = passes["bwd"]["tflops"] / peak
    def roofline(kind):
        # the recorded counters are the headline workload's: other workloads get none
        traffic = traffic_bytes(kind) if w.name == workloads.HEADLINE else None
        return {"bound": "mfma", "achieved": passes[kind]["tflops"], "peak": peak, "unit": "TFLOP/s",
                "frac": passes[kind]["frac"], "traffic": traffic, "kernel": passes[kind]["kernel"],
                "per_launch_flops": f_fwd if kind == "fwd" else f_bwd, "avg_ms": passes[kind]["ms"],
                "median_ms": passes[kind]["median_ms"], "min_ms": passes[kind]["min_ms"],
                "algorithmic_bytes": (metrics.fwd_bytes if kind == "fwd" else metrics.bwd_bytes)(
                    w.B, w.Hq, w.Hkv, w.N, w.d, 2)}
    dom = max(passes, key=lambda n: passes[n]["ms"])
    roof = roofline(dom)

    dt_name = {torch.bfloat16: "bf16", torch.float16: "fp16"}[q.dtype]
    rec = {
        "metric": f"attention fwd/bwd TFLOPS and % MFMA peak at N={w.N} d={w.d} {dt_name} "
                  f"{'causal' if causal else 'non-causal'}",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dt_name, "data": "synthetic (seeded iid N(0,1))",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "causal": causal, "step": "fa_fwd" if args.fwd_only else "fa_fwd + fa_bwd",
                   "flops_per_step": f_fwd + f_bwd},
        "frac_of_peak": value / peak,
        "roofline": roof,
        "roofline_fwd": roofline("fwd"),
        "passes": passes,
    }
    if not args.no_cpu_baseline:
        # one more step outside the timed region, whose outputs the oracle checks
        o_chk, lse_chk = fa.fwd(q, k, v, causal=causal, softmax_scale=w.scale)
        outs = [o_chk, lse_chk]
        if not args.fwd_only:
            outs += list(fa.bwd(q, k, v, o_chk, lse_chk, do, causal=causal, softmax_scale=w.scale, workspace=ws))
        torch.cuda.synchronize()
        outs = [t[:1].cpu() for t in outs]
        rec["cpu_baseline"] = cpu_baseline(w, cpu_inputs, args.cpu_heads, args.fwd_only, outs)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
