"""bench.py's bookkeeping on the CPU: which bench line a recorded kernel belongs to, and the
kernel label it prints for a shape (the same launch rules fa_fwd applies)."""
from __future__ import annotations

import json
import os

import bench


def test_traffic_kind_of_every_recorded_kernel():
    """Each record in profiles/traffic.json names kernels that map back to its own line."""
    with open(os.path.join(bench.ROOT, "profiles", "traffic.json")) as f:
        data = json.load(f)
    assert set(data) == {"fwd", "bwd", "decode", "fp8", "masks"}
    for kind, rec in data.items():
        for name in rec["kernel"].split(" + "):
            assert bench.traffic_kind(name) == kind, (kind, name)


def test_traffic_kind_of_substrings():
    assert bench.traffic_kind("fwd_unit2_kernel") == "fwd"
    assert bench.traffic_kind("fwd_unit_kernel<fa::bf16_tag, 128, false, 12, true, 1>") == "masks"
    assert bench.traffic_kind("fwd_unit_kernel<fa::bf16_tag, 128, true, 8, false, 2>") == "fwd"
    assert bench.traffic_kind("bwd_dkdv64_kernel|bwd_dq_kernel") == "bwd"
    assert bench.traffic_kind("splitkv_kernel|lse_combine_kernel") == "decode"
    assert bench.traffic_kind("fwd_fp8_kernel") == "fp8"


def test_forward_kernel_labels():
    assert bench._fwd_kernel(2, 32, 8192, 128, True) == "fwd_unit2_kernel"          # the metric's shape
    assert bench._fwd_kernel(1, 16, 1024, 128, True).startswith("fwd_unit_kernel (two waves")
    assert bench._fwd_kernel(1, 32, 3072, 128, True) == "fwd_unit_kernel"           # 768 blocks of 128
    assert bench._fwd_kernel(1, 16, 1024, 64, False).startswith("fwd_unit_kernel (two waves")
    assert bench._fwd_kernel(2, 32, 8192, 64, True) == "fwd_unit_kernel"
