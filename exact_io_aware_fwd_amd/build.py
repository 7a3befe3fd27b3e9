"""Build the HIP attention library (libfa.so) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_decode.hip", "fa_fp8_quant.hip", "fa_fwd_fp8.hip"]
# Per-source flags.  The backward kernels keep their long-lived accumulators in AGPRs
# through inline-asm MFMAs; every other MFMA is asked to write VGPRs, which is where
# the elementwise code reads S and dP (otherwise the compiler may place those results
# in AGPRs and copy them back on every step).
SOURCE_FLAGS = {"fa_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _compile(src: str, out: str, extra: list[str]) -> tuple[str, int, str]:
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", out]
    p = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature; that note is harmless
    err = "\n".join(l for l in p.stderr.splitlines() if "packed-fp32-ops" not in l)
    return src, p.returncode, err


def build(verbose: bool = True, extra: list[str] | None = None) -> str:
    """Compile every source and link libfa.so next to this file; returns its path."""
    extra = list(extra or [])
    with tempfile.TemporaryDirectory(prefix="fa_build_") as tmp:
        objs = [os.path.join(tmp, s + ".o") for s in SOURCES]
        with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            results = list(ex.map(lambda so: _compile(so[0], so[1], extra), zip(SOURCES, objs)))
        for src, rc, err in results:
            if err.strip() and verbose:
                print(f"[{src}]\n{err}", file=sys.stderr)
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{err}")
        tmp_lib = LIB + ".tmp"
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        p = subprocess.run(link, capture_output=True, text=True)
        if p.returncode != 0:
            raise RuntimeError(f"link failed:\n{p.stderr}")
        os.replace(tmp_lib, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
