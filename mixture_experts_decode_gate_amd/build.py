"""Build libmoe.so (HIP, gfx950) in-tree with hipcc.

    python -m mixture_experts_decode_gate_amd.build

Every HIP source is compiled for gfx950 only.  Packed-FP32 instruction
selection is disabled (``-packed-fp32-ops``), and floating-point contraction
is off so every fused multiply-add in the kernels is an explicit one.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["moe_abi.hip", "moe_kernels.hip", "moe_gateup_rows_1_4.hip", "moe_gateup_rows_5_8.hip",
           "moe_gateup_rows_9_12.hip", "moe_gateup_rows_13_16.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe.so)")


COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="moe_build_")
    try:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            cmd = [cc, *COMMON, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            out = (r.stdout + r.stderr).strip()
            # hipcc's host pass does not know the gfx950 feature name; that note is expected
            lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(lines))
            if verbose and lines:
                print("\n".join(lines), file=sys.stderr)
            return obj

        with ThreadPoolExecutor(len(SOURCES)) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        tmp_lib = LIB + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
        os.replace(tmp_lib, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
