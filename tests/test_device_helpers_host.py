"""Host checks of the routing kernels' bit-arithmetic helpers (CPU, no GPU).

The union and top-k kernels rely on a few pure integer helpers in
csrc/moe_common.h that are also host-callable: the divide-free t / k that
gives a slot's row, bit ranges of a 64-bit word, the lowest slot of a row's
window across both 64-slot words of the union, and the order-preserving float
key map of top-k.  tests/device_helpers_host.hip includes that header, checks
each helper against a bit-by-bit or arithmetic reference (exhaustively where
the domain is small, over seeded random sets and a dense-near-the-edges walk of
the float line otherwise) and prints one summary line.
"""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_decode_gate_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


def test_device_helpers_on_host(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not installed")
    exe = str(tmp_path / "device_helpers_host")
    src = os.path.join(ROOT, "tests", "device_helpers_host.hip")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O2", "-Xclang", "-target-feature", "-Xclang",
                        "-packed-fp32-ops", "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"),
                        "-I", CSRC, src, "-o", exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout[-3000:]
