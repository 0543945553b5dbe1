"""Host sanitizers on the C ABI's refusal paths (CPU, no GPU).

libmoe.so is rebuilt with AddressSanitizer and UndefinedBehaviorSanitizer on
its host code (the device code is compiled without optimisation and never
launched here), and the refusal tests of test_abi_cpu.py run against that
build in a child process that preloads the sanitizer runtime.  An
out-of-bounds access, a use after free or undefined behaviour in argument
validation, the workspace layout or the error reporting ends the child with a
sanitizer report and fails this test.
"""

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_decode_gate_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
# Sanitizers on the host side only.
SAN_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer"


def asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.fixture(scope="module")
def asan_lib(tmp_path_factory):
    if not os.path.exists(HIPCC) or asan_runtime() is None:
        pytest.skip("hipcc or the clang AddressSanitizer runtime is not installed")
    out = tmp_path_factory.mktemp("asan")
    common = ["--offload-arch=gfx950", "-std=c++17", "-fPIC", "-O1", "-g", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", "-Xarch_device", "-O0", "-Xarch_device", "-g0", *SAN_FLAGS.split(),
              "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def compile_one(src):
        obj = str(out / (os.path.basename(src)[:-4] + ".o"))
        r = subprocess.run([HIPCC, *common, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    so = str(out / "libmoe_asan.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN_FLAGS.split()[:4], "-o", so, *objs],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    with open(so, "rb") as f:
        assert b"__asan_report_load" in f.read(), "the build carries no AddressSanitizer checks"
    return so


CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
import pytest
import mixture_experts_decode_gate_amd as moe
lib = moe.load(sys.argv[2])
assert moe.load() is lib and lib._name == sys.argv[2]
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", sys.argv[3]]))
"""


def test_abi_refusals_under_asan_and_ubsan(asan_lib):
    preload = asan_runtime()
    if os.environ.get("LD_PRELOAD"):
        preload += ":" + os.environ["LD_PRELOAD"]  # the sanitizer runtime must come first
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT, asan_lib, os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       env=env, capture_output=True, text=True, timeout=600)
    report = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert r.returncode == 0, report
    assert "passed" in r.stdout and "failed" not in r.stdout, report
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, report
