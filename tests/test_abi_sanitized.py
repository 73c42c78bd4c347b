"""The C ABI's argument validation under AddressSanitizer and UndefinedBehaviorSanitizer.

The library sources are compiled again with both sanitizers on their host code (the device code is
built as usual and never runs), linked with abi_cases.cpp, and the program runs every validation
case on the CPU: each call is rejected before the library touches the GPU, or is an N = 0 no-op.
A sanitizer report or a wrong status fails the test.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "block_sparse_attention_blocks_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")

# sanitizers on the host pass only; the rest as in the library build
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
HIP_FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Wno-pass-failed",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return res.returncode, res.stdout + res.stderr


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not installed")
def test_abi_validation_under_asan_and_ubsan(tmp_path):
    import sys
    sys.path.insert(0, PKG)
    from build import SOURCES  # the library's own source list
    csrc = os.path.join(PKG, "csrc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", csrc]

    def compile_one(src):
        obj = str(tmp_path / src.replace(".hip", ".o"))
        rc, out = _run([HIPCC, *HIP_FLAGS, *HOST_SANITIZE, *inc, "-c", os.path.join(csrc, src), "-o", obj])
        assert rc == 0, f"{src}:\n{out[-3000:]}"
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    exe = str(tmp_path / "abi_cases")
    rc, out = _run([CLANG, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    *inc, os.path.join(ROOT, "tests", "abi_cases.cpp"), *objs, "-L", os.path.join(ROCM, "lib"),
                    "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe])
    assert rc == 0, out[-3000:]
    env = dict(os.environ)
    # the HIP runtime keeps process-lifetime allocations; leaks are not what this test looks for
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    rc, out = _run([exe], env=env, timeout=300)
    print(out)
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-3000:]
    assert rc == 0, out[-3000:]
    assert "0 failures" in out
    shutil.rmtree(tmp_path, ignore_errors=True)
