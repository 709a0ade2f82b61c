"""The C-ABI host layer built with AddressSanitizer and UndefinedBehaviorSanitizer.

Every source of the library is compiled as it is for the product, except that
the host side is instrumented (each sanitizer flag sits behind -Xarch_host: the
GPU code is left alone and never runs here).  tests/sanitize/abi_driver.c then
calls every entry point and workspace query with edge-value arguments on a
machine without a GPU: validation errors, or HS2_ERR_HIP where the arguments
are valid, and no sanitizer report.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "token_level_sparse_full_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "asan")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _tool(name):
    p = os.path.join("/opt/rocm/llvm/bin", name)
    return p if os.path.exists(p) else shutil.which(name)


def _compile(src):
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    cmd = ["/opt/rocm/bin/hipcc", "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN,
           f"-I{os.path.join(ROOT, 'include')}", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return obj


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs hipcc")
def test_host_layer_under_asan_and_ubsan():
    os.makedirs(OUT, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    drv = os.path.join(OUT, "abi_driver.o")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    r = subprocess.run([_tool("clang"), "-O1", "-g", *san, f"-I{os.path.join(ROOT, 'include')}", "-c",
                        os.path.join(ROOT, "tests", "sanitize", "abi_driver.c"), "-o", drv],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = os.path.join(OUT, "abi_driver")
    r = subprocess.run([_tool("clang++"), *san, *objs, drv, "-L/opt/rocm/lib", "-lamdhip64",
                        "-Wl,-rpath,/opt/rocm/lib", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    report = r.stdout[-2000:] + r.stderr[-4000:]
    assert r.returncode == 0, report
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, report
    assert "0 failed" in r.stdout, report
