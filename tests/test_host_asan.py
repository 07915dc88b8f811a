"""The C ABI's host code under AddressSanitizer.

libiq is built with AddressSanitizer on its host code only (the GPU code as
usual: each -fsanitize= follows -Xarch_host), and tests/host_asan_driver.c
calls every entry point with arguments that the host-side validation settles
by itself (rejected arguments, no-op sizes, the host-only helpers), checking
each status. Nothing is launched, so no GPU is involved. Leak checking is off:
the HIP runtime's own start-up allocations are not this library's.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not found")
def test_host_validation_is_clean_under_asan(tmp_path):
    csrc = os.path.join(ROOT, "quantized_kv_cache_wht_amd", "csrc")
    srcs = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith(".hip"))
    lib = tmp_path / "libiq_asan.so"
    build = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
             "-Xarch_host", "-fsanitize=address",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", csrc, *srcs, "-o", str(lib)]
    subprocess.run(build, check=True, capture_output=True)
    drv = tmp_path / "driver"
    subprocess.run([CLANG, "-g", "-fsanitize=address", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "host_asan_driver.c"), "-L", str(tmp_path), "-liq_asan",
                    f"-Wl,-rpath,{tmp_path}", "-o", str(drv)], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([str(drv)], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    print(out[-2000:])
    assert "AddressSanitizer" not in out
    assert r.returncode == 0 and "0 failure(s)" in r.stdout
