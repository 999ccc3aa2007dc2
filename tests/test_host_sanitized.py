"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer,
on the CPU: tests/host/host_checks.cpp drives the C ABI's host paths (argument
checks, scale intake, the block allocator, the angle table, thread-local
error strings) and is linked with host.cpp built with host-side sanitizers
(the kernels' objects are linked as built; no GPU is touched)."""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp8_e4m3_scaled_amd", "csrc")
OBJ = os.path.join(ROOT, "fp8_e4m3_scaled_amd", "_build")
HIPCC = "/opt/rocm/bin/hipcc"
# -Xarch_host keeps every sanitizer flag on the host side of the build
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "--offload-arch=gfx950",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_host_code_under_asan_ubsan(tmp_path):
    kernels = [os.path.join(OBJ, os.path.basename(s) + ".o") for s in sorted(glob.glob(os.path.join(CSRC, "*.hip")))]
    if not all(os.path.exists(k) for k in kernels):
        from fp8_e4m3_scaled_amd import build as b
        b.build()
    host_o, drv_o, exe = tmp_path / "host.o", tmp_path / "driver.o", tmp_path / "host_checks"
    _run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, "host.cpp"), "-o", str(host_o)])
    _run([HIPCC, *FLAGS, "-c", os.path.join(ROOT, "tests", "host", "host_checks.cpp"), "-o", str(drv_o)])
    _run([HIPCC, "--offload-arch=gfx950", *SAN, str(host_o), str(drv_o), *kernels, "-o", str(exe)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in out and "runtime error" not in out, out
    assert "host checks passed" in out
