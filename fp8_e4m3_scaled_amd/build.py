"""Build the kvfp8 HIP library for gfx950 in-tree.

    python -m fp8_e4m3_scaled_amd.build

Compiles every csrc/*.hip and csrc/*.cpp with hipcc (-O3, gfx950, packed-FP32
instructions disabled) and links fp8_e4m3_scaled_amd/libkvfp8.so.  The E4M3
decode's inline-asm load ring is proven sound on the assembly of the same
source and flags (ring_check.py) before the library is linked: a build whose
register allocation touches an in-flight ring register fails.
"""
from __future__ import annotations

import concurrent.futures
import glob
import importlib.util
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvfp8.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wextra", "-Werror", "-Wno-unused-parameter",
    # packed FP32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators stay in ordinary VGPRs: the softmax rescales them
    # with VALU ops, and AGPR-resident accumulators would be copied every step
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def check_decode_ring() -> int:
    """Compile decode.hip's device code to assembly with the library's flags
    and check every all-E4M3 decode instance (the ones with the inline ring)
    with ring_check; returns the number of instances checked, raises on any
    unsound one."""
    spec = importlib.util.spec_from_file_location("kvfp8_ring_check", os.path.join(PKG, "ring_check.py"))
    rc = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = rc              # dataclasses look their module up by name
    spec.loader.exec_module(rc)
    out = os.path.join(OBJ, "decode.s")
    flags = [f for f in CFLAGS if f not in ("-fPIC", "-Werror")]   # -S: hipcc adds an unused --hip-link
    cmd = [HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, "decode.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
    with open(out) as fh:
        asm = fh.read()
    symbols = re.findall(r"^(_ZN\w*decode_kernelILi\d+ELi\d+ELi1ELi1EE\w*):", asm, re.M)
    if not symbols:
        raise RuntimeError("decode ring check: no all-E4M3 decode instance in the assembly")
    for sym in symbols:
        violations, n_ring = rc.check(rc.kernel_body(asm, sym))
        if n_ring == 0 or violations:
            raise RuntimeError(f"decode ring check failed in {sym}: {n_ring} ring loads, "
                               f"{len(violations)} violations: {violations[:3]}")
    return len(symbols)


def build() -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs) + 1)) as ex:
        ring = ex.submit(check_decode_ring)
        objs = list(ex.map(_compile, srcs))
        ring.result()
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
