"""Build step of the HIP library: hipcc for gfx950 -> block_verify_forward_amd/libbvf.so (in-tree)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbvf.so")
SOURCES = ["bvf_api.cpp", "gemm.hip", "layer_ops.hip"]
ARCH = os.environ.get("BVF_OFFLOAD_ARCH", "gfx950")


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           # packed fp32 (v_pk_*_f32) stays off on this target: compile plain fp32 VALU code only
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-o", LIB + ".tmp"] + [os.path.join(CSRC, s) for s in SOURCES]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed")
    if verbose:
        sys.stderr.write("\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l))
    os.replace(LIB + ".tmp", LIB)
    return LIB


SAN_LIB = os.path.join(ROOT, "_build", "libbvf_san.so")


def build_sanitized() -> str:
    """The same library with AddressSanitizer and UndefinedBehaviorSanitizer on its host code only
    (descriptor checks, arena layout, planners, state bookkeeping), for CPU tests of the host side:
    _build/libbvf_san.so (not a product artefact; the device code is built as usual)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    cmd = [hipcc, f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-o", SAN_LIB + ".tmp"] + [os.path.join(CSRC, s) for s in SOURCES]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc (host sanitizers) failed")
    os.replace(SAN_LIB + ".tmp", SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    print(build(verbose=True))
