"""Build libw4a4.so in-tree with hipcc for gfx950.

    python -m w4a4_quantized_gemm_smooth_amd.build

The host half (C++17) is compiled with g++, the device half with hipcc, and both are linked
into ``w4a4_quantized_gemm_smooth_amd/libw4a4.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libw4a4.so")
PEAK_LIB = os.path.join(PKG, "libw4a4_peak.so")
BUILD_DIR = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops (v_pk_*_f32);
# -ffp-contract=off: every fp32 step that must be bit-reproducible stays a separate IEEE op.
DEVICE_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC]
# Per translation unit: the 4-bit kernels keep MFMA results in VGPRs (the group epilogue reads them
# with plain VALU FMAs); the W8A8 kernels leave the register form of the MFMAs to the compiler.
DEVICE_SOURCES = {
    "w4a4_device.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "w4a4_device_w8a8.hip": [],
}
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-pthread", "-I", INCLUDE, "-I", CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (res.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    host_o = os.path.join(BUILD_DIR, "w4a4_host.o")
    cxx = shutil.which("g++") or "g++"
    _run([cxx, *HOST_FLAGS, "-c", os.path.join(CSRC, "w4a4_host.cpp"), "-o", host_o], verbose)
    objs = [host_o]
    for src, extra in DEVICE_SOURCES.items():
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        _run([HIPCC, *DEVICE_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    # the benchmark's measured-MFMA-peak helper (not part of the layer's library)
    tmp = PEAK_LIB + ".tmp"
    _run([HIPCC, *DEVICE_FLAGS, "-shared", os.path.join(CSRC, "peak_mfma.hip"), "-o", tmp], verbose)
    os.replace(tmp, PEAK_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
