"""Build libssb.so (HIP kernels + C ABI) for gfx950 with hipcc, in the package directory.

Usage: python -m aberration_phase_variance_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libssb.so")
SOURCES = ["ssb_kernels.hip", "ssb_api.cpp", "ssb_fit.cpp", "ssb_detector.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags() -> list:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        # no packed-FP32 (v_pk_*_f32) instructions anywhere in the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option",
    ]


def build(verbose: bool = False) -> str:
    """Compile every source into libssb.so; always recompiles.  Returns the library path."""
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc()] + flags() + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError(f"hipcc failed with exit code {proc.returncode}")
    noise = [ln for ln in proc.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
