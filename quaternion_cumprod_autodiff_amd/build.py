"""Build the gfx950 HIP library libquatcumprod.so in-tree with hipcc.

Every HIP translation unit is compiled with packed-fp32 instructions switched
off (``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass
prints that it does not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libquatcumprod.so")
SOURCES = ["qc_kernels.hip", "qc_abi.cpp", "qc_scan.hip", "qc_scan_schedule.cpp", "gdn2.hip"]
ARCH = "gfx950"


def hipcc_command(out_path: str) -> list[str]:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    return [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *[os.path.join(CSRC, s) for s in SOURCES], "-o", out_path]


def build(verbose: bool = False) -> str:
    """Compile the library (always recompiles) and return its path."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = hipcc_command(tmp)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    log = "\n".join(ln for ln in (proc.stdout + proc.stderr).splitlines() if noise not in ln)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + log)
    if verbose and log.strip():
        print(log, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
