"""Build the gfx950 HIP library libquatcumprod.so in-tree with hipcc.

Every translation unit is compiled to an object in parallel, then linked.
Every HIP translation unit is compiled with packed-fp32 instructions switched
off (``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass
prints that it does not know the feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libquatcumprod.so")
SOURCES = ["qc_kernels.hip", "qc_abi.cpp", "qc_scan.hip", "qc_scan_schedule.cpp", "gdn2.hip", "gdn2_wy.hip", "qc_copy.hip", "qc_noalloc.hip"]
ARCH = "gfx950"
NOISE = "is not a recognized feature for this target"


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def compile_command(src: str, obj: str) -> list[str]:
    return [_hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]


def link_command(objs: list[str], out_path: str) -> list[str]:
    return [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_path]


def _run(cmd: list[str]) -> str:
    proc = subprocess.run(cmd, capture_output=True, text=True)
    log = "\n".join(ln for ln in (proc.stdout + proc.stderr).splitlines() if NOISE not in ln)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + log)
    return log


def build(verbose: bool = False) -> str:
    """Compile the library (always recompiles) and return its path."""
    with tempfile.TemporaryDirectory(prefix="qc_build_") as tmp:
        objs = [os.path.join(tmp, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        workers = max(1, min(len(SOURCES), os.cpu_count() or 1))
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as pool:
            logs = list(pool.map(_run, [compile_command(s, o) for s, o in zip(SOURCES, objs)]))
        out = LIB_PATH + ".tmp%d" % os.getpid()
        logs.append(_run(link_command(objs, out)))
    if verbose:
        text = "\n".join(ln for ln in logs if ln.strip())
        if text:
            print(text, file=sys.stderr)
    os.replace(out, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
