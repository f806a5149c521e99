"""Build libsmoe.so in-tree with hipcc for gfx950.

Usage: python -m quantized_speculative_expert_amd.build  (or build() from Python).
Every call recompiles all sources.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libsmoe.so")

ARCH = "gfx950"
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fno-gpu-rdc",
    # packed fp32 VALU ops stay off (these flags never emit them)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build libsmoe)")
    return path


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def scratch_users(remarks: str):
    """(kernel, bytes per lane) of every kernel the compiler's resource
    remarks show with scratch memory."""
    out, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name is not None and int(m.group(1)) > 0:
            out.append((name, int(m.group(1))))
    return out


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every HIP source and link libsmoe.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    flags = HIPCC_FLAGS + list(extra_flags or [])

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        # the resource-usage remarks name every kernel's scratch use
        cmd = [hipcc, *flags, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        spills = scratch_users(r.stderr)
        if spills:
            raise RuntimeError(f"{os.path.basename(src)}: kernels use scratch memory (register "
                               "spills): " + ", ".join(f"{k} ({b} B/lane)" for k, b in spills))
        if verbose:
            out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                            if "packed-fp32-ops" not in l and "remark:" not in l)
            if out.strip():
                print(out)
        return obj

    jobs = max(1, min(16, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        objs = list(pool.map(compile_one, sources()))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    v = "-v" in sys.argv
    print(build(verbose=v))
