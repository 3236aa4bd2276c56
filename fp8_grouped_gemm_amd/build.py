"""Build the gfx950 shared library ``libmoe_gfx950.so`` in-tree with hipcc.

    python -m fp8_grouped_gemm_amd.build [-j N] [--verbose]

Every source under ``csrc/`` is compiled for gfx950 into ``_build/`` at the repository
root and linked next to this file.  No CPU fallback exists: the Python binding
refuses to load without this library.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_gfx950.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# Packed fp32 (v_pk_*_f32) code generation is switched off for all device code.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fno-gpu-rdc",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"),
]
# per-source additions
FILE_FLAGS = {
    # FP8 GEMM: MFMA results in VGPRs, so the per-block promotion FMAs read them without
    # accvgpr moves
    "gemm_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "gemm_w4a8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "gemm_fp8_big.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def scratch_users(remarks: str) -> list:
    """Kernels the compiler's resource remarks report with private (scratch) memory.

    Several kernels (the GEMMs, the router) wait for their own global->LDS copies by
    counting this wave's outstanding vector memory operations (s_waitcnt vmcnt with a
    fixed count).  Register spills add scratch loads and stores to that count, and the
    wait would then release before the copy landed, so a spilling kernel is a build
    error rather than a slowdown."""
    users, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and int(m.group(1)) > 0:
            users.append(f"{name} ({m.group(1)} bytes/lane)")
    return users


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(os.path.basename(src), []),
           "-Rpass-analysis=kernel-resource-usage", "-x", "hip", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    spills = scratch_users(r.stderr)
    if spills:
        os.remove(obj)
        raise RuntimeError(f"{src}: kernels use scratch memory (register spills), which "
                           f"breaks their counted memory waits: {', '.join(spills)}")
    return obj


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.j, a.verbose))


if __name__ == "__main__":
    sys.exit(main())
