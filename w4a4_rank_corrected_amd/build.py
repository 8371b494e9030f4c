"""Build the in-tree C-ABI library ``libsvdq.so`` for gfx950.

Host code (C-ABI validation, offline preparation) is compiled with g++;
the HIP kernels with hipcc for ``--offload-arch=gfx950``.  Objects go to
``_build/`` next to this file; the shared library to ``libsvdq.so``.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsvdq.so")

HOST_SOURCES = ["api.cpp", "prep.cpp", "bundle.cpp", "plan.cpp"]
HIP_SOURCES = ["act_kernels.hip", "gemm_kernels.hip", "scratch.hip"]
HEADERS = ["internal.h", "device_common.h"]

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
              "-Wall", "-Wextra", "-Wno-unused-parameter", f"-I{INCLUDE}", f"-I{CSRC}"]
# -packed-fp32-ops: no v_pk_*_f32 in any kernel (the host pass warns that it does
# not know the feature; that is harmless).
# -amdgpu-mfma-vgpr-form: MFMA results land in arch VGPRs, where the fp32 scale
# epilogue reads them without v_accvgpr_read copies.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form",
             "-Wno-unused-parameter", f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def kernel_resources(remarks: str) -> list:
    """Per-kernel register and scratch use from the compiler's
    ``-Rpass-analysis=kernel-resource-usage`` remarks: a list of dicts with
    name, vgprs, agprs, sgprs, scratch (bytes per lane) and occupancy."""
    rows, cur = [], None
    keys = {"VGPRs": "vgprs", "AGPRs": "agprs", "SGPRs": "sgprs",
            "ScratchSize [bytes/lane]": "scratch", "Occupancy [waves/SIMD]": "occupancy"}
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            rows.append(cur)
            continue
        if cur is None:
            continue
        for label, key in keys.items():
            m = re.search(re.escape(label) + r": (\d+)", line)
            if m:
                cur[key] = int(m.group(1))
    return rows


def _compile_kernels(src: str, obj: str, verbose: bool) -> None:
    """hipcc for gfx950 with the resource-usage remarks; fails the build if any
    kernel spills to scratch (a spilled kernel is slow, and a spill around a
    divergent region has produced wrong results in a GEMM build)."""
    cmd = [HIPCC, *HIP_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        out = "\n".join(l for l in res.stdout.splitlines() if "remark:" not in l)
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    rows = kernel_resources(res.stdout)
    spilled = [r for r in rows if r.get("scratch", 0) > 0]
    if spilled:
        raise RuntimeError(f"{src}: kernels spill to scratch: " +
                           ", ".join(f"{r['name']} ({r['scratch']} B/lane)" for r in spilled))
    if verbose:
        for r in rows:
            print(f"  {r['name'][:100]}: {r.get('vgprs')} VGPRs, {r.get('sgprs')} SGPRs, "
                  f"occupancy {r.get('occupancy')}, scratch {r.get('scratch')}", flush=True)


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libsvdq.so``; returns its path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _compile_kernels(src, obj, verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs, "-lpthread"], verbose)
    os.replace(tmp, LIB)
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)
    if os.path.exists(LIB):
        os.remove(LIB)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
