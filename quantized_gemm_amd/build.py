"""Build the gfx950 HIP library ``quantized_gemm_amd/lib/libsvdq.so`` in-tree with hipcc.

Flags that the numerics depend on:
  * no fast-math; IEEE float32 division and square root (hipcc's default, stated explicitly);
  * float32 denormals preserved on the GPU;
  * ``-ffp-contract=off``: no implicit fused multiply-adds (the kernels write their FMAs out);
  * packed-FP32 VALU instructions disabled (``-packed-fp32-ops``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libsvdq.so")
# per-kernel register / scratch / occupancy figures reported by the compiler during the build
RESOURCES = os.path.join(LIBDIR, "kernel_resources.txt")

SOURCES = ["api.hip", "quant_act.hip", "w4a4_gemm.hip", "w4a4_gemm_gelu.hip", "w4a4_gemm_qkv.hip", "w4a16_gemv.hip",
           "pack.cpp"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the HIP library)")


def _kernel_resources(src: str, remarks: str) -> list:
    """(source, kernel, VGPRs, AGPRs, scratch bytes per lane, waves per SIMD) from the compiler's
    kernel-resource-usage remarks."""
    rows, cur = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            rows.append(cur)
            continue
        m = re.search(r"remark: +(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).split(" ")[0]] = int(m.group(2))
    return [(src, r["name"], r.get("VGPRs", -1), r.get("AGPRs", -1), r.get("ScratchSize", -1), r.get("Occupancy", -1))
            for r in rows]


def _compile(src: str, verbose: bool):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    hip = src.endswith(".hip")
    lang = ["-x", "hip", "-Rpass-analysis=kernel-resource-usage"] if hip else []
    cmd = [hipcc(), "--offload-arch=gfx950", *COMMON, "-I", os.path.join(ROOT, "include"), *lang, "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj, (_kernel_resources(src, r.stderr) if hip else [])


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library. Returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    objs = [o for o, _ in results]
    kernels = [k for _, ks in results for k in ks]
    with open(RESOURCES, "w") as f:
        f.write("# source kernel VGPRs AGPRs scratch_bytes_per_lane waves_per_SIMD\n")
        for k in kernels:
            f.write(" ".join(str(v) for v in k) + "\n")
    spilled = [k for k in kernels if k[4] != 0]
    if spilled:
        print("warning: kernels using scratch memory (register spills): "
              + ", ".join(f"{k[1]} ({k[4]} B/lane)" for k in spilled), file=sys.stderr, flush=True)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
