"""Builds libck4.so (the HIP kernels + C ABI) in-tree with hipcc for gfx950,
and libck4_bench.so (the benchmark's streaming-read probe, outside the ABI).

Usage: ``python -m int4_w4a4_quantized_amd._build`` or ``build()`` from Python.
Compiles every source each time it is called (objects in parallel), then links.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
LIB = os.path.join(PKG, "libck4.so")
BENCH_LIB = os.path.join(PKG, "libck4_bench.so")
OBJDIR = os.path.join(PKG, "_build")

SOURCES = ["rotate_quant.hip", "gemm.hip", "gemv_w4a4.hip", "skinny_layer.hip", "gemm_fp6.hip", "w4a8_decode.hip", "w4a8_gemv.hip",
           "lora.hip", "ck4_api.cpp"]
BENCH_SOURCES = ["bench_read.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # packed fp32 VALU ops stay disabled in all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, extra_flags: list | None = None) -> str:
    hipcc = _hipcc()
    os.makedirs(OBJDIR, exist_ok=True)
    flags = HIPCC_FLAGS + (extra_flags or []) + ["-I", INCLUDE, "-I", CSRC]

    def compile_one(src: str) -> str:
        obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc, *flags, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(BENCH_SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES + BENCH_SOURCES))
    for lib, lib_objs in ((LIB, objs[:len(SOURCES)]), (BENCH_LIB, objs[len(SOURCES):])):
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *lib_objs, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
