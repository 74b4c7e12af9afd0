"""Build libstrata_moe.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libstrata_moe.so")
SOURCES = ["api.hip", "popularity.hip", "route.hip", "gemv.hip", "gemv_gu3.hip", "gemv_gu2.hip", "gemv_dn3.hip", "gemv_dn2.hip",
           "gemm.hip", "gemm_gu3.hip", "gemm_gu2.hip", "gemm_dn3.hip", "gemm_dn2.hip", "combine.hip",
           "probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU forms are disabled for every kernel in this library.
FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(HERE, "..", "include")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


# The host consumer of the miss list: one object per instruction set (the
# library picks one at run time), built by the host compiler.
HOST_SOURCE = "host_experts.cpp"
HOST_ISAS = {"hx512": ["-mavx512f", "-mavx512bw", "-mavx512dq", "-mavx512vl", "-mfma"],
             "hx256": ["-mavx2", "-mfma"]}
CXX = os.environ.get("CXX_HOST", "g++")


def _compile_host(ns: str) -> str:
    obj = os.path.join(BUILD, f"host_experts_{ns}.o")
    cmd = [CXX, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-psabi", *HOST_ISAS[ns], f"-DHX_NS={ns}",
           "-I", os.path.join(HERE, "..", "include"),
           "-c", os.path.join(CSRC, HOST_SOURCE), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host compile failed for {ns}:\n{r.stdout}\n{r.stderr}")
    return obj


def _compile_host_common() -> str:
    obj = os.path.join(BUILD, "host.o")
    cmd = [CXX, "-O2", "-std=c++17", "-fPIC", "-Wall", "-pthread", "-I", os.path.join(HERE, "..", "include"),
           "-c", os.path.join(CSRC, "host.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host compile failed for host.cpp:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source (always) and link the shared library."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        futs = [ex.submit(_compile, src) for src in SOURCES]
        futs += [ex.submit(_compile_host, ns) for ns in HOST_ISAS]
        futs.append(ex.submit(_compile_host_common))
        objs = [f.result() for f in futs]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
