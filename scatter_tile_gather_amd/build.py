"""Build libstg.so (HIP, gfx950) in-tree with hipcc, and the binding's C++
marshalling module for eager tile_gather calls.

Every HIP translation unit under csrc/ is compiled for gfx950 only and linked
into scatter_tile_gather_amd/libstg.so, which the ctypes binding loads.
csrc/fastcall.cpp (host code: CPython and torch's tensor headers, no kernels)
becomes scatter_tile_gather_amd/_stg_fast*.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libstg.so")
SOURCES = ["common.hip", "gather_scatter.hip", "copy.hip", "ragged.hip", "gemm.hip", "gemm_scaled.hip", "gemm_scaled_general.hip", "gather_backward_static.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}")
    return obj


def build(jobs: int = 4) -> str:
    """Compile every source and link libstg.so; always rebuilds."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}")
    os.replace(tmp, LIB)
    build_fast()
    return LIB


def build_fast() -> str:
    """Compile csrc/fastcall.cpp into the package (always rebuilds).  It reads
    torch tensors directly, so it is built against the installed torch's
    headers and libraries."""
    import sysconfig

    import torch

    tdir = os.path.dirname(torch.__file__)
    inc = [os.path.join(tdir, "include"), os.path.join(tdir, "include", "torch", "csrc", "api", "include"),
           sysconfig.get_paths()["include"], "/opt/rocm/include"]
    lib = os.path.join(tdir, "lib")
    out = os.path.join(PKG, "_stg_fast" + sysconfig.get_config_var("EXT_SUFFIX"))
    abi = int(torch._C._GLIBCXX_USE_CXX11_ABI)
    cmd = [os.environ.get("CXX", "g++"), "-O2", "-std=c++17", "-fPIC", "-shared", f"-D_GLIBCXX_USE_CXX11_ABI={abi}",
           "-D__HIP_PLATFORM_AMD__=1", "-DUSE_ROCM=1", *[f"-I{p}" for p in inc], os.path.join(CSRC, "fastcall.cpp"),
           "-o", out + ".tmp", f"-L{lib}", "-ltorch_python", "-ltorch", "-ltorch_cpu", "-lc10", "-lc10_hip",
           f"-Wl,-rpath,{lib}"]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"fastcall.cpp failed to build:\n{res.stdout}")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
