"""Build the routed-MoE C-ABI library for gfx950 with hipcc (in-tree, no JIT cache).

    python routed_expert_ffn_02_amd/_build.py        # compile csrc/ -> libroutedmoe.so
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(os.path.dirname(HERE), "_build")
LIB = os.path.join(HERE, "libroutedmoe.so")
ARCH = os.environ.get("RMOE_OFFLOAD_ARCH", "gfx950")

HIP_SOURCES = ["route.hip", "lookup.hip", "decode.hip", "prefill.hip", "fill.hip"]
CPP_SOURCES = ["runtime.cpp", "cpu_ffn.cpp", "placement.cpp", "bank.cpp"]

# Packed fp32 VALU ops are disabled for all device code (the host pass warns that it
# does not know the feature; that is harmless).
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-Wno-unused-result", "-fvisibility=hidden"]
CPP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wno-unused-result", "-D__HIP_PLATFORM_AMD__", "-fvisibility=hidden"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def rocm_root() -> str:
    return os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))


def host_cxx() -> str:
    """ROCm's clang++ for the host-only sources (runtime, CPU branch)."""
    cand = os.path.join(rocm_root(), "lib", "llvm", "bin", "clang++")
    return cand if os.path.exists(cand) else (shutil.which("clang++") or "g++")


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    if src.endswith(".hip"):
        cmd = [hipcc()] + HIP_FLAGS + ["-c", path, "-o", obj]
    else:
        cmd = [host_cxx()] + CPP_FLAGS + ["-I", os.path.join(rocm_root(), "include"), "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link libroutedmoe.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = HIP_SOURCES + CPP_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}"] + objs + ["-o", tmp, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
