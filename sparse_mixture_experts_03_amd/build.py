"""Build libmoe.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Every translation unit is compiled with hipcc for gfx950 only.  Packed
fp32 instructions are disabled for device code (the flag is a device
target feature; the host pass warns that it does not know it).
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["moe_api.cpp", "route.hip", "dispatch.hip", "expert_gemm.hip", "combine.hip",
           "shared.hip", "expert_fp8.hip", "backward.hip", "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC] + FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip() and verbose:
        print(out, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    build_c_client(verbose)
    return LIB


# A plain C program against include/moe.h and the HIP runtime's C API, run
# by the GPU tests (tests/c/forward_c.c); built next to the library.
C_CLIENT_SRC = os.path.join(ROOT, "tests", "c", "forward_c.c")
C_CLIENT = os.path.join(PKG, "moe_forward_c")


def build_c_client(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", INCLUDE, "-I", "/opt/rocm/include", C_CLIENT_SRC, "-o", C_CLIENT + ".tmp",
           "-L", PKG, "-lmoe", "-L", "/opt/rocm/lib", "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN", "-Wl,-rpath,/opt/rocm/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(C_CLIENT + ".tmp", C_CLIENT)
    return C_CLIENT


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
