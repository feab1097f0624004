"""Build libws.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libws.so")

SOURCES = ["capi.hip", "kv_append.hip", "fm_euler.hip", "attn_fwd.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libws)")


def compile_command(out: str) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed-FP32 VALU forms are kept out of generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", INCLUDE, "-I", CSRC,
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out,
    ]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libws.so next to this file (always
    recompiles). Returns the library path."""
    tmp = LIB_PATH + ".tmp"
    cmd = compile_command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or res.returncode != 0:
        print(" ".join(cmd))
        if res.stdout:
            print(res.stdout)
        if res.stderr:
            print(res.stderr)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.unlink(tmp)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


DEMO_SRC = os.path.join(PKG_DIR, "examples", "c_abi_demo.c")
DEMO_PATH = os.path.join(PKG_DIR, "examples", "c_abi_demo")


def build_demo(verbose: bool = False) -> str:
    """Compile examples/c_abi_demo.c, a plain C99 caller of include/ws.h,
    against libws.so and the HIP runtime (host code only: gcc, no hipcc)."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", INCLUDE, DEMO_SRC,
           "-L", PKG_DIR, "-lws", "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/..", "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", DEMO_PATH]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or res.returncode != 0:
        print(" ".join(cmd))
        print(res.stdout + res.stderr)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed with exit code {res.returncode}")
    return DEMO_PATH


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_demo(verbose=True))
