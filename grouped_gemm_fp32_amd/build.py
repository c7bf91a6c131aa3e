"""Build libmoe.so (the gfx950 HIP kernels and the C ABI of include/moe.h) with hipcc.

Usage: python -m grouped_gemm_fp32_amd.build   (or __graft_entry__.build()).
Each .hip file is compiled to an object in parallel, then linked into the package directory.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from emitting packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]

    def compile_one(so):
        s, o = so
        return _run([HIPCC, *FLAGS, "-c", s, "-o", o])

    jobs = max(1, min(8, len(srcs), os.cpu_count() or 1))
    with ThreadPoolExecutor(jobs) as ex:
        for out in ex.map(compile_one, zip(srcs, objs)):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    build_c_example()
    return LIB


C_EXAMPLE_SRC = os.path.join(ROOT, "tests", "c_abi", "moe_c_example.c")
C_EXAMPLE = os.path.join(ROOT, "tests", "c_abi", "moe_c_example")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_c_example() -> str:
    """The plain-C caller of the ABI that the GPU tests run (gcc, the HIP runtime's C API, no
    Python): linked against libmoe.so through an rpath relative to its own directory."""
    if not os.path.exists(C_EXAMPLE_SRC):
        return ""
    rel = os.path.relpath(PKG, os.path.dirname(C_EXAMPLE))
    tmp = C_EXAMPLE + ".tmp"
    _run(["gcc", "-std=c11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), C_EXAMPLE_SRC,
          "-o", tmp, "-L", PKG, "-lmoe", f"-Wl,-rpath,$ORIGIN/{rel}",
          "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"])
    os.replace(tmp, C_EXAMPLE)
    return C_EXAMPLE


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
