"""Builds tests/c/abi_use, a C program that uses libar.so through include/ar.h
alone (test infrastructure: the GPU test test_gpu_c_abi.py runs it)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_use.c")
BIN = os.path.join(HERE, "abi_use")


def build():
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    pkg = os.path.join(ROOT, "gradient_all_reduce_ar_amd")
    # host code only (no kernels in it); the library is found next to the
    # binary's relative path, so the tree can move
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    # a C file gets no HIP include path or runtime from the driver: the HIP
    # runtime header needs its platform named, and the runtime is linked
    cmd = [hipcc, "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
           "-I", os.path.join(ROOT, "include"), SRC, "-o", BIN, "-L", pkg, "-lar",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../gradient_all_reduce_ar_amd"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("building tests/c/abi_use failed")
    return BIN


if __name__ == "__main__":
    print(build())
