"""Builds libar.so (the HIP kernels, planner and C ABI) for gfx950, in-tree."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libar.so")
# Host code instrumented with AddressSanitizer and UndefinedBehaviorSanitizer
# (device code unchanged), for the CPU tests of the planner and the C ABI.
# Load it with AR_LIB=<path> and the clang ASan runtime preloaded.
LIB_SANITIZED = os.path.join(HERE, "libar_sanitized.so")
SANITIZE_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined " \
                 "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer".split()
SOURCES = ["plan.cpp", "kernels.hip", "qkernels.hip", "capi.hip"]

# -ffp-contract=off and no fast-math: every add is one IEEE binary32 add.
# -fno-gpu-flush-denormals-to-zero: fp32 denormals are kept on the device.
# packed-fp32 ops are disabled: the kernels are built from scalar adds.
# fp32 division on the device is correctly rounded (the INT8 quantizer).
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(out=LIB, defines=(), verbose=False, sanitize=False):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    objs = []
    tmpdir = os.path.join(HERE, "_build")
    os.makedirs(tmpdir, exist_ok=True)
    defs = [f"-D{d}" for d in defines]
    san = SANITIZE_FLAGS if sanitize else []
    cmd = [hipcc, *HIPCC_FLAGS, *san, *defs, "-o", out] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed")
    # the host pass does not know the packed-fp32 feature and says so; drop that noise
    noise = "'-packed-fp32-ops' is not a recognized feature"
    for line in (r.stdout + r.stderr).splitlines():
        if noise not in line and line.strip() and verbose:
            print(line)
    del objs
    return out


if __name__ == "__main__":
    print(build(verbose=True))
