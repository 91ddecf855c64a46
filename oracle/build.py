"""Builds the CPU oracle (oracle/ar_oracle.c) into oracle/liboracle.so.

TEST INFRASTRUCTURE ONLY: the oracle is the parity authority for the GPU
library and is never part of the product path.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ar_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# Plain single-threaded C; no fast-math and no contraction, so every add is
# one IEEE-754 binary32 add with denormals kept.
CFLAGS = ["-O2", "-std=gnu11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
          "-Wall", "-Wextra", "-Werror"]


def build(out=LIB, extra=()):
    cmd = ["gcc", *CFLAGS, *extra, "-o", out, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return out


# The same oracle with AddressSanitizer and UndefinedBehaviorSanitizer, built
# with ROCm's clang so that it shares one sanitizer runtime with the
# instrumented planner library (load it with ARO_LIB=<path>).
LIB_SANITIZED = os.path.join(HERE, "liboracle_sanitized.so")
CLANG = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")


def build_sanitized(out=LIB_SANITIZED):
    cmd = [CLANG, "-O1", "-g", "-std=gnu11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           "-Wall", "-Wextra", "-Werror", "-o", out, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build())
