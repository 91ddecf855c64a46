"""The C-ABI library loads on a CPU-only host and exports every entry point
include/ar.h declares (no compute calls here)."""
import ctypes
import os
import re
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ar.h")
LIB = os.path.join(ROOT, "gradient_all_reduce_ar_amd", "libar.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ar_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("ar_plan_create", "ar_allreduce", "ar_plan_stats", "ar_plan_destroy",
                     "ar_bucket_plan_create", "ar_bucket_allreduce", "ar_last_error"):
        assert required in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing


def test_library_loads_and_binds():
    lib = ctypes.CDLL(LIB)
    for n in declared_functions():
        assert hasattr(lib, n)
    from gradient_all_reduce_ar_amd import _binding

    assert _binding.lib() is not None


def test_header_compiles_as_c():
    src = '#include "ar.h"\nint main(void){ ar_stats_t s; (void)s; return (int)AR_OK; }\n'
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), "-x", "c", "-",
                        "-fsyntax-only"], input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
