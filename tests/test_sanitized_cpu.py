"""The planner, the C ABI's host code and the oracle under AddressSanitizer
and UndefinedBehaviorSanitizer.

Both libraries are built again with the sanitizers (the library's host code
only; device code is unchanged) by ROCm's clang, so that they share one
sanitizer runtime, which is preloaded into a child pytest process that runs
the CPU tests of the planner (all-reduce and its halves), the bucket fuser,
the debug aids and the oracle against them.  Any sanitizer report aborts that process.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from gradient_all_reduce_ar_amd import build as libbuild  # noqa: E402
from oracle import build as oracle_build  # noqa: E402

SUBSET = ["test_plan_cpu.py", "test_plan_random.py", "test_int8_plan_cpu.py", "test_debug_cpu.py",
          "test_binding_checks.py", "test_buckets.py", "test_oracle_pages.py", "test_oracle_bruteforce.py",
          "test_oracle_int8ef.py", "test_oracle_halves.py", "test_halves_cpu.py", "test_overlap.py",
          "test_zz_no_alloc.py"]


def _stale(lib, sources):
    return not os.path.exists(lib) or os.path.getmtime(lib) < max(os.path.getmtime(s) for s in sources)


def _runtime():
    clang = oracle_build.CLANG
    if not os.path.exists(clang):
        return None
    path = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.timeout(1800)
def test_cpu_suite_under_asan_and_ubsan(tmp_path):
    rt = _runtime()
    if rt is None:
        pytest.skip("ROCm clang's AddressSanitizer runtime is not installed")
    csrc = glob.glob(os.path.join(libbuild.CSRC, "*")) + [os.path.join(ROOT, "include", "ar.h")]
    if _stale(libbuild.LIB_SANITIZED, csrc):
        libbuild.build(out=libbuild.LIB_SANITIZED, sanitize=True)
    if _stale(oracle_build.LIB_SANITIZED, [oracle_build.SRC]):
        oracle_build.build_sanitized()
    log = tmp_path / "sanitizer"
    env = dict(os.environ, LD_PRELOAD=rt, AR_LIB=libbuild.LIB_SANITIZED, ARO_LIB=oracle_build.LIB_SANITIZED,
               ASAN_OPTIONS=f"detect_leaks=0:abort_on_error=1:log_path={log}",
               UBSAN_OPTIONS=f"print_stacktrace=1:halt_on_error=1:log_path={log}")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider", "-n", "4"]
    cmd += [os.path.join(ROOT, "tests", t) for t in SUBSET]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1700)
    reports = "".join(open(f).read() for f in glob.glob(f"{log}*"))
    assert r.returncode == 0 and not reports, (r.stdout[-3000:] + r.stderr[-3000:] + reports[:5000])
