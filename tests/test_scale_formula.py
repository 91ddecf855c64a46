"""The INT8 kernels compute a block's scale RN(max|x| / 127) as an
fma-corrected product instead of a division; this checks that formula on
the CPU for every non-negative finite binary32 value (IEEE fma and division,
no flush to zero)."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.timeout(600)
def test_scale_formula_is_the_correctly_rounded_quotient(tmp_path):
    exe = tmp_path / "scale_div"
    flags = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math"]
    cpuinfo = open("/proc/cpuinfo").read() if os.path.exists("/proc/cpuinfo") else ""
    if " fma " in cpuinfo:
        flags.append("-mfma")  # hardware fma; libm's fmaf is used otherwise (also correctly rounded)
    subprocess.run(["gcc", *flags, "-o", str(exe), os.path.join(HERE, "c", "scale_div_exhaustive.c"), "-lm"],
                   check=True)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, env=env, timeout=600)
    assert out.stdout.strip() == "0"
