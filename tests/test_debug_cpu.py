"""Debug aids on the CPU: the plan description (configuration, step list,
launches) and the AR_TRACE dump at plan destruction."""
import json
import os
import subprocess
import sys

import pytest

from gradient_all_reduce_ar_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("sched,n,g,dtype", [("ring", 4, 1, "fp32"), ("hierarchical", 8, 4, "bf16"),
                                              ("rabenseifner", 8, 1, "int8_ef"), ("double_tree", 4, 1, "bf16_each")])
def test_describe_matches_the_plan(sched, n, g, dtype):
    p = B.ar_plan_create(n, g, 10007, dtype, sched)
    try:
        d = B.ar_plan_describe(p)
        assert (d["nranks"], d["group_size"], d["count"], d["dtype"], d["schedule"], d["exec"]) == \
            (n, g, 10007, dtype, sched, "steps")
        st = B.ar_plan_stats(p)
        assert d["steps"] == st["steps"] and d["hbm_bytes_model"] == st["hbm_bytes_model"]
        # the step list is the transfer list, grouped by step
        x = B.ar_plan_transfers(p)
        flat = [(s["step"], *t) for s in d["step_list"] for t in s["transfers"]]
        want = list(zip(x["step"], x["src"], x["dst"], x["lo"], x["hi"], x["kind"]))
        assert flat == [tuple(int(v) for v in w) for w in want]
        assert [s["step"] for s in d["step_list"]] == sorted({int(v) for v in x["step"]})
        assert len(d["launch_list"]) == B.ar_plan_num_launches(p)
        for i, la in enumerate(d["launch_list"]):
            kind, nops = B.ar_plan_launch_info(p, i)
            assert (la["kind"], la["ops"], la["ms"]) == (kind, nops, None)
    finally:
        B.ar_plan_destroy(p)


def test_ring_step_list_is_figure_4_2():
    """N = 4 ring: in reduce-scatter step s rank i sends chunk (i - s) mod 4
    to rank i + 1 (Primer ch. 4 section 4.2, Figure 4.2), in all-gather step
    s chunk (i + 1 - s) mod 4."""
    p = B.ar_plan_create(4, 1, 4000, "fp32", "ring")
    try:
        d = B.ar_plan_describe(p)
        assert len(d["step_list"]) == 6
        for s in d["step_list"]:
            k = s["step"]
            for src, dst, lo, hi, kind in s["transfers"]:
                c = (src - k) % 4 if k < 3 else (src + 1 - (k - 3)) % 4
                assert dst == (src + 1) % 4 and (lo, hi) == (c * 1000, c * 1000 + 1000)
                assert kind == (0 if k < 3 else 1)
    finally:
        B.ar_plan_destroy(p)


def test_ar_trace_dumps_each_plan(tmp_path):
    out = tmp_path / "trace.jsonl"
    code = ("from gradient_all_reduce_ar_amd import _binding as B\n"
            "for n in (3, 5):\n"
            "    p = B.ar_plan_create(n, 1, 999, 'bf16', 'ring')\n"
            "    B.ar_plan_destroy(p)\n")
    env = dict(os.environ, AR_TRACE=str(out))
    subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, check=True, timeout=120)
    lines = [json.loads(ln) for ln in out.read_text().splitlines()]
    assert [d["nranks"] for d in lines] == [3, 5]
    assert all(d["schedule"] == "ring" and len(d["step_list"]) == 2 * (d["nranks"] - 1) for d in lines)


def test_guard_arguments():
    p = B.ar_plan_create(4, 1, 1000, "bf16", "ring")
    try:
        with pytest.raises(B.ArError):
            B.ar_plan_set_guard(p, 100)  # not a multiple of 256
        B.ar_plan_set_guard(p, 4096)
        B.ar_plan_check_guards(p)  # nothing allocated yet: nothing to check
    finally:
        B.ar_plan_destroy(p)
