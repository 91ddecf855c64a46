"""Planted mistakes in a copy of the oracle must be caught by the pins.

Each mutant is a plausible slip (a wrong index or sign, a dropped term, a
transposed operand, a wrong half, a rounding mistake).  The mutated C source
is compiled to a temporary library and the page pins and brute-force tests
are run against it in a subprocess; every mutant must make them fail.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ar_oracle.c")

MUTANTS = {
    "ring_rs_index": ("int c = mod(i - s, n);", "int c = mod(i + s, n);"),
    "ring_ag_index": ("int c = mod(i + 1 - s, n);", "int c = mod(i - s, n);"),
    "dropped_term": ("float sum = pay[off] + w[x->dst][e];", "float sum = pay[off];"),
    "wrong_sign": ("float sum = pay[off] + w[x->dst][e];", "float sum = pay[off] - w[x->dst][e];"),
    "payload_from_receiver": ("pay[off] = w[x->src][e];", "pay[off] = w[x->dst][e];"),
    "ring_wrong_neighbour": ("members[(i + 1) % n], lo, hi, ARO_REDUCE",
                             "members[(i + n - 1) % n], lo, hi, ARO_REDUCE"),
    "hier_phase1_rotation": ("int k = mod(l - 1 - s, G);", "int k = mod(l - s, G);"),
    "hier_phase3_rotation": ("int k = mod(l - s, G);", "int k = mod(l + 1 - s, G);"),
    "hier_phase2_members": ("members[m] = m * G + l;", "members[m] = (m * G + l + 1) % N;"),
    "raben_half_choice": ("int keep_low = ((i >> (k - 1)) & 1) == 0;",
                          "int keep_low = ((i >> (k - 1)) & 1) == 1;"),
    "raben_partner": ("int p = i ^ (1 << (k - 1));\n      int ca = a[(k - 1) * N + i]",
                      "int p = i ^ (1 << (lg - k));\n      int ca = a[(k - 1) * N + i]"),
    "raben_ag_order": ("for (int k = lg; k >= 1; --k, ++step)", "for (int k = 1; k <= lg; ++k, ++step)"),
    "bf16_round_every_step": ("w[x->dst][e] = sum;", "w[x->dst][e] = widen_bf16(round_bf16(sum));"),
    "bf16_ties_up": ("uint32_t lsb = (u >> 16) & 1u;", "uint32_t lsb = 1u;"),
    "bf16_truncate": ("return (uint16_t)((u + 0x7fffu + lsb) >> 16);", "return (uint16_t)((u + 0u * lsb) >> 16);"),
    "partition_ceil": ("return (int64_t)(((__int128)c * len) / k);",
                       "return (int64_t)(((__int128)c * len + k - 1) / k);"),
    "cost_no_alpha": ("total += alpha_s + worst[r];", "total += worst[r];"),
    "cost_sum_not_max": ("if (t > worst[L.m[j].step]) worst[L.m[j].step] = t;", "worst[L.m[j].step] += t;"),
    "cross_group_label": ("if (L.m[j].src / group_size != L.m[j].dst / group_size) *cross_group_bytes += b;",
                          "if (L.m[j].src % group_size != L.m[j].dst % group_size) *cross_group_bytes += b;"),
    "int8_ef_sign": ("errs[r][lo + i] = x[i] - q_decode(", "errs[r][lo + i] = -x[i] + q_decode("),
    "int8_ef_dropped": ("x[i] = bufs[r][lo + i] + (errs ? errs[r][lo + i] : 0.0f);", "x[i] = bufs[r][lo + i];"),
    "int8_truncate": ("float r = rintf(x[i] / s);", "float r = truncf(x[i] / s);"),
    "int8_scale_255": ("float s = m / 127.0f;", "float s = m / 255.0f;"),
    "int8_block_64": ("#define ARO_QB 128", "#define ARO_QB 64"),
    "int8_dropped_own": ("x[i] = q_decode(pq[eoff + i], ps[boff]) + q_decode(q[m->dst][lo + i], sc[m->dst][b]);",
                         "x[i] = q_decode(pq[eoff + i], ps[boff]);"),
    "int8_scale_of_sender": ("sc[m->dst][b] = ps[boff];", "sc[m->dst][b] = sc[m->dst][b];"),
    "rdouble_bit_order": ("push(L, k, i, i ^ (1 << k), 0, count, ARO_REDUCE, k == lg - 1)",
                          "push(L, k, i, i ^ (1 << (lg - 1 - k)), 0, count, ARO_REDUCE, k == lg - 1)"),
    "tree_reduce_parent": ("push(L, step, i, i - (1 << k), 0, count, ARO_REDUCE, k == lg - 1)",
                           "push(L, step, i, i - 1, 0, count, ARO_REDUCE, k == lg - 1)"),
    "tree_bcast_edge": ("if ((i & ((2 << k) - 1)) == 0 && i + (1 << k) < N)",
                        "if ((i & ((2 << k) - 1)) == 0 && i + (1 << k) < N - 1)"),
    "dtree_mirror_dst": ("int dst = t == 0 ? par : N - 1 - par;", "int dst = t == 0 ? par : par;"),
    "dtree_half": ("int64_t half = part_lo(count, 2, 1);", "int64_t half = part_lo(count, 4, 1);"),
    "rounds_start_late": ("while (j0 < L.n && L.m[j0].step < first_step) ++j0;",
                          "while (j0 < L.n && L.m[j0].step <= first_step) ++j0;"),
    "rounds_end_early": ("int nsteps = (end_step >= 0 && end_step < L.nsteps) ? end_step : L.nsteps;",
                         "int nsteps = (end_step > 0 && end_step <= L.nsteps) ? end_step - 1 : L.nsteps;"),
    "dtree_child_order": ("for (int round = 0; round < lg; ++round)\n    for (int s = 0; s < N; ++s)\n"
                          "      for (int t = 0; t < 2; ++t) {\n        /* in tree 2",
                          "for (int round = 0; round < lg; ++round)\n    for (int s = N - 1; s >= 0; --s)\n"
                          "      for (int t = 0; t < 2; ++t) {\n        /* in tree 2"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-fno-fast-math",
                    "-ffp-contract=off", "-w", "-o", str(lib), str(mut), "-lm"], check=True)
    env = dict(os.environ, ARO_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle_pages.py", "tests/test_oracle_bruteforce.py",
                        "tests/test_oracle_int8ef.py", "tests/test_oracle_halves.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
