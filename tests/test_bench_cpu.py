"""Host-side helpers of bench.py: which probe mix a kernel is set against,
the staged bound of the LDS one-pass folds, read shares and kernel labels
(the names rocprofv3 reports).  No GPU: the helpers are plain Python."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


CEIL = {
    "read 1:0": {"GBps": 7100.0, "read_share": 1.0},
    "write 0:1": {"GBps": 6900.0, "read_share": 0.0},
    "copy 1:1": {"GBps": 6640.0, "read_share": 0.5},
    "reduce 2:1": {"GBps": 6700.0, "read_share": 2 / 3},
    "reduce 2:2": {"GBps": 5930.0, "read_share": 0.5},
    "fold 16:16": {"GBps": 5470.0, "read_share": 0.5},
    "read 16:0": {"GBps": 6680.0, "read_share": 1.0},
    "write 0:16 split": {"GBps": 6500.0, "read_share": 0.0},
    "fold 32:32": {"GBps": 5200.0, "read_share": 0.5},
}


def test_staged_bound_is_the_harmonic_mean_of_the_two_phases():
    # equal bytes read then written: T = S/2/rd + S/2/wr
    want = 1.0 / (0.5 / 6680.0 + 0.5 / 6500.0)
    assert bench.staged_bound(CEIL, 16) == pytest.approx(want, abs=0.06)
    assert 6500.0 < bench.staged_bound(CEIL, 16) < 6680.0
    assert bench.staged_bound(CEIL, 8) is None  # no probes for 8 buffers
    assert bench.staged_bound({"read 16:0": CEIL["read 16:0"]}, 16) is None


@pytest.mark.parametrize("kind,nbuf,staged,want", [
    (0x100, 16, False, "reduce 2:1"),           # chunk_reduce
    (0x100 | 8, 16, False, "reduce 2:2"),       # fused last reduce-scatter + first all-gather
    (0x200 | 4, 16, False, "copy 1:1"),         # chunk_copy
    (0x300, 16, False, "fold 16:16"),           # register one-pass ring, fp32
    (0x500 | 1, 16, False, "fold 16:16"),       # register one-pass tree, bf16
    (0x303, 32, False, "fold 32:32"),           # INT8 one-pass ring: 16 rank + 16 residual buffers
    (0x303, 64, False, "copy 1:1"),             # no probe for that buffer count: nearest read share
    (0x300, 16, True, "read 16:0 then write 0:16 split"),  # LDS-staged one-pass ring
])
def test_attainable_mix(kind, nbuf, staged, want):
    name, rate = bench.attainable_for(CEIL, kind, 4, nbuf, staged=staged)
    assert name == want
    if staged:
        assert rate == bench.staged_bound(CEIL, nbuf)
    else:
        assert rate == CEIL[name]["GBps"]


def test_int8_step_kernels_take_the_nearest_two_buffer_mix():
    # q_hop and q_copy_dec: one-pass probes are never chosen for them
    name, _ = bench.attainable_for(CEIL, 0x800 | 3, 4, 32)
    assert name in ("read 1:0", "write 0:1", "copy 1:1", "reduce 2:1", "reduce 2:2")


@pytest.mark.parametrize("kind,elem,want", [
    (0x100, 4, 8 / 12),             # fp32 reduce: 2 reads, 1 write
    (0x100 | 8, 4, 8 / 16),         # fp32 fused: 2 reads, 2 writes
    (0x100 | 3, 2, 4 / 8),          # bf16 round 0: two bf16 reads, fp32 partial out
    (0x100 | 2 | 4, 2, 6 / 8),      # bf16 last round: fp32 partial + bf16 own in, bf16 out
    (0x200, 4, 0.5),
    (0x300, 4, 0.5),
])
def test_read_share(kind, elem, want):
    assert bench.read_share(kind, elem) == pytest.approx(want)


def test_kernel_labels():
    assert bench.kernel_label(0x100, {"units": 2, "cpol": 16}) == "chunk_reduce<0, 2, 16>"
    assert bench.kernel_label(0x200 | 4, {"units": 2, "cpol": 16}) == "chunk_copy<4, 2, 16>"
    assert bench.kernel_label(0x800 | 2) == "q_hop<2>"
    assert bench.kernel_label(0x900 | 16) == "q_copy_dec<true>"
    assert bench.kernel_label(0x303) == "q_onepass_ring"
    lds = {"units": 2, "batch": 16, "cpol": 18, "lds_bytes": 32768}
    assert bench.kernel_label(0x300, lds, 16) == "onepass_lds<false, false, 16, 16, 18, RingFold>"
    # a 5-rank tree pads to 8 leaves (missing leaves are -0)
    assert bench.kernel_label(0x500 | 1, dict(lds, batch=8), 5) == \
        "onepass_lds<true, false, 16, 8, 18, TreeFold<8, true>>"
    assert bench.kernel_label(0x600 | 2, dict(lds, batch=8), 64) == \
        "onepass_lds<true, true, 64, 8, 18, DTreeFoldOp<64>>"
    # reduce-scatter folds (flag 0x1000) of up to 16 ranks run their own tiles
    own = {"units": 4, "batch": 16, "cpol": 16, "lds_bytes": 65536}
    assert bench.kernel_label(0x1300, own, 16) == "onepass_lds<false, false, 16, 16, 16, OwnerTiles<RingFold>>"
    assert bench.kernel_label(0x1500 | 1, dict(own, batch=8), 16) == \
        "onepass_lds<true, false, 16, 8, 16, OwnerTiles<TreeFold<16, false>>>"
    assert bench.kernel_label(0x1300, dict(lds, batch=8), 32) == "onepass_lds<false, false, 32, 8, 18, RingFold>"
