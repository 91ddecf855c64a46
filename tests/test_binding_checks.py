"""Argument checks of the Python binding, on the CPU.

The C calls read exactly nranks pointers from the host array they are given
and let the kernels touch count elements of every buffer, so the binding
refuses a list of the wrong length and tensors that are not contiguous
device tensors of at least the plan's extent, before anything reaches C.
"""
import pytest

from gradient_all_reduce_ar_amd import _binding as B


class FakeTensor:
    """Stands in for a device tensor: only what the binding inspects."""

    def __init__(self, addr, nbytes, cuda=True, contiguous=True, elem=4):
        self.addr, self.nbytes, self.is_cuda, self.contig, self.elem = addr, nbytes, cuda, contiguous, elem

    def data_ptr(self):
        return self.addr

    def is_contiguous(self):
        return self.contig

    def numel(self):
        return self.nbytes // self.elem

    def element_size(self):
        return self.elem


def _fakes(n, nbytes, **kw):
    return [FakeTensor((r + 1) << 30, nbytes, **kw) for r in range(n)]


@pytest.fixture
def plan():
    p = B.ar_plan_create(4, 1, 1000, "bf16", "ring")
    yield p
    B.ar_plan_destroy(p)


def test_wrong_number_of_rank_buffers(plan):
    with pytest.raises(ValueError, match="3 rank buffers for a plan of 4 ranks"):
        B.ar_allreduce(plan, _fakes(3, 2000))
    with pytest.raises(ValueError, match="5 rank buffers"):
        B.ar_allreduce(plan, [1 << 20] * 5)


def test_rank_buffer_too_small(plan):
    bufs = _fakes(4, 2000, elem=2)
    bufs[2] = FakeTensor(3 << 30, 1998, elem=2)  # 999 bf16 elements, the plan needs 1000
    with pytest.raises(ValueError, match="rank buffer 2 holds 1998 bytes"):
        B.ar_allreduce(plan, bufs)


def test_host_and_strided_tensors_refused(plan):
    import torch

    host = [torch.zeros(1000, dtype=torch.int16) for _ in range(4)]
    with pytest.raises(ValueError, match="not a device tensor"):
        B.ar_allreduce(plan, host)
    bufs = _fakes(4, 2000, elem=2)
    bufs[1] = FakeTensor(2 << 30, 4000, contiguous=False, elem=2)
    with pytest.raises(ValueError, match="rank buffer 1 is not contiguous"):
        B.ar_allreduce(plan, bufs)


def test_error_buffers_checked():
    p = B.ar_plan_create(4, 1, 1000, "int8_ef", "ring")
    try:
        with pytest.raises(ValueError, match="3 error buffers"):
            B.ar_allreduce_ef(p, _fakes(4, 4000), _fakes(3, 4000))
        errs = _fakes(4, 4000)
        errs[0] = FakeTensor(9 << 30, 3996)
        with pytest.raises(ValueError, match="error buffer 0 holds 3996 bytes"):
            B.ar_allreduce_ef(p, _fakes(4, 4000), errs)
    finally:
        B.ar_plan_destroy(p)


def test_bucket_arenas_checked():
    sizes = [300, 5000, 17]
    bp = B.ar_bucket_plan_create(4, 1, sizes, "fp32", "ring", 4096)
    try:
        _, arena = B.ar_bucket_layout(bp, len(sizes))
        with pytest.raises(ValueError, match="2 rank arenas for a plan of 4 ranks"):
            B.ar_bucket_allreduce(bp, _fakes(2, arena * 4))
        short = _fakes(4, arena * 4)
        short[3] = FakeTensor(4 << 30, arena * 4 - 4)
        with pytest.raises(ValueError, match="rank arena 3 holds"):
            B.ar_bucket_allreduce(bp, short)
        with pytest.raises(ValueError, match="rank arena 3 holds"):
            B.ar_bucket_allreduce_after(bp, short)
    finally:
        B.ar_bucket_plan_destroy(bp)
    bq = B.ar_bucket_plan_create(4, 1, sizes, "int8_ef", "ring", 4096)
    try:
        _, arena = B.ar_bucket_layout(bq, len(sizes))
        with pytest.raises(ValueError, match="3 error arenas"):
            B.ar_bucket_allreduce_ef(bq, _fakes(4, arena * 4), _fakes(3, arena * 4))
    finally:
        B.ar_bucket_plan_destroy(bq)


def test_exact_extent_passes_to_c(plan):
    """A list that passes the binding's checks reaches the C checks (here:
    overlapping addresses, which C refuses before any device work)."""
    bufs = [FakeTensor((1 << 30) + 64 * r, 2000, elem=2) for r in range(4)]
    with pytest.raises(B.ArError, match="overlap"):
        B.ar_allreduce(plan, bufs)


@pytest.mark.parametrize("srcs,dsts,nbytes,units,policy", [
    ([], [], 4096, 2, 4),              # one destination per workgroup needs a destination
    ([1 << 30], [2 << 30], 4096, 3, 1),  # 1, 2 or 4 units per thread
    ([1 << 30], [2 << 30], 4096, 2, 3),  # policies 0-2 (+4)
    ([1 << 30], [2 << 30], 4096, 2, 8),
    ([1 << 30], [2 << 30], 4008, 2, 1),  # bytes a multiple of 16
    ([(1 << 30) + 8], [2 << 30], 4096, 2, 1),  # 16-byte aligned buffers
])
def test_probe_arguments_refused(srcs, dsts, nbytes, units, policy):
    """The probe refuses bad arguments before it launches anything."""
    with pytest.raises(B.ArError) as ei:
        B.ar_hbm_probe(srcs, dsts, nbytes, units, policy)
    assert ei.value.status == B.AR_ERR_INVALID_ARG
