"""The HBM probe (ar_hbm_probe) computes what it states: every 16-byte unit
of each destination is the fp32 sum, in source order from 0, of that unit of
the sources, over exactly `bytes` of each buffer, in both store layouts
(each workgroup into every destination, or into one), for every shape and
cache policy.  The bench's ceilings rest on it moving the bytes it claims."""
import sys

import numpy as np
import pytest

from gradient_all_reduce_ar_amd import _binding as B

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _expected(srcs):
    acc = np.zeros_like(srcs[0]) if srcs else None
    for x in srcs:
        acc = (acc + x).astype(np.float32)
    return acc


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("nsrc,ndst", [(0, 1), (1, 1), (2, 1), (0, 5), (3, 4), (9, 2), (16, 16)])
def test_probe_results(nsrc, ndst, split):
    import torch

    if split and ndst == 0:
        pytest.skip("the split layout needs a destination")
    count = 3 * 1024 + 260  # floats: ragged against every tile (256 threads x 1, 2, 4 units)
    nbytes = (count - 4) * 4  # the last unit of every buffer stays outside
    rng = np.random.default_rng(nsrc * 31 + ndst)
    srcs = [rng.standard_normal(count).astype(np.float32) for _ in range(nsrc)]
    want = _expected([x[:count - 4] for x in srcs]) if nsrc else np.zeros(count - 4, np.float32)
    dsrc = [torch.from_numpy(x).to("cuda:0") for x in srcs]
    for units in (1, 2, 4):
        for policy in (0, 1, 2):
            _say(f"case probe nsrc={nsrc} ndst={ndst} split={split} units={units} policy={policy}")
            ddst = [torch.full((count,), 7.0, device="cuda:0") for _ in range(ndst)]
            B.ar_hbm_probe(dsrc, ddst, nbytes, units, policy | (4 if split else 0), torch.cuda.current_stream())
            torch.cuda.synchronize()
            for d in ddst:
                got = d.cpu().numpy()
                assert np.array_equal(got[:count - 4].view(np.uint32), want.view(np.uint32))
                assert np.all(got[count - 4:] == 7.0)
            for x, dx in zip(srcs, dsrc):
                assert np.array_equal(dx.cpu().numpy(), x)


def test_probe_in_place():
    """Destinations equal to sources (the fold mix on the rank buffers)."""
    import torch

    n, count = 4, 2048 + 64
    rng = np.random.default_rng(5)
    xs = [rng.standard_normal(count).astype(np.float32) for _ in range(n)]
    want = _expected(xs)
    for split in (False, True):
        bufs = [torch.from_numpy(x).to("cuda:0") for x in xs]
        B.ar_hbm_probe(bufs, bufs, count * 4, 2, 2 | (4 if split else 0), torch.cuda.current_stream())
        torch.cuda.synchronize()
        if not split:  # each workgroup reads all its sources before it stores
            for b in bufs:
                assert np.array_equal(b.cpu().numpy().view(np.uint32), want.view(np.uint32))
