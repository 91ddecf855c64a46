"""Helpers for the GPU tests: device buffers from numpy and back, and one
all-reduce through the C ABI."""
import numpy as np

from gradient_all_reduce_ar_amd import _binding as B


def storage_view(dtype):
    return np.float32 if dtype == "fp32" else np.int16  # bf16 modes: 16-bit storage


def bits_view(dtype):
    return np.uint32 if dtype == "fp32" else np.uint16


def to_device(xs, dtype):
    import torch

    return [torch.from_numpy(np.ascontiguousarray(x).view(storage_view(dtype))).to("cuda:0") for x in xs]


def to_host_bits(ts, dtype):
    return [t.cpu().numpy().view(bits_view(dtype)) for t in ts]


def gpu_allreduce(xs, dtype, sched, group=1, mode="steps", stream=None, plan=None):
    """Copies xs to the device, runs one all-reduce, returns the result bits."""
    import torch

    bufs = to_device(xs, dtype)
    own = plan is None
    if own:
        plan = B.ar_plan_create(len(xs), group, len(xs[0]), dtype, sched)
        B.ar_plan_set_exec(plan, mode)
    try:
        s = stream or torch.cuda.current_stream()
        B.ar_allreduce(plan, bufs, s)
        torch.cuda.synchronize()
    finally:
        if own:
            B.ar_plan_destroy(plan)
    return to_host_bits(bufs, dtype)
