"""Helpers of the GPU parity tests (device upload, error metrics)."""
import sys

import numpy as np


def say(msg):
    sys.stdout.write(f"[gpu-case] {msg}\n")
    sys.stdout.flush()


def dev():
    import torch
    return torch.device("cuda:0")


def up(a, dtype=None):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint64:
        a = a.view(np.int64)
    t = torch.from_numpy(a).to(dev())
    return t


def empty(shape, dtype):
    import torch
    return torch.empty(shape, dtype=dtype, device=dev())


def normwise(got, ref):
    """max_i |got_i - ref_i| / max_i |ref_i| (per output vector)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))


TOL = 1e-5
