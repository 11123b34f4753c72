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


def pinned_copy(pool):
    """Pinned host copy of an ExpertPool's packed blobs (the sources of an
    expert cache)."""
    import torch
    host = torch.empty(pool.blob.numel(), dtype=torch.uint8, pin_memory=True)
    host.copy_(pool.blob)
    return host


def make_cache(pool, host, n_slots):
    """An expert cache of n_slots slots whose sources are `host`'s blobs."""
    import mxfp4_packed_weight_amd as K
    c = K.k3_cache_create(pool.n_experts, pool.expert_bytes, n_slots)
    eb = pool.expert_bytes
    for e in range(pool.n_experts):
        K.k3_cache_set_source(c, e, host[e * eb:(e + 1) * eb])
    return c


def layer_outputs(pool, R_d, xd, n, hidden, inter, k, ws):
    """One decode-layer call (k3_moe_layer_ex) on device inputs; its outputs on the host."""
    import torch
    import mxfp4_packed_weight_amd as K
    y = empty(hidden, torch.int16)
    y32 = empty(hidden, torch.float32)
    idx = empty(k, torch.int32)
    w = empty(k, torch.float32)
    lg = empty(n, torch.float64)
    K.k3_moe_layer_ex(xd, R_d, pool.table, n, hidden, inter, k, y, ws, y_f32=y32, idx=idx, w=w,
                      logits=lg)
    return dict(y=y.cpu().numpy().view(np.uint16), y32=y32.cpu().numpy(),
                idx=idx.cpu().numpy(), w=w.cpu().numpy(), logits=lg.cpu().numpy())


def assert_same(a, b):
    """Two layer_outputs results bit for bit."""
    for key in ("y", "idx"):
        assert np.array_equal(a[key], b[key]), key
    for key in ("y32", "w", "logits"):
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), key
