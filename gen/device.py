"""Device-side copies of the seeded workloads (inputs only).

Generates canonical tensors with this package's generator and uploads them
with torch; routed experts are loaded into an ``ExpertPool`` of the GPU
library, whose pack kernel re-tiles them. No arithmetic of the method here.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import set_threads
from . import workloads as W


def to_device(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def build_expert_pool(seed, cfg, n_experts, hidden=W.HIDDEN, inter=W.INTER, elo=W.ELO,
                      ehi=W.EHI, device="cuda", workers=8, log=None):
    """ExpertPool holding experts 0..n_experts-1 of (seed, cfg)."""
    import torch
    from mxfp4_packed_weight_amd.pool import ExpertPool
    pool = ExpertPool(n_experts, hidden, inter, device)
    set_threads(1)

    def make(e):
        return W.expert_weights(seed, cfg, e, hidden, inter, elo, ehi)

    with ThreadPoolExecutor(max_workers=workers) as ex:
        for start in range(0, n_experts, workers * 4):
            chunk = list(range(start, min(n_experts, start + workers * 4)))
            for e, E in zip(chunk, ex.map(make, chunk)):
                pool.load(e, E)
            if log and (start // (workers * 4)) % 8 == 0:
                log(f"expert pool: {chunk[-1] + 1}/{n_experts} loaded")
    torch.cuda.synchronize()
    return pool
