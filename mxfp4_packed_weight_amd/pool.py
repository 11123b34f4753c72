"""Device-resident pool of packed routed experts.

Holds n_experts expert blobs (layout of k3_expert_pack) in one device
allocation plus the device table of per-expert pointers that k3_moe_layer
takes. Loading an expert uploads its canonical MXFP4 bytes to a staging
buffer and re-tiles them on the device with k3_expert_pack (the one-time
re-tiling; the hot path only reads the packed pool).
"""
import numpy as np

from . import k3_expert_pack, k3_expert_packed_bytes


class ExpertPool:
    def __init__(self, n_experts, hidden, inter, device="cuda"):
        import torch
        self.n_experts, self.hidden, self.inter = n_experts, hidden, inter
        self.expert_bytes = k3_expert_packed_bytes(hidden, inter)
        if self.expert_bytes == 0:
            raise ValueError(f"unsupported expert shape hidden={hidden} inter={inter}")
        self.device = torch.device(device)
        self.blob = torch.empty(n_experts * self.expert_bytes, dtype=torch.uint8,
                                device=self.device)
        base = self.blob.data_ptr()
        ptrs = np.array([base + e * self.expert_bytes for e in range(n_experts)], np.uint64)
        self.table = torch.from_numpy(ptrs.view(np.int64)).to(self.device)
        self._stage = None

    def expert_view(self, e):
        return self.blob[e * self.expert_bytes:(e + 1) * self.expert_bytes]

    def load(self, e, E, stream=None):
        """Upload canonical expert E (dict gate/up/down -> (nib, sc)) into slot e."""
        import torch
        parts = [E["gate"][0], E["gate"][1], E["up"][0], E["up"][1], E["down"][0], E["down"][1]]
        sizes = [int(np.asarray(p).nbytes) for p in parts]
        offs = np.cumsum([0] + [(s + 255) // 256 * 256 for s in sizes])
        if self._stage is None or self._stage.numel() < offs[-1]:
            self._stage = torch.empty(int(offs[-1]), dtype=torch.uint8, device=self.device)
        host = np.zeros(int(offs[-1]), np.uint8)
        for p, o, s in zip(parts, offs, sizes):
            host[o:o + s] = np.ascontiguousarray(p, np.uint8).ravel()
        self._stage[:host.size].copy_(torch.from_numpy(host))
        views = [self._stage[int(o):int(o) + s] for o, s in zip(offs, sizes)]
        k3_expert_pack(*views, self.hidden, self.inter, self.expert_view(e), stream)
