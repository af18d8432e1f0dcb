"""Moving seeded workloads between numpy (oracle side) and the GPU (HIP side)."""
from __future__ import annotations

import numpy as np


def to_dev(a: np.ndarray, device="cuda"):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def to_host(t) -> np.ndarray:
    """Device tensor -> numpy (bf16 as uint16 bit patterns)."""
    import torch
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def widen_dev(t) -> np.ndarray:
    """Device output tensor -> exact fp64 numpy array."""
    from tests._helpers import widen
    return widen(to_host(t))


class DevWorkload:
    """Device copies of one workload's inputs (the pool before the KV append)."""

    def __init__(self, wl, device="cuda"):
        import torch
        self.wl = wl
        self.k_cache = to_dev(wl.k_cache, device)
        self.v_cache = to_dev(wl.v_cache, device)
        self.k_new = to_dev(wl.k_new, device)
        self.v_new = to_dev(wl.v_new, device)
        self.slot_mapping = to_dev(wl.slot_mapping, device)
        self.q = to_dev(wl.q, device)
        self.block_tables = to_dev(wl.block_tables, device)
        self.context_lens = to_dev(wl.context_lens, device)
        self.out = torch.empty_like(self.q)
        if wl.prefill is not None:
            p = wl.prefill
            self.pq = to_dev(p.q, device)
            self.pout = torch.empty_like(self.pq)
            self.p_block_tables = to_dev(p.block_tables, device)
            self.p_context_lens = to_dev(p.context_lens, device)
            self.p_qsl = to_dev(p.query_start_loc, device)
