"""Synthetic workloads on the device: contexts loaded into a TieredKVCache and the
per-step queries and new key/value rows, drawn by the shared seeded generator."""
from __future__ import annotations

from typing import List, Tuple

import numpy as np
import torch

from .driver import PolicyCfg, Shape, TieredKVCache, to_device
from .synth import SequenceStream, Workload


def shape_of(wl: Workload) -> Shape:
    return Shape(wl.layers, wl.q_heads, wl.kv_heads, wl.head_dim, wl.dtype)


def policy_of(wl: Workload) -> PolicyCfg:
    return PolicyCfg(wl.prompt, wl.sinks, wl.recent, wl.frac_t1, wl.frac_t2, wl.frac_t3,
                     wl.delta)


class DeviceWorkload:
    """A workload's inputs, generated on the host and moved to the device."""

    def __init__(self, wl: Workload, device: str = "cuda"):
        self.wl = wl
        self.device = torch.device(device)
        self.streams = [SequenceStream(wl, b) for b in range(wl.batch)]
        self.dtype = shape_of(wl).torch_dtype

    def make_cache(self, contexts=None, per_sequence: bool = False, **kw) -> TieredKVCache:
        """A cache holding every sequence's initial context (regenerated unless
        `contexts`, a list of (K, V) host arrays per sequence, is given).  per_sequence:
        pools sized for each sequence's own longest length (its context plus the
        workload's steps) rather than the longest sequence's."""
        wl = self.wl
        if per_sequence:
            kw["seq_max_ctx"] = [st.n0 + wl.total_steps + 1 for st in self.streams]
        cache = TieredKVCache(shape_of(wl), policy_of(wl), wl.batch, wl.max_ctx,
                              device=str(self.device), **kw)
        for b, st in enumerate(self.streams):
            K, V = contexts[b] if contexts is not None else st.context()
            cache.load_context(b, K, V)
        return cache

    def host_step(self, k: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """Stacked host inputs of decode step k: q [B][L][Hq][D], k/v [B][L][Hkv][D]."""
        qs, ks, vs = [], [], []
        for st in self.streams:
            qs.append(st.query(k))
            kn, vn = st.new_kv(k)
            ks.append(kn)
            vs.append(vn)
        return np.stack(qs), np.stack(ks), np.stack(vs)

    def device_step(self, k: int) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        q, kn, vn = self.host_step(k)
        return (to_device(q, self.dtype, self.device), to_device(kn, self.dtype, self.device),
                to_device(vn, self.dtype, self.device))

    def preload(self, first: int, last: int) -> List[Tuple[torch.Tensor, ...]]:
        """Device inputs of steps first..last (inclusive), resident before timing."""
        return [self.device_step(k) for k in range(first, last + 1)]
