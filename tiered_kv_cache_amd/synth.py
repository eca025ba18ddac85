"""Seeded synthetic decode workloads: the one input generator both sides use.

This module only draws inputs.  It holds none of the method's arithmetic
(no attention, no importance score, no tier ranking, no quantisation), so the
HIP path and the CPU oracle can share it without sharing any computation.

What it generates follows the workload shapes and the qualitative attention
structure that the summary pages of "Not All Thoughts Need HBM"
(gist.science, paper 2605.09490) describe for reasoning chains:

* every decode step appends one key/value pair per layer and KV head
  (Enonce du probleme);
* attention sinks and a prompt sit at the start of the chain and are kept
  resident (Methodologie section 1, tier T0);
* intermediate results are referenced again, unpredictably, hundreds of
  tokens later (Enonce du probleme; Methodologie section 2) -- modelled by
  "planted" context positions whose keys line up with the query of one
  randomly chosen later decode step.

Recipe (all draws are float32 from numpy's PCG64, one independent stream per
(seed, sequence, kind, index) through ``SeedSequence``; bf16 tensors are the
float32 draws rounded to nearest-even and stored as uint16 bit patterns):

* a unit direction ``u[l, g]`` per layer and KV head;
* query of head h at a step: ``z + a * u[l, g(h)]`` with ``z ~ N(0, I)`` and
  ``g(h) = h // (Hq / Hkv)``;
* context keys ``z``; sink keys ``z + sink_scale * a * u[l, g]``; planted keys
  ``z + plant_sigma * unit(mean over the group's heads of the query at the
  planted step)``; context values and every new decode key/value ``N(0, 1)``.

Unstructured workloads (the tiny fp32 case) use plain ``N(0, 1)`` for all of
q, K and V.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from functools import lru_cache
from typing import Optional, Tuple

import numpy as np

# stream kinds: each (seed, sequence, kind, index) tuple seeds its own PCG64
KIND_DIRECTION = 1
KIND_QUERY = 2
KIND_CTX_K = 3
KIND_CTX_V = 4
KIND_NEW_K = 5
KIND_NEW_V = 6
KIND_PLANT = 7
KIND_LENGTHS = 8


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class Workload:
    """One synthetic decode workload (shapes, policy, seed)."""

    name: str
    description: str
    layers: int
    q_heads: int
    kv_heads: int
    head_dim: int
    dtype: str                      # "bf16" or "f32"
    batch: int
    ctx: Tuple[int, ...]            # initial context length per sequence
    warmup: int                     # untimed decode steps (full cache until the first reassignment)
    steps: int                      # timed decode steps
    prompt: int
    sinks: int
    recent: int
    frac_t1: float
    frac_t2: float
    frac_t3: float
    delta: int
    structured: bool = True
    planted: Tuple[int, ...] = ()   # planted positions per sequence (count)
    q_align: float = 3.0            # a: query offset along u
    sink_scale: float = 8.0         # sink keys: sink_scale * a along u
    plant_sigma: float = 3.0        # planted keys: +plant_sigma along the target query direction
    seed: int = 0

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def total_steps(self) -> int:
        return self.warmup + self.steps

    @property
    def max_ctx(self) -> int:
        return max(self.ctx) + self.total_steps

    def fractions(self) -> Tuple[float, float, float]:
        return (self.frac_t1, self.frac_t2, self.frac_t3)

    def with_fractions(self, f1: float, f2: float, f3: float, suffix: str = "") -> "Workload":
        d = dict(self.__dict__)
        d.update(frac_t1=f1, frac_t2=f2, frac_t3=f3, name=self.name + suffix)
        return Workload(**d)

    def scaled(self, **changes) -> "Workload":
        d = dict(self.__dict__)
        d.update(changes)
        return Workload(**d)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def ragged_lengths(seed: int, batch: int, lo: int, hi: int) -> Tuple[int, ...]:
    """Seeded uniform integer context lengths in [lo, hi]."""
    r = _rng(seed, 0, KIND_LENGTHS, 0)
    return tuple(int(v) for v in r.integers(lo, hi + 1, size=batch))


class SequenceStream:
    """Deterministic generator of one sequence's inputs.

    Any slice (a step's query, a layer's context) can be regenerated on its
    own, so large workloads never need to be materialised whole.
    Step numbers run from 1 to ``warmup + steps``; the token appended at step
    k sits at position ``n0 + k - 1``.
    """

    def __init__(self, wl: Workload, b: int):
        self.wl = wl
        self.b = b
        self.n0 = wl.ctx[b]
        self._dir = None
        self._plant = None

    # ---- helpers -------------------------------------------------------
    def _out(self, x: np.ndarray) -> np.ndarray:
        if self.wl.dtype == "bf16":
            return f32_to_bf16_bits(x)
        return np.ascontiguousarray(x, dtype=np.float32)

    def _as_f32(self, x: np.ndarray) -> np.ndarray:
        return bf16_bits_to_f32(x) if self.wl.dtype == "bf16" else x

    def directions(self) -> np.ndarray:
        """Unit vectors u[l, g] (float32 [L][Hkv][D])."""
        if self._dir is None:
            wl = self.wl
            z = _rng(wl.seed, self.b, KIND_DIRECTION, 0).standard_normal(
                (wl.layers, wl.kv_heads, wl.head_dim), dtype=np.float32)
            self._dir = (z / np.linalg.norm(z, axis=-1, keepdims=True)).astype(np.float32)
        return self._dir

    # ---- planted positions ---------------------------------------------
    def planted(self) -> Tuple[np.ndarray, np.ndarray]:
        """(positions ascending, target step of each) for this sequence."""
        if self._plant is None:
            wl = self.wl
            cnt = wl.planted[self.b] if wl.planted else 0
            lo = max(wl.prompt, wl.sinks)
            hi = self.n0 - wl.recent
            if cnt <= 0 or hi <= lo or wl.steps <= 0:
                self._plant = (np.zeros(0, np.int64), np.zeros(0, np.int64))
            else:
                r = _rng(wl.seed, self.b, KIND_PLANT, 0)
                cnt = min(cnt, hi - lo)
                pos = np.sort(r.choice(np.arange(lo, hi), size=cnt, replace=False))
                tgt = r.integers(wl.warmup + 1, wl.warmup + wl.steps + 1, size=cnt)
                self._plant = (pos.astype(np.int64), tgt.astype(np.int64))
        return self._plant

    # ---- per-step inputs -----------------------------------------------
    def query_f32(self, step: int) -> np.ndarray:
        wl = self.wl
        z = _rng(wl.seed, self.b, KIND_QUERY, step).standard_normal(
            (wl.layers, wl.q_heads, wl.head_dim), dtype=np.float32)
        if wl.structured:
            u = self.directions()
            z = z + np.float32(wl.q_align) * np.repeat(u, wl.group, axis=1)
        return z.astype(np.float32)

    def query(self, step: int) -> np.ndarray:
        """Query of every layer and head at a step: [L][Hq][D] (bf16 bits or f32)."""
        return self._out(self.query_f32(step))

    def new_kv(self, step: int) -> Tuple[np.ndarray, np.ndarray]:
        """Key and value appended at a step: each [L][Hkv][D]."""
        wl = self.wl
        shape = (wl.layers, wl.kv_heads, wl.head_dim)
        k = _rng(wl.seed, self.b, KIND_NEW_K, step).standard_normal(shape, dtype=np.float32)
        v = _rng(wl.seed, self.b, KIND_NEW_V, step).standard_normal(shape, dtype=np.float32)
        return self._out(k), self._out(v)

    # ---- initial context -------------------------------------------------
    def context_layer(self, layer: int) -> Tuple[np.ndarray, np.ndarray]:
        """Context keys and values of one layer: each [Hkv][n0][D]."""
        wl = self.wl
        shape = (wl.kv_heads, self.n0, wl.head_dim)
        k = _rng(wl.seed, self.b, KIND_CTX_K, layer).standard_normal(shape, dtype=np.float32)
        v = _rng(wl.seed, self.b, KIND_CTX_V, layer).standard_normal(shape, dtype=np.float32)
        if wl.structured:
            u = self.directions()[layer]                           # [Hkv][D]
            ns = min(wl.sinks, self.n0)
            k[:, :ns, :] += np.float32(wl.sink_scale * wl.q_align) * u[:, None, :]
            pos, tgt = self.planted()
            for p, t in zip(pos.tolist(), tgt.tolist()):
                q = self._as_f32(self._out(self._query_cached(t)[layer]))   # [Hq][D] as delivered
                qg = q.reshape(wl.kv_heads, wl.group, wl.head_dim).mean(axis=1)
                qg = qg / np.linalg.norm(qg, axis=-1, keepdims=True)
                k[:, p, :] += np.float32(wl.plant_sigma) * qg.astype(np.float32)
        return self._out(k), self._out(v)

    def _query_cached(self, step: int) -> np.ndarray:
        return _query_cache(self.wl, self.b, step)

    def context(self) -> Tuple[np.ndarray, np.ndarray]:
        """Whole initial context: K, V each [L][Hkv][n0][D].  Layers are independent
        streams, generated on a few host threads (NumPy's generators release the GIL)."""
        wl = self.wl
        e = 2 if wl.dtype == "bf16" else 4
        if wl.layers * 2 * wl.kv_heads * self.n0 * wl.head_dim * e < (16 << 20):
            parts = [self.context_layer(l) for l in range(wl.layers)]
        else:
            for t in sorted(set(self.planted()[1].tolist())):
                self._query_cached(t)          # fill the shared cache before the threads
            with ThreadPoolExecutor(max_workers=_host_threads()) as ex:
                parts = list(ex.map(self.context_layer, range(wl.layers)))
        ks, vs = zip(*parts)
        return np.stack(ks), np.stack(vs)


def _host_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


@lru_cache(maxsize=256)
def _query_cache(wl: Workload, b: int, step: int) -> np.ndarray:
    return SequenceStream(wl, b).query_f32(step)


# --------------------------------------------------------------------------
# The five workloads.  Named by what they are; sizes in the names.
# --------------------------------------------------------------------------
_SEED0 = 20261200


def _tiny() -> Workload:
    return Workload(
        name="tiny_L1_h2_d64_f32_ctx256",
        description="1 layer, 2 query heads = 2 KV heads, head_dim 64, fp32 N(0,1) q/K/V, "
                    "context 256 (prompt 32, sinks 4, recent 32), 16 decode steps, delta 4, "
                    "tiers 40/30/20/10",
        layers=1, q_heads=2, kv_heads=2, head_dim=64, dtype="f32", batch=1, ctx=(256,),
        warmup=0, steps=16, prompt=32, sinks=4, recent=32,
        frac_t1=0.30, frac_t2=0.20, frac_t3=0.10, delta=4, structured=False, seed=_SEED0 + 1)


def _small() -> Workload:
    return Workload(
        name="small_L4_h8kv2_d128_bf16_ctx2048",
        description="4 layers, 8 query / 2 KV heads, head_dim 128, bf16, 8 sinks, 64 planted "
                    "positions, context 2048, 64 warm-up + 128 timed steps, tiers 50/30/10/10",
        layers=4, q_heads=8, kv_heads=2, head_dim=128, dtype="bf16", batch=1, ctx=(2048,),
        warmup=64, steps=128, prompt=64, sinks=8, recent=32,
        frac_t1=0.30, frac_t2=0.10, frac_t3=0.10, delta=64, planted=(64,), seed=_SEED0 + 2)


def _chain8k() -> Workload:
    return Workload(
        name="chain8k_L28_h28kv4_d128_bf16_b1",
        description="7B-class reasoning chain: 28 layers, 28 query / 4 KV heads, head_dim 128, "
                    "bf16, 4 sinks, 1% planted resurfacing positions, prompt 256, recent 128, "
                    "context 8192, 64 warm-up + 256 timed steps, batch 1, tiers 50/30/15/5",
        layers=28, q_heads=28, kv_heads=4, head_dim=128, dtype="bf16", batch=1, ctx=(8192,),
        warmup=64, steps=256, prompt=256, sinks=4, recent=128,
        frac_t1=0.30, frac_t2=0.15, frac_t3=0.05, delta=64, planted=(82,), seed=_SEED0 + 3)


def _batch16() -> Workload:
    seed = _SEED0 + 4
    ctx = ragged_lengths(seed, 16, 1024, 8192)
    return Workload(
        name="batch16_L28_h28kv4_d128_bf16_ragged1k-8k",
        description="7B-class shape, batch 16, contexts uniform in [1024, 8192], 64 warm-up + "
                    "64 timed steps, tiers 40/40/15/5, prompt 256, recent 128",
        layers=28, q_heads=28, kv_heads=4, head_dim=128, dtype="bf16", batch=16, ctx=ctx,
        warmup=64, steps=64, prompt=256, sinks=4, recent=128,
        frac_t1=0.40, frac_t2=0.15, frac_t3=0.05, delta=64,
        planted=tuple(max(1, c // 100) for c in ctx), seed=seed)


def _chain32k() -> Workload:
    return Workload(
        name="chain32k_L32_h32kv8_d128_bf16_b4",
        description="long chain: 32 layers, 32 query / 8 KV heads, head_dim 128, bf16, 4 sinks, "
                    "0.5% planted positions, prompt 256, recent 128, context 32768, batch 4, "
                    "64 warm-up + 64 timed steps, tiers 30/50/15/5",
        layers=32, q_heads=32, kv_heads=8, head_dim=128, dtype="bf16", batch=4,
        ctx=(32768,) * 4, warmup=64, steps=64, prompt=256, sinks=4, recent=128,
        frac_t1=0.50, frac_t2=0.15, frac_t3=0.05, delta=64, planted=(164,) * 4,
        seed=_SEED0 + 5)


WORKLOADS = {
    "tiny": _tiny(),
    "small": _small(),
    "chain8k": _chain8k(),
    "batch16": _batch16(),
    "chain32k": _chain32k(),
}
