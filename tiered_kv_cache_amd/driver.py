"""Decode state machine of the tiered KV cache on one GPU.

Holds the device state of a batch of sequences and runs the hot path through
libtkv (every arithmetic step is a HIP kernel; torch only allocates device
memory and supplies the stream):

    step:      tkv_append  -> tkv_decode_step (attention over T0 u T1, alpha,
               fused importance-score update)
    every Delta steps (Methodologie section 4 of the "Not All Thoughts Need
    HBM" summary pages, gist.science paper 2605.09490):
               tkv_assign_tiers -> tkv_compact (the new T2 rows quantised, then
               only the rows whose tier changed move, in place) -> one host
               sync for the new lengths.

The T0 pool and the T1 window are single copies whose slot order is not
position order (t0_pos / t1_pos map slots to positions); the read-back helpers
return rows in ascending position order.  The tier map is double-buffered:
the relocation reads the previous map and the new one.

With ``attend_t2`` the 8-bit rows of T2 stay on the device in a pool of their
own and are attended after T1 as code x scale (the variant whose accuracy the
pages report for offloading to T2, Methodologie section 1); each reassignment
then also runs tkv_t2_update, in the same single host sync.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np
import torch

from . import tkv


def _round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


@dataclass
class Shape:
    layers: int
    q_heads: int
    kv_heads: int
    head_dim: int
    dtype: str  # "bf16" | "f32"

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def kv_code(self):
        return tkv.TKV_BF16 if self.dtype == "bf16" else tkv.TKV_F32


@dataclass
class PolicyCfg:
    prompt: int
    sinks: int
    recent: int
    frac_t1: float
    frac_t2: float
    frac_t3: float
    delta: int


def to_device(x: np.ndarray, dtype, device) -> torch.Tensor:
    """Host bf16 bit patterns (uint16) or float32 -> device tensor of `dtype`."""
    if x.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device=device, dtype=dtype, non_blocking=False)


# Storage order of the pools, windows and staging (see csrc/layout.h).  A tensor
# keeps its [..., cap, D] shape as a container; every 32-slot block holds
#   K-tiles: [tile u][D/8 chunks][16 rows][8], slot 8j + 4u + i at row 4j + i;
#   V-tiles: [D/16][4 panels][16 dims][8 slots of the panel].
def k_rows_to_tiles(x: torch.Tensor) -> torch.Tensor:
    *lead, n, d = x.shape
    t = x.reshape(*lead, n // 32, 4, 2, 4, d // 8, 8)        # blk, j, u, i, chunk, e
    k = len(lead)
    t = t.permute(*range(k), k, k + 2, k + 4, k + 1, k + 3, k + 5)  # blk, u, chunk, j, i, e
    return t.contiguous().reshape(*lead, n, d)


def k_tiles_to_rows(x: torch.Tensor, n: int) -> torch.Tensor:
    *lead, cap, d = x.shape
    t = x.reshape(*lead, cap // 32, 2, d // 8, 4, 4, 8)      # blk, u, chunk, j, i, e
    k = len(lead)
    t = t.permute(*range(k), k, k + 3, k + 1, k + 4, k + 2, k + 5)  # blk, j, u, i, chunk, e
    return t.reshape(*lead, cap, d)[..., :n, :]


def v_rows_to_tiles(x: torch.Tensor) -> torch.Tensor:
    *lead, n, d = x.shape
    t = x.reshape(*lead, n // 32, 4, 8, d // 16, 16)         # blk, panel, e, dh, d15
    k = len(lead)
    t = t.permute(*range(k), k, k + 3, k + 1, k + 4, k + 2)  # blk, dh, panel, d15, e
    return t.contiguous().reshape(*lead, n, d)


def v_tiles_to_rows(x: torch.Tensor, n: int) -> torch.Tensor:
    *lead, cap, d = x.shape
    t = x.reshape(*lead, cap // 32, d // 16, 4, 16, 8)       # blk, dh, panel, d15, e
    k = len(lead)
    t = t.permute(*range(k), k, k + 2, k + 4, k + 1, k + 3)  # blk, panel, e, dh, d15
    return t.reshape(*lead, cap, d)[..., :n, :]


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host uint16 bit patterns (bf16) or float32."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class TieredKVCache:
    """Device state of `batch` sequences that decode in lock step."""

    def __init__(self, shape: Shape, policy: PolicyCfg, batch: int, max_ctx: int,
                 device: str = "cuda", cap0: Optional[int] = None, cap1: Optional[int] = None,
                 t2_cap: Optional[int] = None, attend_t2: bool = False, t0_budget: bool = False,
                 alpha_scratch: bool = False, seq_max_ctx: Optional[List[int]] = None):
        """t0_budget: after the first reassignment, move the T0 pool into one sized by the
        tier budget (tkv_t0_capacity) instead of the whole context.  alpha_scratch: the
        decode calls keep the weights only as the score update's input (alpha holds the
        raw logits afterwards; alpha_of is unavailable).  seq_max_ctx: the longest each
        sequence gets; the T0 pool and the T1 window then give every sequence its own
        capacity (tkv_model.t0_caps / t1_caps, blocks packed sequence after sequence)
        instead of the longest sequence's."""
        self.shape = shape
        self.t0_budget = t0_budget
        self.host_t1 = False       # set by T1Stream: T1 rows live in host memory
        self.reassignments = 0
        self.policy = policy
        self.batch = batch
        self.device = torch.device(device)
        self.max_ctx = _round_up(max_ctx, 64)
        self.cap0 = _round_up(cap0 or self.max_ctx, 64)   # multiples of 32 (tile blocks)
        self.cap1 = _round_up(cap1 if cap1 is not None
                              else int(math.floor(float(np.float32(policy.frac_t1)) * self.max_ctx)) + 64, 64)
        self.t2_cap = _round_up(t2_cap if t2_cap is not None
                                else int(math.floor(float(np.float32(policy.frac_t2)) * self.max_ctx)) + 64, 64)
        self.attend_t2 = attend_t2
        # per-sequence capacities: each sequence's own context bound, and the T1 budget at it
        self.ragged = seq_max_ctx is not None
        if self.ragged:
            if len(seq_max_ctx) != batch:
                raise ValueError("seq_max_ctx needs one bound per sequence")
            f1 = float(np.float32(policy.frac_t1))
            self.seq_max = [_round_up(min(int(x), self.max_ctx), 64) for x in seq_max_ctx]
            self.caps0 = list(self.seq_max)
            self.caps1 = [_round_up(int(math.floor(f1 * x)) + 64, 64) for x in self.seq_max]
            self.cap0 = max(self.caps0)
            self.cap1 = max(self.caps1)
        else:
            self.seq_max = [self.max_ctx] * batch
            self.caps0 = [self.cap0] * batch
            self.caps1 = [self.cap1] * batch
        # the attended T2 pool holds at most as many rows as one reassignment can quantise
        self.cap2 = self.t2_cap if attend_t2 else 0
        self.alpha_stride = _round_up(self.cap0 + self.cap1 + self.cap2, 64)
        self.alpha_scratch = alpha_scratch
        self.model = tkv.make_model(shape.layers, shape.q_heads, shape.kv_heads, shape.head_dim,
                                    shape.kv_code, alpha_scratch=alpha_scratch,
                                    t0_caps=self.caps0 if self.ragged else None,
                                    t1_caps=self.caps1 if self.ragged else None)
        self.tpolicy = tkv.make_policy(policy.prompt, policy.sinks, policy.recent,
                                       policy.frac_t1, policy.frac_t2, policy.frac_t3,
                                       policy.delta)
        L, Hq, Hkv, D = shape.layers, shape.q_heads, shape.kv_heads, shape.head_dim
        dt, dev, B = shape.torch_dtype, self.device, batch
        self.k_t0, self.v_t0 = self._pool(self.caps0), self._pool(self.caps0)
        self.k_t1, self.v_t1 = self._pool(self.caps1), self._pool(self.caps1)
        self.t0_pos = torch.zeros((B, self.cap0), dtype=torch.int32, device=dev)
        self.t1_pos = torch.zeros((B, self.cap1), dtype=torch.int32, device=dev)
        self.tier = [torch.zeros((B, self.max_ctx), dtype=torch.uint8, device=dev) for _ in range(2)]
        self.scores = torch.zeros((B, self.max_ctx), dtype=torch.float32, device=dev)
        self.alpha = torch.zeros((B, L, Hq, self.alpha_stride), dtype=torch.float32, device=dev)
        self.out = torch.zeros((B, L, Hq, D), dtype=torch.float32, device=dev)
        self.counts = torch.zeros((B, 4), dtype=torch.int32, device=dev)
        self.new_lens = torch.zeros((B, 4), dtype=torch.int32, device=dev)
        self.t2_src = torch.zeros((B, self.t2_cap), dtype=torch.int32, device=dev)
        self.t2_pos = torch.zeros((B, self.t2_cap), dtype=torch.int32, device=dev)
        self.t2_codes = torch.zeros((B, self.t2_cap, L, Hkv, 2, D), dtype=torch.int8, device=dev)
        self.t2_scales = torch.zeros((B, self.t2_cap, L, Hkv, 2), dtype=torch.float32, device=dev)
        if attend_t2:
            pool2 = (B, L, Hkv, self.cap2, D)
            self.k_t2 = torch.zeros(pool2, dtype=torch.int8, device=dev)
            self.v_t2 = torch.zeros(pool2, dtype=torch.int8, device=dev)
            self.ks_t2 = torch.zeros(pool2[:-1], dtype=torch.float32, device=dev)
            self.vs_t2 = torch.zeros(pool2[:-1], dtype=torch.float32, device=dev)
            self.t2_slot_pos = torch.zeros((B, self.cap2), dtype=torch.int32, device=dev)
            self.t2_lens_dev = torch.zeros((B, 2), dtype=torch.int32, device=dev)
            self.t2ws_bytes = tkv.tkv_t2_update_workspace_bytes(B, self.cap2)
            self.t2ws = torch.zeros(self.t2ws_bytes, dtype=torch.uint8, device=dev)
        self.ws_bytes = tkv.tkv_decode_workspace_bytes(self.model, B, L, self.cap0,
                                                       self.cap1 + self.cap2)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.cws_bytes = tkv.tkv_compact_workspace_bytes(self.model, B, self.max_ctx, self.cap0,
                                                         self.cap1)
        self.cws = torch.zeros(self.cws_bytes, dtype=torch.uint8, device=dev)
        self.tcur = 0      # which tier map is live
        self.n = [0] * B
        self.t0_len = [0] * B
        self.t1_len = [0] * B
        self.t2_len = [0] * B   # rows in the attended T2 pool
        self.t2_new = [0] * B   # rows quantised at the last reassignment
        self.moved = [0] * B    # row copies of the last relocation
        self.steps = 0
        self.fused_scores = True
        self.fused_append = True   # step(): tkv_append_decode_step rather than the two calls

    # ---- pools ---------------------------------------------------------------
    def _pool(self, caps: List[int]) -> torch.Tensor:
        """A pool of K or V rows: [B][L][Hkv][cap][D] tiles, or with per-sequence
        capacities one flat buffer of the sequences' [L][Hkv][cap_b][D] blocks in order."""
        sh = self.shape
        L, Hkv, D = sh.layers, sh.kv_heads, sh.head_dim
        if not self.ragged:
            return torch.zeros((self.batch, L, Hkv, caps[0], D), dtype=sh.torch_dtype,
                               device=self.device)
        return torch.zeros(sum(caps) * L * Hkv * D, dtype=sh.torch_dtype, device=self.device)

    def block(self, pool: torch.Tensor, caps: List[int], b: int) -> torch.Tensor:
        """Sequence b's [L][Hkv][cap_b][D] block of a pool."""
        if not self.ragged:
            return pool[b]
        sh = self.shape
        per = sh.layers * sh.kv_heads * sh.head_dim
        o = sum(caps[:b]) * per
        return pool[o:o + caps[b] * per].view(sh.layers, sh.kv_heads, caps[b], sh.head_dim)

    # ---- views -------------------------------------------------------------
    @property
    def tiers(self):
        return self.tier[self.tcur]

    def t2_pool(self):
        """The attended T2 pool as the C ABI sees it (None unless attend_t2)."""
        if not self.attend_t2:
            return None
        return tkv.T2Pool(self.k_t2, self.v_t2, self.ks_t2, self.vs_t2, self.t2_slot_pos,
                          self.t2_len, self.cap2)

    # ---- set-up ------------------------------------------------------------
    def load_context(self, b: int, K: np.ndarray, V: np.ndarray) -> None:
        """Initial context of sequence b (all in T0, scores 0): K, V [L][Hkv][n0][D]."""
        n0 = K.shape[2]
        n0p = (n0 + 31) // 32 * 32
        if n0p > self.caps0[b]:
            raise ValueError("context longer than the T0 pool")
        shape = (K.shape[0], K.shape[1], n0p, K.shape[3])
        kpad = torch.zeros(shape, dtype=self.shape.torch_dtype, device=self.device)
        vpad = torch.zeros(shape, dtype=self.shape.torch_dtype, device=self.device)
        kpad[:, :, :n0] = to_device(K, self.shape.torch_dtype, self.device)
        vpad[:, :, :n0] = to_device(V, self.shape.torch_dtype, self.device)
        self.block(self.k_t0, self.caps0, b)[:, :, :n0p] = k_rows_to_tiles(kpad)
        self.block(self.v_t0, self.caps0, b)[:, :, :n0p] = v_rows_to_tiles(vpad)
        self.t0_pos[b, :n0] = torch.arange(n0, dtype=torch.int32, device=self.device)
        self.tier[self.tcur][b].zero_()
        self.scores[b].zero_()
        self.n[b] = n0
        self.t0_len[b] = n0
        self.t1_len[b] = 0
        self.t2_len[b] = 0

    # ---- the step ------------------------------------------------------------
    def append(self, k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> None:
        tkv.tkv_append(self.model, self.batch, k_new, v_new, self.k_t0, self.v_t0, self.cap0,
                       self.t0_len, self.t0_pos, self.n, self.scores, self.tiers, self.max_ctx,
                       stream)
        self.n = [x + 1 for x in self.n]
        self.t0_len = [x + 1 for x in self.t0_len]

    def attend(self, q: torch.Tensor, stream=None, layer_begin: int = 0,
               layer_end: Optional[int] = None, fused_scores: Optional[bool] = None,
               out: Optional[torch.Tensor] = None, alpha: Optional[torch.Tensor] = None) -> None:
        """Attention of layers [layer_begin, layer_end) (default all) over T0 u T1.

        A layer subset needs contiguous `out` [B][Lr][Hq][D] and `alpha`
        [B][Lr][Hq][alpha_stride] buffers from the caller.
        """
        le = self.shape.layers if layer_end is None else layer_end
        fused = self.fused_scores if fused_scores is None else fused_scores
        full = layer_begin == 0 and le == self.shape.layers
        if out is None or alpha is None:
            if not full:
                raise ValueError("a layer subset needs caller-supplied out and alpha buffers")
            out, alpha = self.out, self.alpha
        if self.attend_t2:
            if not fused:
                raise ValueError("attended T2 rows need the fused score update")
            tkv.tkv_decode_step_t2(self.model, self.batch, layer_begin, le, q, self.k_t0,
                                   self.v_t0, self.t0_len, self.cap0, self.k_t1, self.v_t1,
                                   self.t1_len, self.cap1, self.t2_pool(), out, alpha,
                                   self.alpha_stride, self.t0_pos, self.t1_pos, self.scores,
                                   self.max_ctx, self.ws, self.ws_bytes, stream)
            return
        tkv.tkv_decode_step(self.model, self.batch, layer_begin, le, q, self.k_t0, self.v_t0,
                            self.t0_len, self.cap0, self.k_t1, self.v_t1, self.t1_len, self.cap1,
                            out, alpha, self.alpha_stride, self.t0_pos, self.t1_pos,
                            self.scores if fused else None, self.max_ctx, self.ws, self.ws_bytes,
                            stream)
        if not fused:
            tkv.tkv_update_scores(self.model, self.batch, layer_begin, le, alpha,
                                  self.alpha_stride, self.t0_pos, self.t0_len, self.cap0,
                                  self.t1_pos, self.t1_len, self.cap1, self.scores,
                                  self.max_ctx, stream)

    def append_attend(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                      stream=None) -> None:
        """append() then attend() over all layers, as one pass (tkv_append_decode_step)."""
        if not self.fused_scores:
            self.append(k_new, v_new, stream)
            self.attend(q, stream)
            return
        if self.attend_t2:
            tkv.tkv_append_decode_step_t2(self.model, self.batch, k_new, v_new, self.n,
                                          self.tiers, q, self.k_t0, self.v_t0, self.t0_len,
                                          self.cap0, self.k_t1, self.v_t1, self.t1_len,
                                          self.cap1, self.t2_pool(), self.out, self.alpha,
                                          self.alpha_stride, self.t0_pos, self.t1_pos,
                                          self.scores, self.max_ctx, self.ws, self.ws_bytes,
                                          stream)
            self.n = [x + 1 for x in self.n]
            self.t0_len = [x + 1 for x in self.t0_len]
            return
        tkv.tkv_append_decode_step(self.model, self.batch, k_new, v_new, self.n, self.tiers, q,
                                   self.k_t0, self.v_t0, self.t0_len, self.cap0, self.k_t1,
                                   self.v_t1, self.t1_len, self.cap1, self.out, self.alpha,
                                   self.alpha_stride, self.t0_pos, self.t1_pos, self.scores,
                                   self.max_ctx, self.ws, self.ws_bytes, stream)
        self.n = [x + 1 for x in self.n]
        self.t0_len = [x + 1 for x in self.t0_len]

    def step(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, stream=None,
             reassign: bool = True) -> bool:
        """One decode step; returns True when it ended with a reassignment."""
        if self.fused_append:
            self.append_attend(q, k_new, v_new, stream)
        else:
            self.append(k_new, v_new, stream)
            self.attend(q, stream)
        self.steps += 1
        if reassign and self.steps % self.policy.delta == 0:
            self.reassign(stream)
            return True
        return False

    def reassign(self, stream=None) -> None:
        """Rank, quantise the new T2 rows, relocate in place; one host sync for the new lengths."""
        if self.host_t1:
            raise RuntimeError("T1 rows live in host memory: reassign through T1Stream")
        tnx = 1 - self.tcur
        B = self.batch
        tkv.tkv_assign_tiers(B, self.n, self.max_ctx, self.scores, self.tpolicy,
                             self.tier[self.tcur], self.tier[tnx], self.counts, stream)
        tkv.tkv_compact(self.model, B, self.n, self.max_ctx, self.tier[self.tcur], self.tier[tnx],
                        self.k_t0, self.v_t0, self.t0_pos, self.t0_len, self.cap0,
                        self.k_t1, self.v_t1, self.t1_pos, self.t1_len, self.cap1,
                        self.t2_src, self.t2_pos, self.t2_cap, self.t2_codes, self.t2_scales,
                        self.new_lens, self.cws, self.cws_bytes, stream)
        if self.attend_t2:
            tkv.tkv_t2_update(self.model, B, self.n, self.max_ctx, self.tier[tnx], self.k_t2,
                              self.v_t2, self.ks_t2, self.vs_t2, self.t2_slot_pos, self.t2_len,
                              self.cap2, self.t2_pos, self.t2_codes, self.t2_scales,
                              self.new_lens[:, 2:], 4, self.t2_cap, self.t2_lens_dev, self.t2ws,
                              self.t2ws_bytes, stream)
            both = torch.cat([self.new_lens, self.t2_lens_dev], dim=1).cpu().numpy()
            lens, t2l = both[:, :4], both[:, 4:]    # the one sync per reassignment
            if (t2l < 0).any():
                raise RuntimeError(f"T2 pool state error reported by the device: {t2l.tolist()}")
            self.t2_len = t2l[:, 0].tolist()
        else:
            lens = self.new_lens.cpu().numpy()      # the one sync per reassignment
        self.finish_reassign(lens, tnx)

    def finish_reassign(self, lens: np.ndarray, tnx: int) -> None:
        """New lengths of a reassignment; the T0 pool moves to its budget after the first."""
        if (lens < 0).any():
            raise RuntimeError(f"tier state error reported by the device: {lens.tolist()}")
        self.t0_len = lens[:, 0].tolist()
        self.t1_len = lens[:, 1].tolist()
        self.t2_new = lens[:, 2].tolist()
        self.moved = lens[:, 3].tolist()
        self.tcur = tnx
        self.reassignments += 1
        if self.t0_budget and self.reassignments == 1:
            if self.ragged:
                caps = [min(c, tkv.tkv_t0_capacity(self.tpolicy, n, m))
                        for c, n, m in zip(self.caps0, self.n, self.seq_max)]
                if caps != self.caps0:
                    self.resize_t0(caps)
            else:
                cap = tkv.tkv_t0_capacity(self.tpolicy, min(self.n), self.max_ctx)
                if cap < self.cap0:
                    self.resize_t0([cap] * self.batch)

    def resize_t0(self, caps0: List[int]) -> None:
        """Move the T0 pool into one of per-sequence capacities caps0 (multiples of 32
        that hold every current row; one value for every sequence unless the cache has
        per-sequence capacities): slots [0, t0_len) keep their rows; the weights, the
        decode and the relocation workspaces follow the new capacity."""
        if not self.ragged and len(set(caps0)) != 1:
            raise ValueError("one T0 capacity for every sequence")
        for c, n in zip(caps0, self.t0_len):
            if c % 32 or c < _round_up(n, 32):
                raise ValueError("each new T0 capacity must be a multiple of 32 holding its rows")
        torch.cuda.synchronize(self.device)
        B, L = self.batch, self.shape.layers
        old_k, old_v, old_caps = self.k_t0, self.v_t0, self.caps0
        self.caps0 = list(caps0)
        k, v = self._pool(self.caps0), self._pool(self.caps0)
        cap0 = max(self.caps0)
        pos = torch.zeros((B, cap0), dtype=torch.int32, device=self.device)
        for b in range(B):
            m = min(old_caps[b], _round_up(self.t0_len[b], 32))   # whole 32-slot blocks
            self.block(k, self.caps0, b)[:, :, :m] = self.block(old_k, old_caps, b)[:, :, :m]
            self.block(v, self.caps0, b)[:, :, :m] = self.block(old_v, old_caps, b)[:, :, :m]
            pos[b, :m] = self.t0_pos[b, :m]
        del old_k, old_v
        self.k_t0, self.v_t0, self.t0_pos = k, v, pos
        self.cap0 = cap0
        tkv.set_caps(self.model, self.caps0 if self.ragged else None,
                     self.caps1 if self.ragged else None)
        self.alpha_stride = _round_up(self.cap0 + self.cap1 + self.cap2, 64)
        self.alpha = torch.zeros((B, L, self.shape.q_heads, self.alpha_stride),
                                 dtype=torch.float32, device=self.device)
        self.ws_bytes = tkv.tkv_decode_workspace_bytes(self.model, B, L, self.cap0,
                                                       self.cap1 + self.cap2)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self.alloc_compact_workspace()
        torch.cuda.synchronize(self.device)

    def alloc_compact_workspace(self) -> None:
        if self.host_t1:
            self.cws_bytes = tkv.tkv_compact_host_t1_workspace_bytes(
                self.model, self.batch, self.max_ctx, self.cap0, self.cap1)
        else:
            self.cws_bytes = tkv.tkv_compact_workspace_bytes(self.model, self.batch, self.max_ctx,
                                                             self.cap0, self.cap1)
        self.cws = torch.zeros(self.cws_bytes, dtype=torch.uint8, device=self.device)

    def resident_kv_bytes(self) -> int:
        """Device bytes that hold key/value rows: the T0 pool, the T1 window (when it is
        on the device) and the attended int8 T2 pool."""
        t = [self.k_t0, self.v_t0, self.k_t1, self.v_t1]
        if self.attend_t2:
            t += [self.k_t2, self.v_t2, self.ks_t2, self.vs_t2]
        return sum(x.numel() * x.element_size() for x in t if x is not None)

    def full_cache_bytes(self) -> int:
        """Bytes of every sequence's K/V rows at its current length (a full cache)."""
        sh = self.shape
        e = 2 if sh.dtype == "bf16" else 4
        return sum(self.n) * sh.layers * sh.kv_heads * sh.head_dim * e * 2

    # ---- read-back helpers (tests, tools): ascending position order -------------
    def _order(self, b: int):
        """Slot orders of the pool and the window that sort their positions."""
        p0 = self.t0_pos[b, :self.t0_len[b]].cpu().numpy()
        p1 = self.t1_pos[b, :self.t1_len[b]].cpu().numpy()
        return np.argsort(p0, kind="stable"), np.argsort(p1, kind="stable"), p0, p1

    def t0_positions(self, b: int) -> np.ndarray:
        o0, _, p0, _ = self._order(b)
        return p0[o0].astype(np.int64)

    def t1_positions(self, b: int) -> np.ndarray:
        _, o1, _, p1 = self._order(b)
        return p1[o1].astype(np.int64)

    def t2_order(self, b: int):
        """Slot order of the attended T2 pool that sorts its positions, and the positions."""
        if not self.attend_t2 or self.t2_len[b] == 0:
            return np.zeros(0, dtype=np.int64), np.zeros(0, dtype=np.int64)
        p2 = self.t2_slot_pos[b, :self.t2_len[b]].cpu().numpy()
        return np.argsort(p2, kind="stable"), p2

    def t2_positions(self, b: int) -> np.ndarray:
        o2, p2 = self.t2_order(b)
        return p2[o2].astype(np.int64)

    def attended_positions(self, b: int) -> np.ndarray:
        """T0 positions, then T1 positions, then attended T2 positions, each ascending."""
        o0, o1, p0, p1 = self._order(b)
        o2, p2 = self.t2_order(b)
        return np.concatenate([p0[o0], p1[o1], p2[o2]]).astype(np.int64)

    def t0_rows(self, b: int):
        """Host copies (bf16 bits or float32) of the T0 rows of sequence b in ascending
        position order: K, V [L][Hkv][n][D]."""
        o0 = self._order(b)[0]
        n = self.t0_len[b]
        return (to_host_bits(k_tiles_to_rows(self.block(self.k_t0, self.caps0, b), n))[:, :, o0],
                to_host_bits(v_tiles_to_rows(self.block(self.v_t0, self.caps0, b), n))[:, :, o0])

    def t1_rows(self, b: int):
        """Host copies of the T1 rows of sequence b in ascending position order."""
        o1 = self._order(b)[1]
        n = self.t1_len[b]
        return (to_host_bits(k_tiles_to_rows(self.block(self.k_t1, self.caps1, b), n))[:, :, o1],
                to_host_bits(v_tiles_to_rows(self.block(self.v_t1, self.caps1, b), n))[:, :, o1])

    def alpha_of(self, b: int) -> np.ndarray:
        """alpha [L][Hq][n_att] in attended_positions() order."""
        if self.alpha_scratch:
            raise RuntimeError("alpha_scratch: the decode calls store no weights")
        o0, o1, _, _ = self._order(b)
        o2, _ = self.t2_order(b)
        n01 = self.t0_len[b] + self.t1_len[b]
        m = n01 + len(o2)
        a = self.alpha[b, :, :, :m].cpu().numpy()
        return a[:, :, np.concatenate([o0, self.t0_len[b] + o1, n01 + o2]).astype(np.int64)]

    def t2_pool_rows(self, b: int):
        """Attended T2 rows of sequence b in ascending position order: codes
        [L][Hkv][n2][D] int8 for K and V, and scales [L][Hkv][n2] for K and V."""
        o2, _ = self.t2_order(b)
        n = self.t2_len[b]
        kc = k_tiles_to_rows(self.k_t2[b], n).cpu().numpy()[:, :, o2]
        vc = v_tiles_to_rows(self.v_t2[b], n).cpu().numpy()[:, :, o2]
        ks = self.ks_t2[b, :, :, :n].cpu().numpy()[:, :, o2]
        vs = self.vs_t2[b, :, :, :n].cpu().numpy()[:, :, o2]
        return kc, vc, ks, vs

    def last_t2(self, b: int):
        r = self.t2_new[b]
        return (self.t2_pos[b, :r].cpu().numpy(), self.t2_codes[b, :r].cpu().numpy(),
                self.t2_scales[b, :r].cpu().numpy())


class T1Stream:
    """T1 rows in host memory, streamed to the device chunk of layers by chunk of layers
    (Methodologie section 1 of the pages: T1 stays in host DDR at full precision and is
    brought to the GPU before each attention step; section 4: tiers change every Delta
    steps and only the newly promoted tokens go from host memory to the GPU).

    Host memory holds a store of full-precision rows by position [B][L][Hkv][max_ctx][D]
    and the streamed window [B][L][Hkv][2][cap1][D] (pinned, tiles, window-slot order).
    The device holds the T0 pool and a two-buffer window of chunk_layers layers
    [2][B][chunk][Hkv][2][cap1][D]; the cache's own T1 window is released.

    Every step (tkv_decode_step_streamed): the live 32-slot blocks of every layer's T1
    rows cross the link while the previous chunk attends.  Every Delta steps
    (tkv_assign_tiers, tkv_compact_host_t1): only the rows that enter T1 from T0 go to the
    host store and only the rows that leave T1 (for T0 or T2) come back; the window slots
    whose position changed are rewritten on the host.  `link_step` / `link_reassign` count
    the bytes that crossed the link.
    """

    def __init__(self, cache: TieredKVCache, chunk_layers: int = 1):
        if cache.attend_t2:
            raise ValueError("the streamed T1 window is built for the T0 u T1 step")
        if any(cache.t1_len):
            raise ValueError("T1 must be empty when its rows move to host memory")
        self.cache = cache
        sh = cache.shape
        B, L, Hkv, D = cache.batch, sh.layers, sh.kv_heads, sh.head_dim
        dt, dev = sh.torch_dtype, cache.device
        self.chunk = max(1, min(chunk_layers, L))
        self.store_k = torch.empty((B, L, Hkv, cache.max_ctx, D), dtype=dt)
        self.store_v = torch.empty((B, L, Hkv, cache.max_ctx, D), dtype=dt)
        self.t1_host = torch.empty((B, L, Hkv, 2, cache.cap1, D), dtype=dt, pin_memory=True)
        self.t1_host.zero_()
        self.win = torch.zeros((2, B, self.chunk, Hkv, 2, cache.cap1, D), dtype=dt, device=dev)
        self.scratch_bytes = tkv.tkv_compact_host_t1_scratch_bytes(cache.model, B, cache.max_ctx,
                                                                   cache.cap1)
        self.scratch = torch.empty(self.scratch_bytes, dtype=torch.uint8, pin_memory=True)
        self.side = torch.cuda.Stream(device=dev)
        self.side2 = torch.cuda.Stream(device=dev)   # chunks alternate between the two
        self.events = [torch.cuda.Event() for _ in range(4)]
        main = torch.cuda.current_stream(dev)
        for e in self.events:        # creates the underlying events
            e.record(main)
        # the device no longer holds T1 rows, nor a staging area for them
        cache.host_t1 = True
        cache.k_t1 = cache.v_t1 = None
        cache.alloc_compact_workspace()
        self.link_step = 0
        self.link_reassign: List[int] = []

    def window_bytes(self) -> int:
        """Device bytes of the two-buffer chunk window."""
        return self.win.numel() * self.win.element_size()

    def resident_kv_bytes(self) -> int:
        """Device bytes that hold key/value rows: the T0 pool and the chunk window."""
        return self.cache.resident_kv_bytes() + self.window_bytes()

    def link_bytes_per_step(self) -> int:
        """Bytes the last step sent over the host link."""
        return self.link_step

    def reassign(self) -> None:
        """Tier reassignment with the T1 rows in host memory (one host-synchronous call)."""
        c = self.cache
        tnx = 1 - c.tcur
        tkv.tkv_assign_tiers(c.batch, c.n, c.max_ctx, c.scores, c.tpolicy, c.tier[c.tcur],
                             c.tier[tnx], c.counts)
        lens, link = tkv.tkv_compact_host_t1(
            c.model, c.batch, c.n, c.max_ctx, c.tier[c.tcur], c.tier[tnx], c.k_t0, c.v_t0,
            c.t0_pos, c.t0_len, c.cap0, c.t1_pos, c.t1_len, c.cap1, self.store_k, self.store_v,
            self.t1_host, c.t2_src, c.t2_pos, c.t2_cap, c.t2_codes, c.t2_scales, c.new_lens,
            c.cws, c.cws_bytes, self.scratch, self.scratch_bytes)
        self.link_reassign.append(link)
        c.finish_reassign(lens, tnx)

    def t1_rows(self, b: int):
        """Host copies of the T1 rows of sequence b in ascending position order."""
        o1 = self.cache._order(b)[1]
        n = self.cache.t1_len[b]
        k = k_tiles_to_rows(self.t1_host[b, :, :, 0], n)
        v = v_tiles_to_rows(self.t1_host[b, :, :, 1], n)
        return to_host_bits(k)[:, :, o1], to_host_bits(v)[:, :, o1]

    def attend(self, q: torch.Tensor) -> None:
        """Attention of every layer over T0 and the streamed T1 rows, with the score update;
        outputs land in the cache's `out` and `alpha` as with TieredKVCache.attend."""
        c = self.cache
        self.link_step = tkv.tkv_decode_step_streamed(
            c.model, c.batch, q, c.k_t0, c.v_t0, c.t0_len, c.cap0, self.t1_host, c.t1_len,
            c.cap1, self.win, self.chunk, c.out, c.alpha, c.alpha_stride, c.t0_pos, c.t1_pos,
            c.scores, c.max_ctx, c.ws, c.ws_bytes, torch.cuda.current_stream(c.device), self.side,
            self.events, side_stream2=self.side2)

    def step(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
             reassign: bool = True) -> bool:
        """One decode step with streamed T1 rows; returns True when it ended with a
        reassignment."""
        c = self.cache
        c.append(k_new, v_new)
        self.attend(q)
        c.steps += 1
        if reassign and c.steps % c.policy.delta == 0:
            self.reassign()
            return True
        return False
