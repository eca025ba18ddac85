"""CPU oracle of the tiered KV-cache decode step.  TEST INFRASTRUCTURE ONLY.

Only the test-suite, the package smoke check and the benchmark's CPU-baseline
leg may import this module.  The product path (the HIP library and its Python
binding) never imports, calls or links it, and it imports nothing from the
product path: the two share no kernels, helpers, tables or constants.

Plain, slow and meant to be checked against the pages by eye.  Floating point
is float64 except where the method fixes another precision (the 8-bit T2
format below works in float32, as the GPU does, so that codes are comparable
bit for bit).

Source: the technical summary pages of "Not All Thoughts Need HBM"
(gist.science, paper 2605.09490; the French page is cited, the Dutch, Italian
and Spanish pages repeat it).  Section names below are the French page's.

* Methodologie section 1 ("Classification a quatre niveaux"): the four tiers.
  T0 lives in HBM and holds the protected tokens (prompt, attention sinks,
  recent window) plus the most important reasoning tokens; T1 sits in host DDR
  at full precision and is brought to the GPU before every attention step; T2
  is kept on the host in reduced precision (8-bit quantisation is the example
  given); T3 is the lowest-importance tail, dropped for good.
* Methodologie section 2 ("Notation de l'importance"), the score equation:
  s_i(t) = s_i(t-1) + (1/|L|) sum over layers l of (1/H) sum over heads h of
  alpha_{l,h}(t)[i].
* Methodologie section 3 ("Dechargement a erreur d'approximation nulle"),
  Proposition 1: because T1 arrives at full precision before attention runs,
  the output depends only on which tokens were evicted (T3), never on how the
  survivors are split between HBM and DDR.
* Methodologie section 4 ("Implementation systeme"): tiers are reassigned
  every Delta = 64 decode steps.

Readings where the pages leave a step open (each is listed, with its reason,
in the design notes of the repository):

* alpha is the softmax of the scaled logits over the attended set
  A = T0 u T1 (T2 and T3 are not attended); scale 1/sqrt(D);
* H counts query heads; under grouped-query attention head h reads KV head
  h // (Hq / Hkv);
* a token appended at a step starts with score 0 and attends to itself;
* scores are a plain running sum, never decayed or reset;
* protected = positions [0, max(prompt, sinks)) and the last ``recent``
  positions at reassignment time;
* tier budgets are fractions of the current length n: N_k = floor(f_k * n)
  for k = 1, 2, 3 (float64 product of the float32 fraction), T0 takes the
  rest;
* ranking ("keep order"): higher score first; equal scores keep the lower
  position first;
* T3 is absorbing; T2 can only move to T3 (its full precision is gone);
  T0 and T1 exchange freely;
* 8-bit T2 format: symmetric, one float32 scale per (position, layer, KV head,
  K-or-V) row of D values, scale = absmax / 127 and code = round-half-even of
  x / scale (both float32 IEEE divisions), clamped to [-127, 127]; an all-zero
  row has scale 0 and codes 0;
* the T1 staging buffer lists T1 positions in ascending order, laid out
  [layer][KV head][row][D], keys then values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

T0, T1, T2, T3 = 0, 1, 2, 3
BF16_NAN = np.uint16(0x7FC0)


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------
def widen(x: np.ndarray) -> np.ndarray:
    """Exact float64 value of bf16 bit patterns (uint16) or of float32 data."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


# --------------------------------------------------------------------------
# attention over the attended set  (Methodologie sections 1 and 3)
# --------------------------------------------------------------------------
def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float
              ) -> Tuple[np.ndarray, np.ndarray]:
    """Decode attention of one layer.

    q: [Hq][D]; K, V: [Hkv][m][D] (any real dtype; widened to float64).
    Returns O [Hq][D] and alpha [Hq][m], both float64.  Query head h reads KV
    head h // (Hq / Hkv).  With m == 0 the output is 0 and alpha is empty.
    """
    q = widen(q)
    K = widen(K)
    V = widen(V)
    hq, d = q.shape
    hkv, m, _ = K.shape
    group = hq // hkv
    O = np.zeros((hq, d))
    alpha = np.zeros((hq, m))
    if m == 0:
        return O, alpha
    for h in range(hq):
        g = h // group
        z = (K[g] @ q[h]) * scale                  # logits of every attended token
        e = np.exp(z - z.max())
        a = e / e.sum()                            # softmax weights
        alpha[h] = a
        O[h] = a @ V[g]
    return O, alpha


# --------------------------------------------------------------------------
# importance score  (Methodologie section 2, score equation)
# --------------------------------------------------------------------------
def score_increment(alpha: np.ndarray) -> np.ndarray:
    """(1/|L|) sum_l (1/H) sum_h alpha[l][h][i]   for alpha of shape [L][H][m]."""
    n_layers, n_heads, m = alpha.shape
    total = np.zeros(m)
    for l in range(n_layers):
        per_layer = np.zeros(m)
        for h in range(n_heads):
            per_layer += alpha[l, h]
        total += per_layer / n_heads
    return total / n_layers


# --------------------------------------------------------------------------
# tier assignment  (Methodologie sections 1 and 4)
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Policy:
    prompt: int
    sinks: int
    recent: int
    frac_t1: float
    frac_t2: float
    frac_t3: float
    delta: int


def budgets(n: int, policy: Policy) -> Tuple[int, int, int, int]:
    """(N0, N1, N2, N3): floor of float32 fraction times n (in float64); T0 takes the rest."""
    def cnt(f: float) -> int:
        return int(math.floor(float(np.float32(f)) * float(n)))
    n1, n2, n3 = cnt(policy.frac_t1), cnt(policy.frac_t2), cnt(policy.frac_t3)
    return n - n1 - n2 - n3, n1, n2, n3


def protected_mask(n: int, policy: Policy) -> np.ndarray:
    """Prompt and sink positions at the start, the recent window at the end."""
    m = np.zeros(n, dtype=bool)
    m[:min(n, max(policy.prompt, policy.sinks))] = True
    if policy.recent > 0:
        m[max(0, n - policy.recent):] = True
    return m


def keep_order(scores: np.ndarray, positions: Sequence[int]) -> List[int]:
    """Positions from most to least important: score descending, then position ascending."""
    return sorted(positions, key=lambda i: (-float(scores[i]), int(i)))


def assign_tiers(scores: np.ndarray, tier_prev: np.ndarray, n: int, policy: Policy
                 ) -> Tuple[np.ndarray, np.ndarray]:
    """New tier of positions [0, n) and the counts [c0, c1, c2, c3].

    Steps, each applied to the keep order of its candidate set and always
    taking the *least* important candidates:
      1. T3 already holds E (absorbing).  Evict e = clamp(N3 - |E|, 0, |pool|)
         more from pool = non-protected positions in T0, T1 or T2.
      2. Old T2 positions that survived stay T2.  Move
         q = clamp(N2 - |survivors|, 0, |live|) more into T2 from
         live = non-protected T0/T1 positions that were not just evicted.
      3. The next min(N1, |live left|) go to T1.
      4. Everything else -- live leftovers and protected T0/T1 positions -- is T0.
    """
    prot = protected_mask(n, policy)
    _, n1, n2, n3 = budgets(n, policy)
    prev = np.asarray(tier_prev[:n]).astype(np.int64)
    new = prev.copy()

    evicted_before = [i for i in range(n) if prev[i] == T3]
    pool = keep_order(scores, [i for i in range(n) if not prot[i] and prev[i] in (T0, T1, T2)])
    e = min(max(n3 - len(evicted_before), 0), len(pool))
    evict = set(pool[len(pool) - e:]) if e > 0 else set()
    for i in evict:
        new[i] = T3

    survivors = [i for i in range(n) if prev[i] == T2 and i not in evict]
    live = keep_order(scores, [i for i in range(n)
                               if not prot[i] and prev[i] in (T0, T1) and i not in evict])
    q = min(max(n2 - len(survivors), 0), len(live))
    to_t2 = live[len(live) - q:] if q > 0 else []
    for i in to_t2:
        new[i] = T2
    live = live[:len(live) - q]

    r = min(n1, len(live))
    to_t1 = live[len(live) - r:] if r > 0 else []
    for i in to_t1:
        new[i] = T1
    for i in live[:len(live) - r]:
        new[i] = T0
    for i in range(n):
        if prot[i] and prev[i] in (T0, T1):
            new[i] = T0

    counts = np.array([(new == t).sum() for t in (T0, T1, T2, T3)], dtype=np.int64)
    return new.astype(np.uint8), counts


# --------------------------------------------------------------------------
# T2: 8-bit rows  (Methodologie section 1, T2)
# --------------------------------------------------------------------------
def quantize_rows(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric int8 per row of the last axis.  x: float32 [..., D].

    scale = absmax / 127 and code = rint(x / scale) as float32 IEEE operations,
    clamped to [-127, 127]; all-zero rows give scale 0 and codes 0.
    """
    x = np.asarray(x, dtype=np.float32)
    absmax = np.max(np.abs(x), axis=-1)
    scale = (absmax / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    quot = (x / safe[..., None]).astype(np.float32)
    codes = np.clip(np.rint(quot), -127, 127)
    codes = np.where(scale[..., None] > 0, codes, 0).astype(np.int8)
    return codes, scale


def dequantize_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    return codes.astype(np.float32) * scale[..., None].astype(np.float32)


# --------------------------------------------------------------------------
# T1 gather  (Methodologie section 1, T1 brought to the GPU before attention)
# --------------------------------------------------------------------------
def gather_rows(store: np.ndarray, positions: Sequence[int]) -> np.ndarray:
    """Rows of a [L][Hkv][cap][D] store at the given positions, in that order."""
    idx = np.asarray(positions, dtype=np.int64)
    return np.ascontiguousarray(store[:, :, idx, :])


# --------------------------------------------------------------------------
# one sequence, stepped
# --------------------------------------------------------------------------
class TieredSequence:
    """State of one sequence under the four-tier hierarchy.

    ``K``/``V`` play the full-precision host store ([L][Hkv][cap][D], bf16 bits
    or float32).  Rows that enter T2 or T3 lose full precision: the store
    row is overwritten with NaN so any later use would poison the output.
    Attention runs over the T0 rows (resident) followed by the T1 staging
    rows gathered at the last reassignment, exactly as the two halves arrive
    on the device.

    With ``attend_t2`` the T2 rows are attended too, in their reduced
    precision: each is rebuilt as code * scale from the 8-bit row stored when
    it entered T2 (Methodologie section 1 keeps T2 at reduced precision; the
    accuracy the pages report for offloading to T2 is that of this variant).
    They follow T1 in ascending position order, enter the same softmax, and
    their scores grow like any attended position's.  T2 still never returns
    to full precision.
    """

    def __init__(self, K0: np.ndarray, V0: np.ndarray, policy: Policy, cap: int,
                 scale: Optional[float] = None, attend_t2: bool = False):
        L, hkv, n0, d = K0.shape
        self.policy = policy
        self.layers, self.kv_heads, self.head_dim = L, hkv, d
        self.scale = (1.0 / math.sqrt(d)) if scale is None else float(scale)
        self.K = np.zeros((L, hkv, cap, d), dtype=K0.dtype)
        self.V = np.zeros((L, hkv, cap, d), dtype=V0.dtype)
        self.K[:, :, :n0] = K0
        self.V[:, :, :n0] = V0
        self.n = n0
        self.s = np.zeros(cap)
        self.tier = np.zeros(cap, dtype=np.uint8)
        self.t1_positions = np.zeros(0, dtype=np.int64)
        self.t1_K = np.zeros((L, hkv, 0, d), dtype=K0.dtype)
        self.t1_V = np.zeros((L, hkv, 0, d), dtype=V0.dtype)
        self.t2_codes: Dict[int, Tuple[np.ndarray, np.ndarray]] = {}
        self.attend_t2 = attend_t2
        self.steps_done = 0

    # ---- helpers -------------------------------------------------------
    def t2_positions(self) -> np.ndarray:
        """Attended T2 positions (ascending); empty unless ``attend_t2``."""
        if not self.attend_t2:
            return np.zeros(0, dtype=np.int64)
        return np.nonzero(self.tier[:self.n] == T2)[0].astype(np.int64)

    def t2_rows(self, positions: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        """Rebuilt T2 rows, the exact products code * scale (float64):
        K, V [L][Hkv][len(positions)][D]."""
        L, hkv, d = self.layers, self.kv_heads, self.head_dim
        K = np.zeros((L, hkv, len(positions), d))
        V = np.zeros((L, hkv, len(positions), d))
        for j, p in enumerate(positions.tolist()):
            codes, scales = self.t2_codes[p]          # [L][Hkv][2][D], [L][Hkv][2]
            c = codes.astype(np.float64)
            sc = scales.astype(np.float64)
            K[:, :, j, :] = c[:, :, 0] * sc[:, :, 0, None]
            V[:, :, j, :] = c[:, :, 1] * sc[:, :, 1, None]
        return K, V

    def attended_positions(self) -> np.ndarray:
        """Device order: T0 positions ascending, then the T1 staging order, then the
        attended T2 positions ascending."""
        t0 = np.nonzero(self.tier[:self.n] == T0)[0]
        return np.concatenate([t0, self.t1_positions, self.t2_positions()]).astype(np.int64)

    def _poison(self, i: int) -> None:
        nan = BF16_NAN if self.K.dtype == np.uint16 else np.float32(np.nan)
        self.K[:, :, i, :] = nan
        self.V[:, :, i, :] = nan

    # ---- the decode step -------------------------------------------------
    def append(self, k_new: np.ndarray, v_new: np.ndarray) -> int:
        """Every generated token adds one key/value pair; it enters T0 with score 0."""
        p = self.n
        self.K[:, :, p, :] = k_new
        self.V[:, :, p, :] = v_new
        self.tier[p] = T0
        self.s[p] = 0.0
        self.n += 1
        return p

    def attend(self, q: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """Attention of every layer over T0 (resident) + T1 (staged).

        Returns O [L][Hq][D], alpha [L][Hq][m] in device order, and the
        positions of those m attended rows.
        """
        t0 = np.nonzero(self.tier[:self.n] == T0)[0]
        t2 = self.t2_positions()
        pos = np.concatenate([t0, self.t1_positions, t2]).astype(np.int64)
        K2, V2 = self.t2_rows(t2)
        outs, alphas = [], []
        for l in range(self.layers):
            K_att = np.concatenate([widen(self.K[l][:, t0, :]), widen(self.t1_K[l]), K2[l]], axis=1)
            V_att = np.concatenate([widen(self.V[l][:, t0, :]), widen(self.t1_V[l]), V2[l]], axis=1)
            O, a = attention(q[l], K_att, V_att, self.scale)
            outs.append(O)
            alphas.append(a)
        return np.stack(outs), np.stack(alphas), pos

    def step(self, q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
             reassign: bool = True) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """Append, attend, add the score increment; reassign tiers every Delta steps."""
        self.append(k_new, v_new)
        O, alpha, pos = self.attend(q)
        self.s[pos] += score_increment(alpha)
        self.steps_done += 1
        if reassign and self.steps_done % self.policy.delta == 0:
            self.reassign()
        return O, alpha, pos

    def reassign(self, scores: Optional[np.ndarray] = None) -> np.ndarray:
        """Rank into tiers, quantise new T2 rows, drop new T3 rows, gather T1.

        ``scores`` replaces the oracle's own scores for the ranking only (used
        to follow another implementation's float32 scores exactly).
        Returns the counts [c0, c1, c2, c3].
        """
        n = self.n
        ranking = self.s[:n] if scores is None else np.asarray(scores[:n], dtype=np.float64)
        prev = self.tier[:n].copy()
        new, counts = assign_tiers(ranking, prev, n, self.policy)
        for i in np.nonzero((new == T2) & (prev != T2))[0].tolist():
            k = widen(self.K[:, :, i, :]).astype(np.float32)
            v = widen(self.V[:, :, i, :]).astype(np.float32)
            ck, sk = quantize_rows(k)
            cv, sv = quantize_rows(v)
            self.t2_codes[i] = (np.stack([ck, cv], axis=2), np.stack([sk, sv], axis=2))
            self._poison(i)
        for i in np.nonzero((new == T3) & (prev != T3))[0].tolist():
            self.t2_codes.pop(i, None)
            self._poison(i)
        self.tier[:n] = new
        self.t1_positions = np.nonzero(new == T1)[0].astype(np.int64)
        self.t1_K = gather_rows(self.K, self.t1_positions)
        self.t1_V = gather_rows(self.V, self.t1_positions)
        return counts
