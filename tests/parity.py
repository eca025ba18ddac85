"""Helpers of the GPU parity tests: run the HIP path and the CPU oracle side by side.

Tolerances (written here once, used by every parity test):
* attention output O: per (sequence, layer, head), max|O_gpu - O_ref| / max|O_ref| <= 2e-3;
* attention weights alpha: the same per-row bar, plus elementwise |d alpha| <= 1e-3 alpha + 1e-9;
* importance scores: elementwise |s_gpu - s_ref| <= 1e-5 s_ref + 1e-12;
* tiers, counts, slot maps, T1 window bytes, int8 codes and scales: bit-exact, given the
  same float32 scores (the oracle ranks the GPU's scores at each reassignment).
"""
from __future__ import annotations

import sys
from collections import defaultdict

import numpy as np
import torch

from oracle import Policy, TieredSequence, attention, assign_tiers, quantize_rows, widen
from tiered_kv_cache_amd.driver import T1Stream, to_device, to_host_bits
from tiered_kv_cache_amd.synth import SequenceStream, Workload
from tiered_kv_cache_amd.workload import DeviceWorkload

O_TOL = 2e-3
S_RTOL = 1e-5
S_ATOL = 1e-12


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_policy(wl: Workload) -> Policy:
    return Policy(wl.prompt, wl.sinks, wl.recent, wl.frac_t1, wl.frac_t2, wl.frac_t3, wl.delta)


def rel_rows(got: np.ndarray, ref: np.ndarray) -> float:
    """max over rows (last axis = row content) of max|got-ref| / max|ref|."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return float((np.abs(got - ref).max(axis=-1) / den).max()) if ref.size else 0.0


def check_output(got, ref, stats, what="O"):
    r = rel_rows(got, ref)
    stats[what] = max(stats[what], r)
    assert r <= O_TOL, f"{what}: relative error {r:.3e} > {O_TOL}"


def check_alpha(got, ref, stats):
    check_output(got, ref, stats, "alpha_row")
    err = np.abs(np.asarray(got, np.float64) - ref)
    bad = err > 1e-3 * np.abs(ref) + 1e-9
    stats["alpha_el"] = max(stats["alpha_el"], float((err / np.maximum(ref, 1e-30)).max()))
    assert not bad.any(), f"alpha elementwise: {int(bad.sum())} entries off, max {err.max():.3e}"


def check_scores(got, ref, stats):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    lim = S_RTOL * np.abs(ref) + S_ATOL
    rel = float((err / np.maximum(np.abs(ref), 1e-30)).max()) if ref.size else 0.0
    stats["score_rel"] = max(stats["score_rel"], rel)
    assert (err <= lim).all(), f"scores: {int((err > lim).sum())} positions off, max rel {rel:.3e}"


def check_reassignment(cache, b, seq: TieredSequence, prev_tiers, gpu_scores, stats,
                       window=None):
    """After both sides reassigned from the same float32 scores: bit-exact state.
    `window` reads the T1 rows (default: the cache's device window)."""
    n = seq.n
    t_gpu = cache.tiers[b, :n].cpu().numpy()
    assert np.array_equal(t_gpu, seq.tier[:n]), \
        f"tiers differ at {np.nonzero(t_gpu != seq.tier[:n])[0][:10]}"
    counts = cache.counts[b].cpu().numpy()
    assert counts.tolist() == [int((seq.tier[:n] == t).sum()) for t in range(4)]
    t0 = np.nonzero(seq.tier[:n] == 0)[0]
    assert cache.t0_len[b] == len(t0) and cache.t1_len[b] == len(seq.t1_positions)
    assert np.array_equal(cache.t0_positions(b), t0)
    assert np.array_equal(cache.t1_positions(b), seq.t1_positions)
    k1, v1 = (window or cache).t1_rows(b)
    assert k1.tobytes() == np.ascontiguousarray(seq.t1_K).tobytes(), "T1 window keys differ"
    assert v1.tobytes() == np.ascontiguousarray(seq.t1_V).tobytes(), "T1 window values differ"
    new_t2 = np.nonzero((seq.tier[:n] == 2) & (prev_tiers[:n] <= 1))[0]
    pos, codes, scales = cache.last_t2(b)
    assert np.array_equal(pos, new_t2), "newly-T2 positions differ"
    for i, p in enumerate(pos.tolist()):
        rc, rs = seq.t2_codes[p]
        assert np.array_equal(codes[i], rc), f"int8 codes differ at position {p}"
        assert np.array_equal(scales[i].view(np.uint32), rs.view(np.uint32)), \
            f"scales differ at position {p}"
    stats["t2_rows"] += len(pos)
    stats["reassignments"] += 1
    if cache.attend_t2:
        check_t2_pool(cache, b, seq, stats)


def check_t2_pool(cache, b, seq: TieredSequence, stats):
    """The attended T2 pool holds exactly the oracle's T2 positions, each with the
    int8 codes and scales the oracle stored when it entered T2 (bit-exact)."""
    t2 = np.nonzero(seq.tier[:seq.n] == 2)[0]
    assert cache.t2_len[b] == len(t2), f"T2 pool length {cache.t2_len[b]} != {len(t2)}"
    assert np.array_equal(cache.t2_positions(b), t2), "T2 pool positions differ"
    kc, vc, ks, vs = cache.t2_pool_rows(b)
    for j, p in enumerate(t2.tolist()):
        rc, rs = seq.t2_codes[p]                    # [L][Hkv][2][D], [L][Hkv][2]
        assert np.array_equal(kc[:, :, j], rc[:, :, 0]), f"T2 pool key codes differ at {p}"
        assert np.array_equal(vc[:, :, j], rc[:, :, 1]), f"T2 pool value codes differ at {p}"
        assert np.array_equal(ks[:, :, j].view(np.uint32), rs[:, :, 0].view(np.uint32))
        assert np.array_equal(vs[:, :, j].view(np.uint32), rs[:, :, 1].view(np.uint32))
    stats["t2_pool_rows"] = max(stats["t2_pool_rows"], len(t2))


def step_inputs(cache, dw, q, kn, vn, fused_append: bool) -> None:
    """Append the step's new rows and attend, fused or as two calls."""
    qd = to_device(q, dw.dtype, dw.device)
    kd, vd = to_device(kn, dw.dtype, dw.device), to_device(vn, dw.dtype, dw.device)
    if fused_append:
        cache.append_attend(qd, kd, vd)
    else:
        cache.append(kd, vd)
        cache.attend(qd)


def streamed_step_link(cache) -> int:
    """Bytes a streamed step must send: the live 32-slot blocks of every sequence's T1
    rows, keys and values of every (layer, KV head)."""
    sh = cache.shape
    e = 2 if sh.dtype == "bf16" else 4
    return sum(-(-n // 32) * 32 for n in cache.t1_len) * sh.head_dim * e * sh.layers * sh.kv_heads * 2


def reassign_link_rows(prev_tiers, new_tiers) -> int:
    """Rows a reassignment with host-resident T1 must move over the link: those that
    enter T1 from T0 (device -> host) and those that leave T1 for T0 or T2 (host ->
    device).  Rows that stay, and every other transition, move no row."""
    rows = 0
    for p, w in zip(prev_tiers, new_tiers):
        rows += int(((p == 0) & (w == 1)).sum() + ((p == 1) & ((w == 0) | (w == 2))).sum())
    return rows


def check_reassign_link(streamer, prevs, news, stats):
    """The link bytes of the last reassignment: the rows that changed side, plus the tier
    maps and T1 slot maps the host reads (2 max_ctx + 16 cap1 + 32 bytes per sequence)."""
    c = streamer.cache
    sh = c.shape
    e = 2 if sh.dtype == "bf16" else 4
    row = sh.layers * sh.kv_heads * 2 * sh.head_dim * e
    maps = c.batch * (2 * c.max_ctx + 16 * c.cap1 + 32)
    rows = reassign_link_rows(prevs, news)
    got = streamer.link_reassign[-1]
    assert got == rows * row + maps, f"reassignment link bytes {got} != {rows} rows + maps"
    stats["link_rows"] += rows


def run_lockstep(wl: Workload, n_steps: int = None, label: str = "",
                 fused_scores: bool = True, fused_append: bool = True,
                 attend_t2: bool = False, t1_streamed: int = 0, t0_budget: bool = False,
                 alpha_scratch: bool = False, per_sequence: bool = False) -> dict:
    """Every step compared; re-sync of the ranking at each reassignment.
    fused_scores=False adds alpha to the scores with the stand-alone tkv_update_scores;
    fused_append=False appends with tkv_append before tkv_decode_step instead of
    tkv_append_decode_step; attend_t2 attends the 8-bit T2 rows after T1 on both sides
    (the _t2 entry points and the oracle's attend_t2 mode); t1_streamed > 0 keeps the T1
    rows in host memory and attends chunks of that many layers with them streamed from
    pinned memory (T1Stream), checking the link bytes of every step and reassignment;
    t0_budget shrinks the T0 pool to its budget after the first reassignment;
    alpha_scratch runs the calls that store no weights (alpha is then checked through
    the scores, which every step compares); per_sequence gives every sequence pools of
    its own capacity (packed one after the other)."""
    n_steps = n_steps or wl.total_steps
    dw = DeviceWorkload(wl)
    cache = dw.make_cache(attend_t2=attend_t2, t0_budget=t0_budget, alpha_scratch=alpha_scratch,
                          per_sequence=per_sequence)
    cache.fused_scores = fused_scores
    cap0_start = cache.cap0
    streamer = T1Stream(cache, chunk_layers=t1_streamed) if t1_streamed else None
    pol = oracle_policy(wl)
    seqs = []
    for b in range(wl.batch):
        K, V = dw.streams[b].context()
        seqs.append(TieredSequence(K, V, pol, cap=cache.max_ctx, attend_t2=attend_t2))
    stats = defaultdict(float)
    for k in range(1, n_steps + 1):
        q, kn, vn = dw.host_step(k)
        if streamer is not None:
            streamer.step(to_device(q, dw.dtype, dw.device), to_device(kn, dw.dtype, dw.device),
                          to_device(vn, dw.dtype, dw.device), reassign=False)
            assert streamer.link_step == streamed_step_link(cache), f"step link bytes, step {k}"
        else:
            step_inputs(cache, dw, q, kn, vn, fused_append)
            cache.steps += 1
        torch.cuda.synchronize()
        out = cache.out.cpu().numpy()
        for b, seq in enumerate(seqs):
            O, alpha, pos = seq.step(q[b], kn[b], vn[b], reassign=False)
            assert np.array_equal(cache.attended_positions(b), pos), f"attended set, step {k}"
            check_output(out[b], O, stats)
            if not alpha_scratch:
                check_alpha(cache.alpha_of(b), alpha, stats)
            check_scores(cache.scores[b, :seq.n].cpu().numpy(), seq.s[:seq.n], stats)
        if k % wl.delta == 0:
            gpu_scores = cache.scores.cpu().numpy()
            prevs = [s.tier.copy() for s in seqs]
            if streamer is not None:
                streamer.reassign()
            else:
                cache.reassign()
            torch.cuda.synchronize()
            for b, seq in enumerate(seqs):
                seq.reassign(scores=gpu_scores[b])
                check_reassignment(cache, b, seq, prevs[b], gpu_scores[b], stats, streamer)
            if streamer is not None:
                check_reassign_link(streamer, [p[:s.n] for p, s in zip(prevs, seqs)],
                                    [s.tier[:s.n] for s in seqs], stats)
            if t0_budget and cache.reassignments == 1:
                assert cache.cap0 <= cap0_start
                stats["cap0"] = cache.cap0
    stats["steps"] = n_steps
    say(f"[{label or wl.name}] lockstep ok: " +
        ", ".join(f"{k}={v:.3g}" for k, v in sorted(stats.items())))
    return stats


class HostStore:
    """Full-precision copy of every sequence's K/V rows ([L][Hkv][cap][D] per sequence),
    filled from the shared generator: the inputs the sampled full-size checks read."""

    def __init__(self, dw: DeviceWorkload, cap: int):
        self.K, self.V = [], []
        for st in dw.streams:
            K0, V0 = st.context()
            L, H, n0, D = K0.shape
            K = np.zeros((L, H, cap, D), K0.dtype)
            V = np.zeros((L, H, cap, D), V0.dtype)
            K[:, :, :n0] = K0
            V[:, :, :n0] = V0
            self.K.append(K)
            self.V.append(V)

    def put(self, b, pos, k, v):
        self.K[b][:, :, pos] = k
        self.V[b][:, :, pos] = v


def run_sampled(wl: Workload, n_steps: int, sample_steps, heads, full_inc_steps=(),
                label: str = "", byte_seqs=None, attend_t2: bool = False,
                t1_streamed: int = 0, t0_budget: bool = False, alpha_scratch: bool = False,
                per_sequence: bool = False) -> dict:
    """Full-size run, checked on samples the oracle computes one at a time:
    * O and alpha of the sampled (layer, head) pairs over the GPU's attended set;
    * the whole score increment at `full_inc_steps` (all layers and heads);
    * total score mass == steps (any size);
    * at every reassignment: tiers from the oracle ranking of the GPU's scores, the
      counts and slot maps of every sequence; the T0/T1 row bytes and the int8 rows of
      new T2 positions of the sequences in `byte_seqs` (default: all);
    * with attend_t2, the attended T2 rows enter the oracle as code x scale of the int8
      rows of the full-precision store (bit-exact codes, as the quantizer is), and the T2
      pool's positions are checked at every reassignment; with t1_streamed > 0 the T1
      rows live in host memory and the steps run through T1Stream with chunks of that
      many layers (link bytes of every step and reassignment checked); t0_budget shrinks
      the T0 pool after the first reassignment.
    """
    byte_seqs = set(range(wl.batch)) if byte_seqs is None else set(byte_seqs)
    dw = DeviceWorkload(wl)
    cache = dw.make_cache(attend_t2=attend_t2, t0_budget=t0_budget, alpha_scratch=alpha_scratch,
                          per_sequence=per_sequence)
    streamer = T1Stream(cache, chunk_layers=t1_streamed) if t1_streamed else None
    store = HostStore(dw, cache.max_ctx)
    pol = oracle_policy(wl)
    scale = 1.0 / np.sqrt(wl.head_dim)
    stats = defaultdict(float)
    group = wl.q_heads // wl.kv_heads
    for k in range(1, n_steps + 1):
        q, kn, vn = dw.host_step(k)
        for b in range(wl.batch):
            store.put(b, cache.n[b], kn[b], vn[b])
        s_before = cache.scores.cpu().numpy() if k in full_inc_steps else None
        if streamer is not None:
            streamer.step(to_device(q, dw.dtype, dw.device), to_device(kn, dw.dtype, dw.device),
                          to_device(vn, dw.dtype, dw.device), reassign=False)
            assert streamer.link_step == streamed_step_link(cache), f"step link bytes, step {k}"
        else:
            step_inputs(cache, dw, q, kn, vn, True)
            cache.steps += 1
        if k in sample_steps or k in full_inc_steps:
            torch.cuda.synchronize()
            out = cache.out.cpu().numpy()
            for b in range(wl.batch):
                pos = cache.attended_positions(b)
                alpha_gpu = None if alpha_scratch else cache.alpha_of(b)
                layers = range(wl.layers) if k in full_inc_steps else sorted({l for l, _ in heads})
                inc = np.zeros(cache.n[b])
                t2 = set(cache.t2_positions(b).tolist()) if attend_t2 else set()
                t2_idx = np.array([j for j, p in enumerate(pos.tolist()) if p in t2], np.int64)
                for l in layers:
                    Kl = store.K[b][l][:, pos]
                    Vl = store.V[b][l][:, pos]
                    if len(t2_idx):  # attended T2 rows: code x scale, float64
                        Kl, Vl = widen(Kl), widen(Vl)
                        for X in (Kl, Vl):
                            c_, s_ = quantize_rows(X[:, t2_idx].astype(np.float32))
                            X[:, t2_idx] = c_.astype(np.float64) * s_.astype(np.float64)[..., None]
                    hs = range(wl.q_heads) if k in full_inc_steps else [h for ll, h in heads if ll == l]
                    for h in hs:
                        g = h // group
                        O, a = attention(q[b][l][h:h + 1], Kl[g:g + 1], Vl[g:g + 1], scale)
                        check_output(out[b, l, h][None], O, stats)
                        if alpha_gpu is not None:
                            check_alpha(alpha_gpu[l, h][None], a, stats)
                        inc[pos] += a[0]
                if k in full_inc_steps:
                    inc /= (wl.layers * wl.q_heads)
                    got = cache.scores[b, :cache.n[b]].cpu().numpy().astype(np.float64) - s_before[b, :cache.n[b]]
                    err = np.abs(got - inc)
                    # the difference of two float32 values carries their rounding (a few
                    # ulp of s); every path adds the step's increment to s once
                    lim = 1e-5 * inc + 2.0 ** -24 * 4 * np.abs(s_before[b, :cache.n[b]]) + 1e-12
                    assert (err <= lim).all(), f"score increment, step {k}, seq {b}: max {err.max():.3e}"
                    stats["inc_checked"] += 1
        if k % wl.delta == 0:
            torch.cuda.synchronize()
            gpu_scores = cache.scores.cpu().numpy()
            prev = cache.tiers.cpu().numpy()
            for b in range(wl.batch):
                mass = float(gpu_scores[b, :cache.n[b]].astype(np.float64).sum())
                assert abs(mass - k) <= 1e-5 * k, f"score mass {mass} after {k} steps"
            if streamer is not None:
                streamer.reassign()
            else:
                cache.reassign()
            torch.cuda.synchronize()
            if streamer is not None:
                news = [cache.tiers[b, :cache.n[b]].cpu().numpy() for b in range(wl.batch)]
                check_reassign_link(streamer, [prev[b, :cache.n[b]] for b in range(wl.batch)],
                                    news, stats)
            for b in range(wl.batch):
                n = cache.n[b]
                t_ref, counts = assign_tiers(gpu_scores[b, :n].astype(np.float64), prev[b, :n], n, pol)
                t_gpu = cache.tiers[b, :n].cpu().numpy()
                assert np.array_equal(t_gpu, t_ref), f"tiers differ (step {k}, seq {b})"
                assert cache.counts[b].cpu().numpy().tolist() == counts.tolist()
                t0 = np.nonzero(t_ref == 0)[0]
                t1 = np.nonzero(t_ref == 1)[0]
                assert np.array_equal(cache.t0_positions(b), t0)
                assert np.array_equal(cache.t1_positions(b), t1)
                if attend_t2:
                    assert np.array_equal(cache.t2_positions(b), np.nonzero(t_ref == 2)[0])
                    stats["t2_pool_rows"] = max(stats["t2_pool_rows"], cache.t2_len[b])
                stats["reassignments"] += 1
                if b not in byte_seqs:
                    continue
                k1, v1 = (streamer or cache).t1_rows(b)
                assert k1.tobytes() == np.ascontiguousarray(store.K[b][:, :, t1]).tobytes()
                assert v1.tobytes() == np.ascontiguousarray(store.V[b][:, :, t1]).tobytes()
                k0, v0 = cache.t0_rows(b)
                assert k0.tobytes() == np.ascontiguousarray(store.K[b][:, :, t0]).tobytes()
                assert v0.tobytes() == np.ascontiguousarray(store.V[b][:, :, t0]).tobytes()
                new_t2 = np.nonzero((t_ref == 2) & (prev[b, :n] <= 1))[0]
                pos, codes, scales = cache.last_t2(b)
                assert np.array_equal(pos, new_t2)
                if len(pos):
                    ck, sk = quantize_rows(widen(store.K[b][:, :, pos]).astype(np.float32))
                    cv, sv = quantize_rows(widen(store.V[b][:, :, pos]).astype(np.float32))
                    # oracle layout [L][Hkv][rows][D] -> [rows][L][Hkv][2][D]
                    ref_codes = np.stack([ck, cv], axis=3).transpose(2, 0, 1, 3, 4)
                    ref_scales = np.stack([sk, sv], axis=3).transpose(2, 0, 1, 3)
                    assert np.array_equal(codes, ref_codes), "int8 codes differ"
                    assert np.array_equal(scales.view(np.uint32), ref_scales.view(np.uint32))
                stats["t2_rows"] += len(pos)
    stats["steps"] = n_steps
    say(f"[{label or wl.name}] sampled ok: " +
        ", ".join(f"{k}={v:.3g}" for k, v in sorted(stats.items())))
    return stats
