"""Decode-step throughput of the tiered KV-cache hot path on one MI355X.

A step is one pass of the whole device path over one batch of synthetic input:
append the new token's K/V, attention over T0 u T1 with the normalised weights
written out, the fused importance-score update, and every Delta steps the tier
ranking, the compaction of the T0 pool / T1 window and the int8 rows of new T2
tokens.  Inputs are resident in HBM before the timed region starts; the T1
rows are in their device window (the host-link transfer is measured on its own
and reported under "pcie", never in `value`).

The timed steps always start from the tiered state: the warm-up runs at least
Delta steps, so the first reassignment (every position in T0 until then) is
behind it.  When the K timed steps hold no reassignment (K < Delta), the
untimed steps continue to the next multiple of Delta and that reassignment is
timed on its own; K / Delta of its cost is added to the timed interval, so
`value` always pays for the tier work at the method's cadence.

Prints one JSON line.  Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import gc
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, vendor figure


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=256)
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--workload", default="chain8k")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-pcie", action="store_true")
    p.add_argument("--no-flush-run", action="store_true",
                   help="skip the run that reads a 512 MB buffer before every step")
    p.add_argument("--no-stream-leg", action="store_true",
                   help="skip the run that streams T1 layer by layer from pinned host memory "
                        "(reported under \"t1_streamed\", never in value)")
    p.add_argument("--stream-chunk", type=int, default=1,
                   help="layers per streamed chunk of T1 rows (two chunks are resident)")
    p.add_argument("--no-t2-leg", action="store_true",
                   help="skip the run that also attends the 8-bit T2 rows (reported under "
                        "\"attend_t2\", never in value)")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="bound on the oracle's timed CPU work")
    p.add_argument("--repeats", type=int, default=5,
                   help="repetitions of the measured run; value and roofline are their medians")
    p.add_argument("--eviction-curve", action="store_true",
                   help="instead of the bench line: output error against full attention, per "
                        "step, for eviction-only policies and tiered policies that keep the same "
                        "share of the context in HBM (one JSON line)")
    p.add_argument("--read-ceiling", action="store_true",
                   help="instead of the bench line: the read bandwidth of the attention kernel's "
                        "access pattern without its arithmetic (tkv_read_probe) on the bytes of "
                        "one attention launch of the workload, 512 MB read before each repetition "
                        "(one JSON line)")
    p.add_argument("--read-ceiling-sweep", action="store_true",
                   help="with --read-ceiling (implied): also the read probe at 0.5 to 8 waves "
                        "per SIMD over the launch's bytes, four and sixteen times them (a second "
                        "JSON line)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run one plain 256 MiB read + 256 MiB write elementwise kernel first "
                        "(scale reference for HBM byte counters)")
    return p.parse_args()


def step_bytes(wl, n_att: int, n: int) -> dict:
    """Algorithmic HBM bytes of one decode step (per sequence, all layers)."""
    L, Hq, Hkv, D = wl.layers, wl.q_heads, wl.kv_heads, wl.head_dim
    e = 2 if wl.dtype == "bf16" else 4
    kv = 2 * L * Hkv * n_att * D * e          # K and V rows of the attended set
    q = L * Hq * D * e
    o = L * Hq * D * 4
    alpha = 2 * L * Hq * n_att * 4             # weights: written, read back by the score
    s = 8 * n_att                              # score read-modify-write
    append = 2 * 2 * L * Hkv * D * e           # new row read + pool write
    minimal = kv + q + o + s + append
    return {"kv": kv, "q": q, "o": o, "alpha": alpha, "scores": s, "append": append,
            "minimal": minimal, "total": minimal + alpha}


def attn_partial_bytes(wl, n_att: int, n_t2: int = 0) -> int:
    """Algorithmic bytes of one attn_partial launch: K/V of the attended set, the
    queries, and the raw logits it writes (read back once to normalise).  n_att counts
    the full-precision rows (T0, T1); the n_t2 attended 8-bit rows read D one-byte codes
    and one float32 scale for K and for V per (layer, KV head)."""
    L, Hq, Hkv, D = wl.layers, wl.q_heads, wl.kv_heads, wl.head_dim
    e = 2 if wl.dtype == "bf16" else 4
    return (2 * L * Hkv * n_att * D * e + 2 * L * Hkv * n_t2 * (D + 4) + L * Hq * D * e
            + L * Hq * (n_att + n_t2) * 4)


def reassign_bytes(wl, n: int, n0: int, n1: int, r2: int, moved: int) -> int:
    """Algorithmic bytes of one reassignment (amortised over Delta steps)."""
    L, Hkv, D = wl.layers, wl.kv_heads, wl.head_dim
    e = 2 if wl.dtype == "bf16" else 4
    tiers = n * (4 + 1 + 1)                    # scores + previous map read, new map write
    # maps: two tier maps and an inverse map over positions, the slot maps;
    # rows: each copy reads and writes a K and a V row of every (layer, KV head)
    compact = n * (2 + 8) + (n0 + n1) * 8 + moved * 2 * L * Hkv * D * e * 2
    quant = r2 * L * Hkv * 2 * (D * e + D + 4)
    return tiers + compact + quant


EVERY_STEP_KERNELS = ("append", "attn_partial", "attn_merge", "score_update")


def kernel_sum(kernels: dict, steps: int, reassignments: int = None, delta: int = None) -> dict:
    """Per-step kernel time: the launches of every step plus the per-Delta launches
    amortised.  With `reassignments` and `delta`, the per-Delta launches were timed over
    that many reassignments and each costs 1/delta of it per step; otherwise they ran
    inside the `steps` timed steps (each kernel's total time / steps)."""
    step = sum(k["total_ms"] * 1e3 / steps for n, k in kernels.items() if n in EVERY_STEP_KERNELS)
    re_total = sum(k["total_ms"] * 1e3 for n, k in kernels.items() if n not in EVERY_STEP_KERNELS)
    if reassignments:
        reassign = re_total / reassignments / delta
    else:
        reassign = re_total / steps
    return {"every_step": step, "reassignment_amortised": reassign, "total": step + reassign}


def budget_counts(wl, n: int):
    """Tier counts the stated split gives at length n (T1..T3 = floor(f * n) of the
    float32 fractions, T0 the rest)."""
    import numpy as np
    n1, n2, n3 = (int(math.floor(float(np.float32(f)) * n)) for f in wl.fractions())
    return [n - n1 - n2 - n3, n1, n2, n3]


COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_partial_{workload}_hbm_counters.md")


def counter_traffic(workload: str, attended_rows: float):
    """HBM bytes per attn_partial launch from the committed counter summary, or None when
    there is none for this workload, the kernel sources changed since it was taken, or
    its launches attended another mean number of rows than this run's (more than 0.5%
    apart): counter bytes of one state are not the traffic of another."""
    import hashlib
    path = COUNTERS_FILE.format(workload=workload)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", "`")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    try:
        h = hashlib.sha256()
        for f in fields["source_files"].split():
            with open(os.path.join(ROOT, f), "rb") as fh:
                h.update(fh.read())
        if h.hexdigest() != fields["source_sha256"]:
            return None
        rows = float(fields["attended_rows_per_launch"])
        if abs(rows - attended_rows) > 0.005 * attended_rows:
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def cpu_baseline(wl, seconds: float) -> dict:
    """The oracle, as it stands, on a bounded sample of the same workload in its tiered
    state: two steps on the full cache, one reassignment (the stated split), then timed
    steps with the BLAS pool at its default size and with one thread; the faster of the
    two is the value (its thread count is `cores`), the other is reported beside it."""
    import numpy as np
    from oracle import Policy, TieredSequence
    from tiered_kv_cache_amd.synth import SequenceStream

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        blas_threads = 1
    st = SequenceStream(wl, 0)
    K, V = st.context()
    pol = Policy(wl.prompt, wl.sinks, wl.recent, wl.frac_t1, wl.frac_t2, wl.frac_t3, wl.delta)
    seq = TieredSequence(K, V, pol, cap=wl.max_ctx)
    k = 0

    def one_step():
        nonlocal k
        k += 1
        q = st.query(k)
        kn, vn = st.new_kv(k)
        t0 = time.perf_counter()
        seq.step(q, kn, vn, reassign=False)
        return time.perf_counter() - t0

    for _ in range(2):
        one_step()
    t0 = time.perf_counter()
    counts = seq.reassign()
    t_re = time.perf_counter() - t0
    attended, n_re = int(counts[0] + counts[1]), seq.n

    def timed(limit_s):
        out, t_start = [], time.perf_counter()
        while len(out) < wl.delta and (time.perf_counter() - t_start) < limit_s:
            out.append(one_step())
        return out

    runs = {int(blas_threads): timed(seconds / 2)}
    if threadpool_limits is not None and blas_threads > 1:
        with threadpool_limits(limits=1):
            runs[1] = timed(seconds / 2)
    rates = {c: 1.0 / (float(np.mean(v)) + t_re / wl.delta) for c, v in runs.items() if v}
    best = max(rates, key=rates.get)
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": rates[best], "unit": "steps/s", "cores": best,
            "other_thread_counts": {str(c): {"value": r, "steps_timed": len(runs[c])}
                                    for c, r in rates.items() if c != best},
            "kind": "oracle",
            "sample": (f"{len(runs[best])} decode steps of {wl.name} in its tiered state (two "
                       f"steps on the full cache, then one reassignment: {attended} of "
                       f"{n_re} positions attended at its start; float64 "
                       f"NumPy) plus one reassignment amortised over delta={wl.delta}"),
            "ms_per_step": float(np.mean(runs[best])) * 1e3, "reassign_ms": t_re * 1e3,
            "cpu": model, "affinity_cpus": len(os.sched_getaffinity(0))}


def pcie_leg(wl, cache, positions, device_step_s: float) -> dict:
    """Host-link path of a full T1 gather (tkv_gather_t1): host pack of every T1 row into
    pinned staging, then one 2-D copy to a device window on a side stream.  This is what
    a T1 set moved wholesale would cost; the host-resident mode (the t1_streamed leg)
    moves only the rows that change tier at a reassignment and streams the window."""
    import numpy as np
    import torch
    from tiered_kv_cache_amd import tkv

    L, Hkv, D = wl.layers, wl.kv_heads, wl.head_dim
    cap1, max_ctx = cache.cap1, cache.max_ctx
    dt = cache.shape.torch_dtype
    r = np.random.default_rng(0)
    host_k = torch.from_numpy(r.integers(0, 1 << 15, size=(L, Hkv, max_ctx, D), dtype=np.int16)).view(dt)
    host_v = host_k.clone()
    stg = torch.empty((L, Hkv, 2, cap1, D), dtype=dt, pin_memory=True)
    dev = torch.empty((L, Hkv, 2, cap1, D), dtype=dt, device="cuda")
    side = torch.cuda.Stream()
    n1 = len(positions)
    bytes_t1 = 2 * L * Hkv * n1 * D * dev.element_size()
    packs = []
    for _ in range(3):  # the first call also starts the host threads and touches the staging
        t0 = time.perf_counter()
        tkv.tkv_gather_t1(cache.model, host_k, host_v, max_ctx, positions, n1, stg, cap1, None,
                          side, None)
        packs.append(time.perf_counter() - t0)
    t_pack = float(np.median(packs))
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    ev0.record(side)
    for _ in range(reps):
        tkv.tkv_gather_t1(cache.model, None, None, max_ctx, None, n1, stg, cap1, dev, side, None)
    ev1.record(side)
    ev1.synchronize()
    t_h2d = ev0.elapsed_time(ev1) / 1e3 / reps
    return {"t1_rows": n1, "t1_bytes": bytes_t1, "pack_ms": t_pack * 1e3,
            "pack_ms_each": [x * 1e3 for x in packs],
            "pack_gbps": bytes_t1 / t_pack / 1e9 if t_pack > 0 else None,
            "h2d_ms": t_h2d * 1e3, "h2d_gbps": bytes_t1 / t_h2d / 1e9 if t_h2d > 0 else None}


def read_ceiling(wl, n_att: int, repeats: int = 20) -> dict:
    """The attention kernel's access pattern without its arithmetic: one wave per SIMD,
    contiguous per-wave ranges, 16 KB units of 1 KB non-temporal wave loads, over the
    bytes one attention launch of the workload reads (K/V of n_att rows per layer and
    KV head, and the logits it writes, counted as reads), 512 MB read before every
    repetition so the memory-side cache is cold."""
    import numpy as np
    import torch
    from tiered_kv_cache_amd import tkv

    nbytes = attn_partial_bytes(wl, n_att)
    nbytes = (nbytes + (16 << 10) - 1) // (16 << 10) * (16 << 10)
    buf = torch.randint(0, 1 << 30, (nbytes // 4,), dtype=torch.int32, device="cuda")
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    waves = 4 * cus
    sink = torch.zeros(waves, dtype=torch.int32, device="cuda")
    times = []
    for _ in range(repeats):
        flush.sum()
        tkv.tkv_timing_select(["read_probe"])
        tkv.tkv_timing_reset()
        tkv.tkv_timing_enable(True)
        tkv.tkv_read_probe(buf, nbytes, waves, sink)
        tkv.tkv_timing_enable(False)
        torch.cuda.synchronize()
        ms, _ = tkv.tkv_timing_read("read_probe")
        times.append(ms * 1e3)
    tkv.tkv_timing_select(None)
    us = float(np.median(times))
    return {"read_ceiling": {"bytes": nbytes, "waves": waves, "median_us": us,
                             "min_us": float(min(times)), "gbps": nbytes / (us * 1e-6) / 1e9,
                             "frac_of_peak": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                             "attended_rows": n_att, "repeats": repeats,
                             "workload": f"{wl.name}: {wl.description}"}}


def read_ceiling_sweep(wl, n_att: int, repeats: int = 10) -> dict:
    """The read probe over the launch's bytes, four and sixteen times them, with 0.5 to 8
    waves per SIMD: whether the one-wave-per-SIMD figure is the chip's streaming rate or an artefact of
    the geometry, and what a launch's fixed ramp and tail cost at this size."""
    import numpy as np
    import torch
    from tiered_kv_cache_amd import tkv

    base = attn_partial_bytes(wl, n_att)
    base = (base + (16 << 10) - 1) // (16 << 10) * (16 << 10)
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows = []
    for scale in (1, 4, 16):
        nbytes = base * scale
        buf = torch.randint(0, 1 << 30, (nbytes // 4,), dtype=torch.int32, device="cuda")
        for per_simd in (0.5, 1, 2, 4, 8):
            waves = int(4 * cus * per_simd)
            sink = torch.zeros(waves, dtype=torch.int32, device="cuda")
            times = []
            for _ in range(repeats):
                flush.sum()
                tkv.tkv_timing_select(["read_probe"])
                tkv.tkv_timing_reset()
                tkv.tkv_timing_enable(True)
                tkv.tkv_read_probe(buf, nbytes, waves, sink)
                tkv.tkv_timing_enable(False)
                torch.cuda.synchronize()
                ms, _ = tkv.tkv_timing_read("read_probe")
                times.append(ms * 1e3)
            us = float(np.median(times))
            rows.append({"bytes": nbytes, "waves": waves, "waves_per_simd": per_simd,
                         "median_us": us, "gbps": nbytes / (us * 1e-6) / 1e9,
                         "frac_of_peak": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS})
            print(f"[bench] read probe {nbytes / 1e6:.1f} MB, {waves} waves: {us:.1f} us",
                  file=sys.stderr, flush=True)
        del buf
    tkv.tkv_timing_select(None)
    return {"read_ceiling_sweep": {"rows": rows, "repeats": repeats, "attended_rows": n_att,
                                   "workload": f"{wl.name}: {wl.description}"}}


def eviction_curve(wl, shares=(0.05, 0.10, 0.20, 0.30, 0.50)) -> dict:
    """Mechanism-level accuracy of the tiers on synthetic inputs.

    For each share x of the context kept out of HBM, four policies run the same
    inputs as a full-attention run (every position in T0): eviction only (T3 = x),
    tiered (T1 = x, nothing evicted), T2 = x (8-bit rows, not attended, so at the
    attention level the same as evicting them), T2 = x attended as code x scale (the
    quantisation error alone), and a fixed eviction with the rest
    offloaded (T1 = x - 0.05, T3 = 0.05), which Proposition 1 of the pages says
    must match eviction only at 0.05.  Error of one step: max over (sequence,
    layer, head) rows of max|O - O_full| / max|O_full|."""
    import numpy as np
    import torch
    from tiered_kv_cache_amd.workload import DeviceWorkload

    dw = DeviceWorkload(wl.with_fractions(0.0, 0.0, 0.0, "_full"))
    contexts = [st.context() for st in dw.streams]
    inputs = dw.preload(1, wl.total_steps)

    def run(f1, f2, f3, attend_t2=False):
        cache = DeviceWorkload(wl.with_fractions(f1, f2, f3)).make_cache(contexts=contexts,
                                                                         attend_t2=attend_t2)
        outs = []
        for k in range(1, wl.total_steps + 1):
            cache.step(*inputs[k - 1])
            if k > wl.warmup:
                outs.append(cache.out.clone())
        torch.cuda.synchronize()
        return outs

    full = run(0.0, 0.0, 0.0)

    def err(outs):
        e = []
        for o, r in zip(outs, full):
            num = (o - r).abs().amax(dim=-1)
            den = r.abs().amax(dim=-1).clamp_min(1e-30)
            e.append(float((num / den).max()))
        return {"mean": float(np.mean(e)), "max": float(np.max(e))}

    rows = []
    for x in shares:
        row = {"off_hbm_share": x,
               "eviction_only": err(run(0.0, 0.0, x)),
               "tiered_t1": err(run(x, 0.0, 0.0)),
               "t2_not_attended": err(run(0.0, x, 0.0)),
               "t2_attended": err(run(0.0, x, 0.0, attend_t2=True))}
        if x > 0.05:
            row["t1_plus_fixed_eviction_0.05"] = err(run(x - 0.05, 0.0, 0.05))
        rows.append(row)
        print(f"[curve] {x}: {row}", file=sys.stderr, flush=True)
    return {"eviction_curve": rows, "workload": f"{wl.name}: {wl.description}",
            "timed_steps": wl.steps, "warmup": wl.warmup, "delta": wl.delta,
            "error": "per step: max over (sequence, layer, head) of max|O - O_full| / "
                     "max|O_full|; mean and max over the timed steps"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the tiered "
              "path would shard by sequence or by KV head (one all-reduce of the partial "
              "scores every Delta steps), and this program measures one GPU's share",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from tiered_kv_cache_amd import tkv
    from tiered_kv_cache_amd.synth import WORKLOADS
    from tiered_kv_cache_amd.workload import DeviceWorkload

    tkv.lib()
    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)       # reads 256 MiB, writes 256 MiB
        torch.cuda.synchronize()
        del src, dst
    base = WORKLOADS[args.workload]
    delta = base.delta
    K = args.steps
    # the timed steps start from the tiered state: the first reassignment (after step
    # Delta) lies inside the warm-up
    W = max(args.warmup, delta)
    # untimed steps after the timed ones, up to the next reassignment, when the timed
    # steps hold none: that reassignment is timed on its own and amortised
    extra = 0 if K >= delta else (-(W + K)) % delta
    wl = base.scaled(steps=K + extra, warmup=W)
    if args.eviction_curve:
        print(json.dumps(eviction_curve(base.scaled(steps=K, warmup=W))), flush=True)
        return
    if args.read_ceiling or args.read_ceiling_sweep:
        # attended rows of the tiered 8K chain right after a reassignment (T0 + T1 of 8 256)
        n_att = sum(budget_counts(base, base.ctx[0] + delta)[:2]) + 1
        print(json.dumps(read_ceiling(base, n_att)), flush=True)
        if args.read_ceiling_sweep:
            print(json.dumps(read_ceiling_sweep(base, n_att)), flush=True)
        return
    print(f"[bench] {wl.name}: generating inputs", file=sys.stderr, flush=True)
    dw = DeviceWorkload(wl)
    contexts = [st.context() for st in dw.streams]
    inputs = dw.preload(1, W + K + extra)

    flush_buf = None
    re_kernels = "assign_tiers,reloc_scan,quantize_t2,reloc_stage,reloc_to_t1,reloc_to_t0,t2_scan,t2_move"

    def release():
        """Hand what the last run left (its cache, which may sit in reference cycles) back
        to torch's caching allocator, so that the next run's cache takes the same blocks.
        Memory returned to the driver (torch.cuda.empty_cache) is cleared by it in the
        background, and that clearing took HBM bandwidth from the next run's timed steps
        (3-4% fewer steps/s)."""
        gc.collect()

    def run(timed_kernels, every=1, flush=False, attend_t2=False, alpha_scratch=False):
        """Fresh cache, W warm-up steps (at least Delta: the first reassignment is behind
        them), then exactly K steps between two syncs with the kernel timers on for
        `timed_kernels` (None = all) on every `every`-th step (each pair of events adds a
        few microseconds around the launch it brackets).  With `flush`, a 512 MB buffer is
        read before every step (outside the kernel timers).  With `attend_t2`, the 8-bit
        T2 rows are attended too; the attended counts are then (full-precision rows, T2
        rows) pairs.  With `alpha_scratch`, the decode calls store no normalised weights
        (they still enter the scores).  When the K steps hold no reassignment, the steps
        continue untimed to the next multiple of Delta and that reassignment alone is timed
        (wall clock between two syncs, its kernels under the timers when `timed_kernels`
        is None)."""
        cache = dw.make_cache(contexts=contexts, attend_t2=attend_t2, t0_budget=True,
                              alpha_scratch=alpha_scratch, per_sequence=True)
        torch.cuda.synchronize()
        for k in range(1, W + 1):
            cache.step(*inputs[k - 1])
        torch.cuda.synchronize()
        state = {"n": [int(x) for x in cache.n],
                 "counts": cache.counts.cpu().numpy().astype(int).tolist(),
                 "n_at_reassignment": [int(x) - (W % delta) for x in cache.n],
                 "resident_kv_bytes": cache.resident_kv_bytes(),
                 "full_cache_kv_bytes": cache.full_cache_bytes(), "cap0": cache.cap0,
                 "caps0": list(cache.caps0), "caps1": list(cache.caps1),
                 "alpha_bytes": cache.alpha.numel() * cache.alpha.element_size(),
                 "cap1": cache.cap1}
        n_att, n_all, re, sampled = [], [], [], []
        timed = timed_kernels is None or len(timed_kernels) > 0
        tkv.tkv_timing_select(timed_kernels)
        tkv.tkv_timing_reset()
        tkv.tkv_timing_enable(timed)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(W + 1, W + K + 1):
            full_rows = sum(cache.t0_len) + sum(cache.t1_len) + wl.batch
            n_att.append((full_rows, sum(cache.t2_len)) if attend_t2 else full_rows)
            n_all.append(sum(cache.n) + wl.batch)
            if flush:
                flush_buf.sum()
            if timed and every > 1:
                on = (k - W - 1) % every == 0
                tkv.tkv_timing_enable(on)
                if on:
                    sampled.append(n_att[-1])
            if cache.step(*inputs[k - 1]):
                re.append((sum(cache.n), sum(cache.t0_len), sum(cache.t1_len), sum(cache.t2_new),
                           sum(cache.moved)))
        issued = time.perf_counter() - t0  # host time to queue the K steps
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        tkv.tkv_timing_enable(False)
        re_alone = None
        if not re:
            for k in range(W + K + 1, W + K + extra + 1):
                cache.step(*inputs[k - 1], reassign=False)
            assert cache.steps % delta == 0
            tkv.tkv_timing_enable(timed_kernels is None)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            cache.reassign()
            torch.cuda.synchronize()
            re_alone = time.perf_counter() - t1
            tkv.tkv_timing_enable(False)
            re_alone_info = (sum(cache.n), sum(cache.t0_len), sum(cache.t1_len),
                             sum(cache.t2_new), sum(cache.moved))
        else:
            re_alone_info = None
        kernels = {}
        for name in ("append", "attn_partial", "attn_merge", "alpha_score", "score_update",
                     "assign_tiers", "reloc_scan", "quantize_t2", "reloc_stage", "reloc_to_t1",
                     "reloc_to_t0", "t2_scan", "t2_move"):
            ms, cnt = tkv.tkv_timing_read(name)
            if cnt:
                kernels[name] = {"launches": cnt, "avg_us": ms * 1e3 / cnt, "total_ms": ms}
        tkv.tkv_timing_select(None)
        return {"cache": cache, "elapsed": elapsed, "issued": issued, "n_att": n_att,
                "n_all": n_all, "re": re,
                "kernels": kernels, "sampled": sampled or n_att, "re_alone": re_alone,
                "re_alone_info": re_alone_info, "state": state}

    def amortised_elapsed(r):
        """Timed interval plus K / Delta of a reassignment timed on its own, when the K
        timed steps held none."""
        return r["elapsed"] + (K / delta * r["re_alone"] if r["re_alone"] is not None else 0.0)

    def check_split(r):
        """The tier counts left by the last reassignment before the timed steps must be
        those of the stated split at that length (refuse to report a mislabelled state)."""
        st = r["state"]
        for b in range(wl.batch):
            want = budget_counts(wl, st["n_at_reassignment"][b])
            if st["counts"][b] != want:
                print(f"[bench] sequence {b}: tier counts {st['counts'][b]} at n = "
                      f"{st['n_at_reassignment'][b]} differ from the split {want}; no line "
                      "printed", file=sys.stderr, flush=True)
                sys.exit(3)

    # the measured runs carry no kernel timer at all (value); the roofline runs time the
    # attention kernel on every timed step with events the kernel records itself
    print(f"[bench] warm-up {W} steps, {K} timed steps", file=sys.stderr, flush=True)
    # repeated: the reported figures are the medians over the repetitions
    reps = []
    for _ in range(max(1, args.repeats)):
        r = run([])
        check_split(r)
        reps.append((amortised_elapsed(r), r["elapsed"], r["re_alone"], r["issued"]))
        last = r
        del r["cache"]
        release()
    att_reps = []
    for _ in range(max(1, (args.repeats + 1) // 2)):
        r = run(["attn_partial"])
        att_reps.append(r["kernels"].get("attn_partial", {}).get("avg_us", float("nan")))
        last_att = r
        del r["cache"]
        release()
    elapsed = float(np.median([x[0] for x in reps]))
    attn_med = float(np.median(att_reps))
    n_att_steps, n_steps, re_info = last["n_att"], last["n_all"], last["re"]
    n_att_timed = last_att["sampled"]
    # a second, identical run with every kernel timed (the per-kernel breakdown only)
    print("[bench] breakdown run", file=sys.stderr, flush=True)
    bd = run(None)
    cache = bd["cache"]
    kernels = bd["kernels"]

    steps_per_s = K / elapsed
    step_b = [step_bytes(wl, n_att, n) for n_att, n in zip(n_att_steps, n_steps)]
    if re_info:
        re_b = sum(reassign_bytes(wl, *x) for x in re_info)
    else:
        re_b = K / delta * reassign_bytes(wl, *last["re_alone_info"])
    alg_bytes = (sum(x["total"] for x in step_b) + re_b) / K
    min_bytes = (sum(x["minimal"] for x in step_b) + re_b) / K
    attn = {"avg_us": attn_med}
    attn_bytes = float(np.mean([attn_partial_bytes(wl, n) for n in n_att_timed]))
    attn_rows = float(np.mean(n_att_timed))
    achieved = attn_bytes / (attn["avg_us"] * 1e-6) / 1e9
    st = last["state"]
    counts = np.array(st["counts"]).sum(axis=0).tolist()
    traffic = counter_traffic(args.workload, attn_rows)

    out = {
        "metric": "decode steps/sec (attn+score+tier) at 8K ctx; achieved HBM GB/s vs peak",
        "value": steps_per_s,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": elapsed / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded generator: sinks, planted resurfacing keys, N(0,1) K/V)",
        "config": {"workload": f"{base.name}: {base.description}", "batch": wl.batch,
                   "context": list(wl.ctx) if wl.batch > 1 else wl.ctx[0],
                   "layers": wl.layers, "q_heads": wl.q_heads, "kv_heads": wl.kv_heads,
                   "head_dim": wl.head_dim,
                   "tiers_t0_t1_t2_t3": [round(1 - wl.frac_t1 - wl.frac_t2 - wl.frac_t3, 4),
                                         wl.frac_t1, wl.frac_t2, wl.frac_t3],
                   "delta": delta, "warmup_steps_run": W,
                   "tier_counts_before_timed_steps": counts,
                   "context_at_that_reassignment": int(sum(st["n_at_reassignment"])),
                   "mean_attended_rows": float(np.mean(n_att_steps)),
                   "reassignments_timed": len(re_info),
                   "reassignment_timed_alone_ms": (float(np.median([x[2] for x in reps])) * 1e3
                                                   if not re_info else None),
                   "rows_copied_per_reassignment": ([x[4] for x in re_info] if re_info
                                                    else [last["re_alone_info"][4]]),
                   "value_basis": ("timed steps as measured (they hold the reassignments)"
                                   if re_info else
                                   f"timed steps plus {K}/{delta} of one reassignment timed "
                                   "alone at the next multiple of delta")},
        "repetitions": {"count": len(reps),
                        "steps_per_s": [K / x[0] for x in reps],
                        "timed_interval_steps_per_s": [K / x[1] for x in reps],
                        "host_issue_us_per_step": [x[3] / K * 1e6 for x in reps],
                        "attn_partial_avg_us": att_reps,
                        "note": "steps_per_s: runs without kernel timers; attn_partial_avg_us: "
                                "separate runs timing that kernel on every timed step; "
                                "host_issue_us_per_step: host time to queue a timed step (the "
                                "GPU is the bound while it stays below the step time)"},
        "roofline": {"bound": "hbm", "kernel": "attn_partial", "achieved": achieved,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic, "bytes_per_launch": attn_bytes,
                     "attended_rows_per_launch": attn_rows,
                     "avg_launch_us": attn["avg_us"]},
        "step_hbm": {"algorithmic_bytes_per_step": alg_bytes,
                     "achieved_gbps": alg_bytes * steps_per_s / 1e9,
                     "frac": alg_bytes * steps_per_s / 1e9 / PEAK_HBM_GBS,
                     "minimal_bytes_per_step": min_bytes,
                     "frac_minimal": min_bytes * steps_per_s / 1e9 / PEAK_HBM_GBS,
                     "note": "bytes with the alpha round trip (written, read by the score "
                             "update) and minimal bytes (K/V, q, O, score RMW, append), "
                             "plus the per-Delta terms amortised",
                     "mean_attended_tokens": float(np.mean(n_att_steps))},
        "hbm_resident": {"kv_bytes": st["resident_kv_bytes"],
                         "full_cache_kv_bytes": st["full_cache_kv_bytes"],
                         "ratio": st["resident_kv_bytes"] / st["full_cache_kv_bytes"],
                         "t0_capacity": st["cap0"], "t1_window_capacity": st["cap1"],
                         "t0_capacity_sum": sum(st["caps0"]),
                         "t1_window_capacity_sum": sum(st["caps1"]),
                         "alpha_scratch_bytes": st["alpha_bytes"],
                         "note": "device bytes holding K/V rows after the first "
                                 "reassignment (each sequence's T0 pool at its budget, its T1 "
                                 "window) against every row of the context at full precision; "
                                 "capacities: the largest, and the sum over the sequences"},
        "kernels": kernels,
        "kernels_sum_us_per_step": (kernel_sum(kernels, K) if bd["re"] else
                                    kernel_sum(kernels, K, 1, delta)),
        "kernels_note": ("per-kernel averages from another identical run with every kernel "
                         "timed (events between launches slow that run to "
                         f"{K / amortised_elapsed(bd):.0f} steps/s); value comes from runs with "
                         "no timers, the roofline from runs timing attn_partial alone"),
    }
    if not args.no_flush_run:
        # a real decode streams the model weights between two visits of a layer, which
        # evicts the memory-side cache: the same steps with 512 MB read before each one
        del cache, bd
        release()
        print("[bench] cache-flushed run", file=sys.stderr, flush=True)
        flush_buf = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
        fr = run(["attn_partial"], flush=True)
        cache = fr["cache"]
        fa = fr["kernels"].get("attn_partial")
        if fa:
            fb = float(np.mean([attn_partial_bytes(wl, n) for n in fr["sampled"]]))
            out["flushed"] = {"attn_partial_avg_us": fa["avg_us"],
                              "achieved_gbps": fb / (fa["avg_us"] * 1e-6) / 1e9,
                              "frac": fb / (fa["avg_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS,
                              "note": "512 MB read before every step (memory-side cache "
                                      "cold, as after a model's weight stream)"}
        del flush_buf, fr
    # the same steps with the weights kept only for the score update (tkv_model.alpha_scratch):
    # what a caller that never reads alpha saves; not the headline, which stores alpha
    print("[bench] weights-as-scratch run", file=sys.stderr, flush=True)
    sr = [run([], alpha_scratch=True) for _ in range(max(1, (args.repeats + 1) // 2))]
    out["alpha_scratch"] = {
        "steps_per_s": float(np.median([K / amortised_elapsed(r) for r in sr])),
        "note": "normalised weights not stored (tkv_model.alpha_scratch = 1); the scores, "
                "outputs and tiers are the same; not part of value"}
    for r in sr:
        del r["cache"]
    del sr
    release()
    if not args.no_t2_leg:
        # the variant that attends the 8-bit T2 rows after T1: same inputs and policy
        del cache
        release()
        print("[bench] attended-T2 run", file=sys.stderr, flush=True)
        tr = run(["attn_partial"], attend_t2=True)
        cache = tr["cache"]
        a2 = tr["kernels"].get("attn_partial")
        if a2:
            b2 = float(np.mean([attn_partial_bytes(wl, f, t) for f, t in tr["sampled"]]))
            out["attend_t2"] = {
                "steps_per_s": K / amortised_elapsed(tr), "attn_partial_avg_us": a2["avg_us"],
                "bytes_per_launch": b2, "achieved_gbps": b2 / (a2["avg_us"] * 1e-6) / 1e9,
                "frac": b2 / (a2["avg_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS,
                "mean_t2_rows": float(np.mean([t for _, t in tr["n_att"]])),
                "note": "T0 u T1 u T2 attended, T2 as int8 code x float32 scale per row "
                        "(one run, attn_partial timed on every timed step); not part of value"}
        del tr
    if not args.no_stream_leg:
        # T1 streamed from pinned host memory every step, layer by layer through a
        # two-buffer device window (the copy of layer l + 2 overlaps the attention of
        # layer l + 1): the whole step as the pages describe it, host-link bound
        from tiered_kv_cache_amd.driver import T1Stream
        del cache
        release()
        print("[bench] streamed-T1 run", file=sys.stderr, flush=True)
        cache = dw.make_cache(contexts=contexts, t0_budget=True, per_sequence=True)
        stream = T1Stream(cache, chunk_layers=args.stream_chunk)
        for k in range(1, W + 1):
            stream.step(*inputs[k - 1])
        torch.cuda.synchronize()
        first_re = list(stream.link_reassign)
        t0 = time.perf_counter()
        link = 0
        t1_rows = []
        for k in range(W + 1, W + K + 1):
            t1_rows.append(sum(cache.t1_len))
            stream.step(*inputs[k - 1])
            link += stream.link_bytes_per_step()
        torch.cuda.synchronize()
        el_s = time.perf_counter() - t0
        re_s = None
        if len(stream.link_reassign) == len(first_re):      # none in the timed steps
            for k in range(W + K + 1, W + K + extra + 1):
                stream.step(*inputs[k - 1], reassign=False)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            stream.reassign()
            re_s = time.perf_counter() - t1
        el_amort = el_s + (K / delta * re_s if re_s is not None else 0.0)
        sh = cache.shape
        row = sh.layers * sh.kv_heads * 2 * sh.head_dim * (2 if sh.dtype == "bf16" else 4)
        out["t1_streamed"] = {
            "steps_per_s": K / el_amort, "ms_per_step": el_amort / K * 1e3,
            "link_bytes_per_step": link / K,
            "link_gbps": link / el_s / 1e9,
            "mean_t1_rows": float(np.mean(t1_rows)),
            "t1_row_bytes_per_step": float(np.mean(t1_rows)) * row,
            "link_bytes_per_reassignment": {"first": first_re[0] if first_re else None,
                                            "later": stream.link_reassign[len(first_re):]},
            "resident_kv_bytes": stream.resident_kv_bytes(),
            "full_cache_kv_bytes": cache.full_cache_bytes(),
            "resident_over_full": stream.resident_kv_bytes() / cache.full_cache_bytes(),
            "device_window_bytes": stream.window_bytes(),
            "t0_capacity": cache.cap0,
            "chunk_layers": stream.chunk,
            "note": "T1 rows in host memory (pinned window, full-precision store by position); "
                    "every step: append, then per chunk of layers the live T1 blocks cross the "
                    "link while the previous chunk attends (tkv_decode_step_streamed); every "
                    "Delta steps only the rows that enter T1 from T0 go to the host and only the "
                    "rows that leave T1 come back (tkv_compact_host_t1); HBM holds the T0 pool "
                    "at its budget and a two-chunk window; not part of value"}
        del stream
    if not args.no_pcie:
        try:
            t1 = cache.t1_pos[0, :cache.t1_len[0]].cpu().numpy().tolist()   # window slot order
            out["pcie"] = pcie_leg(wl, cache, t1, 1.0 / steps_per_s)
            out["pcie"]["note"] = ("a whole T1 set through tkv_gather_t1 (host pack into pinned "
                                   "staging, one 2-D copy on a side stream); not part of value")
        except Exception as e:  # reported, never fatal for the device number
            out["pcie"] = {"error": repr(e)}
    if not args.no_cpu_baseline:
        print("[bench] oracle CPU baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(base.scaled(steps=K, warmup=W), args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
