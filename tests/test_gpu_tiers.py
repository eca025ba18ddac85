"""GPU tier classifier (tkv_assign_tiers) against the oracle's ranking on score arrays built
to stress it: continuous scores, few distinct values (long runs of ties), all-equal scores,
signed zeros and subnormals, earlier tier maps with T2/T3 history, ragged batches with lengths
from 0 to 70000.  The kernel keeps a sequence's keys in registers when the launch's longest
sequence has at most 1024 * {8, 16, 32, 48} positions and streams them from memory above that,
so each batch below tops out in another of those ranges (at its edge).  The tier maps and counts
must be bit-identical."""
import numpy as np
import pytest
import torch

from oracle import Policy, assign_tiers
from tests.parity import say
from tiered_kv_cache_amd import tkv

pytestmark = pytest.mark.gpu

BATCHES = {
    "le8k": [0, 1, 5, 37, 1000, 4097, 8192],
    "le16k": [8193, 37, 16384],
    "le32k": [16385, 1000, 32768],
    "le48k": [32769, 5, 49152],
    "streamed": [49153, 0, 70000],
}


def make_scores(rng, n, kind):
    if kind == 0:                                   # continuous, distinct
        return rng.random(n, dtype=np.float32) * np.float32(3.0)
    if kind == 1:                                   # few distinct values: long tie runs
        return (rng.integers(0, 5, n) / np.float32(4.0)).astype(np.float32)
    if kind == 2:                                   # all equal
        return np.full(n, np.float32(0.125), np.float32)
    # signed zeros, subnormals and a few normal values
    vals = np.array([0.0, -0.0, 1e-45, 3e-44, 1e-40, 2.5e-38, 1e-3, 0.5], np.float32)
    return vals[rng.integers(0, len(vals), n)]


def history(rng, n, pol):
    """A reachable earlier tier map: an assignment at an earlier length."""
    prev = np.zeros(n, np.uint8)
    if n:
        n_old = int(rng.integers(0, n + 1))
        s_old = rng.random(n_old)
        prev[:n_old], _ = assign_tiers(s_old, np.zeros(n_old, np.uint8), n_old, pol)
    return prev


@pytest.mark.parametrize("pol", [
    Policy(256, 4, 128, 0.30, 0.15, 0.05, 64),
    Policy(0, 0, 0, 0.40, 0.40, 0.15, 64),
    Policy(32, 64, 16, 0.00, 0.60, 0.30, 8),
    Policy(8, 2, 4000, 0.25, 0.25, 0.25, 8),
], ids=["chain", "unprotected", "sinks_gt_prompt", "recent_dominates"])
@pytest.mark.parametrize("batch", list(BATCHES))
def test_assign_tiers_bit_exact(pol, batch):
    rng = np.random.default_rng(20261298)
    lengths = [n for n in BATCHES[batch] for _ in range(4)]   # every length with every kind
    B = len(lengths)
    max_ctx = (max(lengths) + 63) // 64 * 64
    scores = np.zeros((B, max_ctx), np.float32)
    prev = np.zeros((B, max_ctx), np.uint8)
    for b, n in enumerate(lengths):
        scores[b, :n] = make_scores(rng, n, b % 4)
        if (b // 4) % 2 == 0 or b % 4 == 1:
            prev[b, :n] = history(rng, n, pol)
    dev = torch.device("cuda")
    s_d = torch.from_numpy(scores).to(dev)
    p_d = torch.from_numpy(prev).to(dev)
    n_d = torch.full((B, max_ctx), 9, dtype=torch.uint8, device=dev)
    c_d = torch.zeros((B, 4), dtype=torch.int32, device=dev)
    policy = tkv.make_policy(pol.prompt, pol.sinks, pol.recent, pol.frac_t1, pol.frac_t2,
                             pol.frac_t3, pol.delta)
    tkv.tkv_assign_tiers(B, lengths, max_ctx, s_d, policy, p_d, n_d, c_d)
    torch.cuda.synchronize()
    got = n_d.cpu().numpy()
    counts = c_d.cpu().numpy()
    for b, n in enumerate(lengths):
        ref, ref_counts = assign_tiers(scores[b].astype(np.float64), prev[b], n, pol)
        bad = np.nonzero(got[b, :n] != ref[:n])[0]
        assert bad.size == 0, f"n={n} kind={b % 4}: tiers differ at {bad[:8]}"
        assert counts[b].tolist() == list(ref_counts), f"n={n}: counts"
    say(f"[assign_tiers {batch}] {B} sequences bit-exact")
