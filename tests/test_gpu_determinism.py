"""Determinism: two runs of the device path on identical inputs give identical bits.

The attention splits its work by a fixed rule (worker count and unit ranges depend only
on the launch's sizes), the merge and the score update sum in a fixed order, and the
tier ranking breaks ties by position, so nothing may depend on timing.  Checked on the
device after every step (output, weights, scores) and after every reassignment (tier
maps, counts, pools, window, slot maps, int8 rows, the attended T2 pool)."""
import pytest
import torch

from tests.parity import say
from tiered_kv_cache_amd.synth import WORKLOADS
from tiered_kv_cache_amd.workload import DeviceWorkload

pytestmark = pytest.mark.gpu


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("name,attend_t2,warmup,steps", [("small", False, 64, 8),
                                                         ("small", True, 64, 8),
                                                         ("chain8k", False, 64, 4)],
                         ids=["small", "small_attend_t2", "chain8k"])
def test_two_runs_identical_bits(name, attend_t2, warmup, steps):
    wl = WORKLOADS[name].scaled(warmup=warmup, steps=steps)
    dw = DeviceWorkload(wl)
    contexts = [st.context() for st in dw.streams]
    inputs = dw.preload(1, wl.total_steps)
    runs = [dw.make_cache(contexts=contexts, attend_t2=attend_t2) for _ in range(2)]
    per_step = ("out", "alpha", "scores")
    per_reassign = ("tiers", "counts", "k_t0", "v_t0", "t0_pos", "k_t1", "v_t1", "t1_pos",
                    "t2_pos", "t2_codes", "t2_scales", "new_lens")
    if attend_t2:
        per_reassign += ("k_t2", "v_t2", "ks_t2", "vs_t2", "t2_slot_pos")
    checked = 0
    for k in range(1, wl.total_steps + 1):
        flags = [c.step(*inputs[k - 1]) for c in runs]
        torch.cuda.synchronize()
        a, b = runs
        for f in per_step:
            assert same_bits(getattr(a, f), getattr(b, f)), f"{f} differs at step {k}"
        if flags[0]:
            assert a.t0_len == b.t0_len and a.t1_len == b.t1_len and a.t2_len == b.t2_len
            for f in per_reassign:
                assert same_bits(getattr(a, f), getattr(b, f)), f"{f} differs at step {k}"
            checked += 1
    assert checked >= 1
    say(f"[determinism {name}{' attend_t2' if attend_t2 else ''}] {wl.total_steps} steps, "
        f"{checked} reassignments: identical bits")
