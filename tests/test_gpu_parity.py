"""GPU parity of the whole decode path against the CPU oracle, through the C ABI.

Small workloads are compared at every step; full-size workloads on sampled outputs
the oracle computes one at a time and on size-independent properties.  Tolerances are
in tests/parity.py.
"""
import numpy as np
import pytest
import torch

from oracle import attention
from tests.parity import check_alpha, check_output, check_scores, run_lockstep, run_sampled, say
from tiered_kv_cache_amd.driver import to_device
from tiered_kv_cache_amd.synth import WORKLOADS
from tiered_kv_cache_amd.workload import DeviceWorkload

pytestmark = pytest.mark.gpu


def test_tiny_fp32_lockstep():
    wl = WORKLOADS["tiny"]
    st = run_lockstep(wl)
    assert st["reassignments"] == 4 and st["t2_rows"] > 0


def test_tiny_prop1_no_eviction_equals_full_attention():
    # T2 = T3 = 0 (40/60/0/0): the tiered output equals full attention at every step
    wl = WORKLOADS["tiny"].with_fractions(0.6, 0.0, 0.0, "_40-60-0-0")
    st = run_lockstep(wl)
    assert st["reassignments"] == 4 and st["t2_rows"] == 0


def test_small_eviction_only_lockstep():
    # the eviction-only baseline mode (T1 = T2 = 0, 30% evicted): the same path with
    # only T0 and T3, checked step by step like the tiered policy
    wl = WORKLOADS["small"].with_fractions(0.0, 0.0, 0.3, "_evict30").scaled(warmup=8, steps=72)
    st = run_lockstep(wl, label="small_eviction_only")
    assert st["reassignments"] == 1 and st["t2_rows"] == 0


def test_small_gqa4_lockstep():
    wl = WORKLOADS["small"]
    st = run_lockstep(wl)
    assert st["reassignments"] == 3


def test_small_separate_append_call():
    # tkv_append then tkv_decode_step (the other tests use tkv_append_decode_step)
    wl = WORKLOADS["small"].scaled(warmup=8, steps=72)
    st = run_lockstep(wl, fused_append=False, label="small_separate_append")
    assert st["reassignments"] == 1


def test_small_standalone_score_update():
    # the score update as its own call (tkv_update_scores on the normalised alpha)
    wl = WORKLOADS["small"].scaled(warmup=8, steps=72)
    st = run_lockstep(wl, fused_scores=False, label="small_standalone_scores")
    assert st["reassignments"] == 1


@pytest.mark.parametrize("hq,hkv,d", [(16, 1, 128), (4, 4, 64), (6, 2, 128), (8, 1, 64)],
                         ids=["group16_d128", "mha_d64", "group3_d128", "group8_d64"])
def test_head_groupings_lockstep(hq, hkv, d):
    # every query-head grouping the matrix-core kernel supports shape-wise: 1, 3, 8, 16
    # query heads per KV head, both head sizes, a ragged pair of sequences
    base = WORKLOADS["small"]
    wl = base.scaled(name=f"groups_h{hq}kv{hkv}_d{d}", layers=2, q_heads=hq, kv_heads=hkv,
                     head_dim=d, batch=2, ctx=(190, 333), warmup=4, steps=8, delta=4, prompt=8,
                     recent=8, sinks=2, planted=(3, 5), frac_t1=0.3, frac_t2=0.15,
                     frac_t3=0.05)
    st = run_lockstep(wl)
    assert st["reassignments"] == 3 * 2


def test_ragged_batch_d64_lockstep():
    base = WORKLOADS["small"]
    wl = base.scaled(name="ragged5_L2_h8kv2_d64", layers=2, head_dim=64, batch=5,
                     ctx=(130, 700, 257, 1100, 64), warmup=8, steps=16, delta=8, prompt=16,
                     recent=16, sinks=4, planted=(2, 8, 4, 10, 0), frac_t1=0.4, frac_t2=0.15,
                     frac_t3=0.05)
    st = run_lockstep(wl)
    assert st["reassignments"] == 3 * 5          # counted per sequence


def test_batch70_crosses_the_per_launch_sequence_limit():
    # 70 ragged sequences: the library splits them over two launches of <= 64
    base = WORKLOADS["small"]
    ctx = tuple(int(c) for c in np.random.default_rng(7).integers(33, 400, size=70))
    wl = base.scaled(name="batch70_L1_h4kv2_d64", layers=1, q_heads=4, kv_heads=2, head_dim=64,
                     batch=70, ctx=ctx, warmup=4, steps=8, delta=4, prompt=8, recent=8, sinks=2,
                     planted=(0,) * 70, frac_t1=0.3, frac_t2=0.1, frac_t3=0.1)
    st = run_lockstep(wl)
    assert st["reassignments"] == 3 * 70


@pytest.mark.parametrize("batch", [5, 70], ids=["ragged5", "batch70_two_launches"])
def test_per_sequence_pools_lockstep(batch):
    # every sequence's T0 pool and T1 window sized for its own length (tkv_model.t0_caps /
    # t1_caps, blocks packed sequence after sequence), the T0 pools shrunk to each
    # sequence's budget after the first reassignment; with 70 sequences the second
    # launch's sequences start after the first launch's blocks
    base = WORKLOADS["small"]
    if batch == 5:
        wl = base.scaled(name="percap_ragged5_L2_h8kv2_d64", layers=2, head_dim=64, batch=5,
                         ctx=(130, 700, 257, 1100, 64), warmup=8, steps=16, delta=8, prompt=16,
                         recent=16, sinks=4, planted=(2, 8, 4, 10, 0), frac_t1=0.4,
                         frac_t2=0.15, frac_t3=0.05)
    else:
        ctx = tuple(int(c) for c in np.random.default_rng(11).integers(33, 400, size=70))
        wl = base.scaled(name="percap_batch70_L1_h4kv2_d64", layers=1, q_heads=4, kv_heads=2,
                         head_dim=64, batch=70, ctx=ctx, warmup=4, steps=8, delta=4, prompt=8,
                         recent=8, sinks=2, planted=(0,) * 70, frac_t1=0.3, frac_t2=0.1,
                         frac_t3=0.1)
    st = run_lockstep(wl, per_sequence=True, t0_budget=True, alpha_scratch=batch == 70,
                      label=wl.name)
    assert st["reassignments"] == (3 if batch == 5 else 3) * batch


def test_per_sequence_pools_fp32():
    # the float32 path (vector-ALU attention, separate append) with per-sequence pools
    wl = WORKLOADS["tiny"].scaled(name="percap_tiny3_fp32", batch=3, ctx=(256, 100, 33),
                                  planted=(0, 0, 0))
    st = run_lockstep(wl, per_sequence=True, t0_budget=True, label=wl.name)
    assert st["reassignments"] == 4 * 3


def test_empty_sequence_in_batch():
    # one sequence of the batch has no attended token: its output rows are zero and the
    # other sequences are unaffected (one attention call, no append)
    from collections import defaultdict
    wl = WORKLOADS["small"].scaled(name="empty_mix_L2_h8kv2_d128", layers=2, batch=3,
                                   ctx=(300, 0, 77), planted=(0, 0, 0), warmup=0, steps=1,
                                   prompt=8, recent=8, sinks=2)
    dw = DeviceWorkload(wl)
    cache = dw.make_cache()
    q, _, _ = dw.host_step(1)
    cache.out.fill_(float("nan"))
    cache.attend(to_device(q, dw.dtype, dw.device))
    torch.cuda.synchronize()
    out = cache.out.cpu().numpy()
    stats = defaultdict(float)
    scale = 1.0 / np.sqrt(wl.head_dim)
    for b, n in enumerate(wl.ctx):
        if n == 0:
            assert np.all(out[b] == 0.0), "rows of the empty sequence must be zero"
            continue
        K, V = dw.streams[b].context()
        alpha_gpu = cache.alpha_of(b)
        inc = np.zeros(n)
        for l in range(wl.layers):
            for h in range(wl.q_heads):
                g = h // wl.group
                O, a = attention(q[b][l][h:h + 1], K[l][g:g + 1], V[l][g:g + 1], scale)
                check_output(out[b, l, h][None], O, stats)
                check_alpha(alpha_gpu[l, h][None], a, stats)
                inc += a[0]
        check_scores(cache.scores[b, :n].cpu().numpy(), inc / (wl.layers * wl.q_heads), stats)
    say(f"[empty sequence] ok: " + ", ".join(f"{k}={v:.3g}" for k, v in sorted(stats.items())))


def test_small_t0_budget_lockstep():
    # the T0 pool moved into one sized by the tier budget after the first reassignment:
    # the same results, step by step
    wl = WORKLOADS["small"]
    st = run_lockstep(wl, t0_budget=True, label="small_t0_budget")
    assert st["reassignments"] == 3 and st["cap0"] < 2048


def test_small_alpha_scratch_lockstep():
    # the calls that keep the weights only for the score update (the alpha buffer is
    # scratch): output and scores every step, tiers and rows at every reassignment
    wl = WORKLOADS["small"]
    st = run_lockstep(wl, t0_budget=True, alpha_scratch=True, label="small_alpha_scratch")
    assert st["reassignments"] == 3


def test_chain8k_full_size_sampled():
    # the bench's configuration: per-sequence pools, the T0 pool at its budget after the
    # first reassignment, the normalised weights stored
    wl = WORKLOADS["chain8k"]
    heads = [(0, 0), (0, 6), (13, 20), (27, 27)]
    st = run_sampled(wl, n_steps=130, sample_steps={1, 63, 64, 65, 100, 128, 129},
                     heads=heads, full_inc_steps={2, 66, 100, 129}, t0_budget=True,
                     per_sequence=True)
    assert st["reassignments"] == 2 and st["inc_checked"] == 4


def test_chain8k_alpha_scratch_full_size_sampled():
    # the same with the weights kept only for the score update (the bench's
    # alpha_scratch leg): outputs and the whole score increment at full size
    wl = WORKLOADS["chain8k"]
    st = run_sampled(wl, n_steps=70, sample_steps={1, 65, 70}, heads=[(0, 0), (27, 27)],
                     full_inc_steps={66, 70}, t0_budget=True, per_sequence=True,
                     alpha_scratch=True)
    assert st["reassignments"] == 1 and st["inc_checked"] == 2


def test_batch16_ragged_full_size_sampled():
    # 16 sequences with contexts from 1024 to 8192 tokens, the 7B-class shape
    wl = WORKLOADS["batch16"]
    heads = [(0, 0), (11, 13), (27, 27)]
    st = run_sampled(wl, n_steps=wl.total_steps, sample_steps={1, 64, 65, 97, 128},
                     heads=heads, full_inc_steps={2, 70}, byte_seqs={0, 7, 15})
    assert st["reassignments"] == 2 * 16


def test_batch16_per_sequence_pools_full_size_sampled():
    # the bench's batch configuration: per-sequence pools, T0 at each sequence's budget
    wl = WORKLOADS["batch16"]
    heads = [(0, 0), (11, 13), (27, 27)]
    st = run_sampled(wl, n_steps=wl.total_steps, sample_steps={1, 64, 65, 97, 128},
                     heads=heads, full_inc_steps={2, 70, 128}, byte_seqs={0, 7, 15},
                     per_sequence=True, t0_budget=True)
    assert st["reassignments"] == 2 * 16


def test_chain32k_full_size_sampled():
    # 4 sequences of 32768 tokens, 32 layers, 32 query / 8 KV heads
    wl = WORKLOADS["chain32k"]
    heads = [(0, 3), (17, 20), (31, 31)]
    st = run_sampled(wl, n_steps=wl.total_steps, sample_steps={1, 64, 65, 128},
                     heads=heads, full_inc_steps={66}, byte_seqs={1})
    assert st["reassignments"] == 2 * 4


def test_chain32k_per_sequence_pools_full_size_sampled():
    # the bench's long-chain configuration: per-sequence pools, T0 at each sequence's
    # budget; its 430 MB of logits per launch take the non-temporal stage flushes
    wl = WORKLOADS["chain32k"]
    heads = [(0, 0), (9, 12), (31, 31)]
    st = run_sampled(wl, n_steps=wl.total_steps, sample_steps={65, 128},
                     heads=heads, full_inc_steps={70}, byte_seqs={3},
                     per_sequence=True, t0_budget=True)
    assert st["reassignments"] == 2 * 4
