"""The benchmark's byte accounting (the numerator of every roofline figure), checked on the
CPU against the arithmetic of the 7B-class 8K chain written out by hand: 28 layers, 28 query
and 4 KV heads, head_dim 128, bf16, 6 555 attended tokens (tiers 50/30/15/5 of 8 192)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from tiered_kv_cache_amd.synth import WORKLOADS  # noqa: E402


def test_step_bytes_of_the_8k_chain():
    wl = WORKLOADS["chain8k"]
    n_att, n = 6555, 8192
    b = bench.step_bytes(wl, n_att, n)
    assert b["kv"] == 28 * 4 * 6555 * 128 * 2 * 2 == 375_889_920      # K and V, bf16
    assert b["q"] == 28 * 28 * 128 * 2 and b["o"] == 28 * 28 * 128 * 4
    assert b["alpha"] == 2 * 28 * 28 * 6555 * 4                        # written, read back
    assert b["scores"] == 8 * 6555                                     # read-modify-write
    assert abs((b["total"] - b["append"]) / 1e6 - 417.65) < 0.01
    assert b["total"] - b["minimal"] == b["alpha"]


def test_attention_launch_bytes():
    wl = WORKLOADS["chain8k"]
    # K/V of the attended rows + queries + the raw logits written once
    assert bench.attn_partial_bytes(wl, 6715) == (2 * 28 * 4 * 6715 * 128 * 2 + 28 * 28 * 128 * 2
                                                  + 28 * 28 * 6715 * 4)
    # attended 8-bit T2 rows: D one-byte codes and one float32 scale for K and for V
    full = bench.attn_partial_bytes(wl, 6715)
    assert bench.attn_partial_bytes(wl, 6715, 1252) - full == \
        2 * 28 * 4 * 1252 * (128 + 4) + 28 * 28 * 1252 * 4


def test_kernel_sum_amortises_reassignment_launches():
    k = {"attn_partial": {"total_ms": 2.56}, "attn_merge": {"total_ms": 0.256},
         "score_update": {"total_ms": 0.128}, "assign_tiers": {"total_ms": 0.064}}
    s = bench.kernel_sum(k, 256)
    assert s["every_step"] == pytest.approx(11.5) and s["reassignment_amortised"] == \
        pytest.approx(0.25) and s["total"] == pytest.approx(11.75)
