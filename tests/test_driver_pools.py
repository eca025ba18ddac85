"""Host-side layout of the driver's pools (no GPU: the tensors live in host memory and
no kernel runs).  Per-sequence capacities (tkv_model.t0_caps / t1_caps) pack each
sequence's [L][Hkv][cap_b][D] block after the previous one; each sequence's block must
hold exactly its own rows, and the pools must be smaller than the uniform layout, which
gives every sequence the longest one's capacity."""
import numpy as np

from tiered_kv_cache_amd.synth import WORKLOADS
from tiered_kv_cache_amd.workload import DeviceWorkload


def ragged_workload():
    return WORKLOADS["small"].scaled(name="pools_ragged4_L2_h8kv2_d64", layers=2, head_dim=64,
                                     batch=4, ctx=(130, 700, 33, 1100), warmup=8, steps=16,
                                     delta=8, prompt=16, recent=16, sinks=4, planted=(2, 8, 0, 10),
                                     frac_t1=0.4, frac_t2=0.15, frac_t3=0.05)


def test_per_sequence_capacities_and_blocks():
    wl = ragged_workload()
    dw = DeviceWorkload(wl, device="cpu")
    per = dw.make_cache(per_sequence=True)
    uni = dw.make_cache()
    f1 = float(np.float32(wl.frac_t1))
    for b, st in enumerate(dw.streams):
        bound = st.n0 + wl.total_steps + 1                 # the sequence's longest length
        assert per.caps0[b] == (bound + 63) // 64 * 64
        assert per.caps1[b] == (int(np.floor(f1 * per.caps0[b])) + 64 + 63) // 64 * 64
        K, V = st.context()
        k, v = per.t0_rows(b)                              # read back from its own block
        assert np.array_equal(k, K) and np.array_equal(v, V)
        blk = per.block(per.k_t0, per.caps0, b)
        assert blk.shape == (wl.layers, wl.kv_heads, per.caps0[b], wl.head_dim)
    # the blocks tile the flat pool exactly, in sequence order
    starts = [per.block(per.k_t0, per.caps0, b).data_ptr() for b in range(wl.batch)]
    elem = per.k_t0.element_size()
    sizes = [c * wl.layers * wl.kv_heads * wl.head_dim * elem for c in per.caps0]
    assert starts[0] == per.k_t0.data_ptr()
    assert all(starts[b + 1] - starts[b] == sizes[b] for b in range(wl.batch - 1))
    assert sum(sizes) == per.k_t0.numel() * elem
    assert per.cap0 == max(per.caps0) == uni.cap0
    assert per.resident_kv_bytes() < 0.6 * uni.resident_kv_bytes()
    # the model carries the capacities to the library
    assert per.model.t0_caps is not None and per.model.t1_caps is not None
    assert uni.model.t0_caps is None and uni.model.t1_caps is None
